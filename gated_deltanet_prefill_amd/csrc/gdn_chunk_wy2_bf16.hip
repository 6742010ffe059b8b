// gdn_chunk_wy2_bf16.hip -- the pipelined chunk kernel's four-slice form for
// bf16 q/k/v/y, built with the instruction-level-parallelism scheduler (the
// build passes -mllvm -amdgpu-sched-strategy=max-ilp for this file only).
#include "gdn_chunk_dispatch.h"

namespace gdn {
hipError_t launch_wy2_bf16(const FwdArgs &a, hipStream_t st, unsigned nblocks, int xcd_group) {
    return launch_wy2_kernel<__bf16>(a, st, nblocks, xcd_group);
}
}  // namespace gdn
