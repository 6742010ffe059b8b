// gdn_chunk_vg_bf16.hip -- per-key-dimension-gate chunk kernel instantiations for bf16 q/k/v/y.
#include "gdn_chunk_vgp.h"

namespace gdn {
hipError_t launch_chunk_vg_bf16(const FwdArgs &a, hipStream_t s) { return launch_chunk_vg_any<__bf16>(a, s); }
}  // namespace gdn
