// gdn_chunk_bf16.hip -- chunk kernel instantiations for bf16 q/k/v/y.
#include "gdn_chunk_dispatch.h"

namespace gdn {
hipError_t launch_chunk_bf16(const FwdArgs &a, hipStream_t s) { return launch_chunk_typed<__bf16>(a, s); }
}  // namespace gdn
