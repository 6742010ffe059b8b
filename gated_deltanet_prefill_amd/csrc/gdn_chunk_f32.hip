// gdn_chunk_f32.hip -- chunk kernel instantiations for f32 q/k/v/y.
#include "gdn_chunk_dispatch.h"

namespace gdn {
hipError_t launch_chunk_f32(const FwdArgs &a, hipStream_t s) { return launch_chunk_typed<float>(a, s); }
}  // namespace gdn
