// gdn_chunk_vg_f32.hip -- per-key-dimension-gate chunk kernel instantiations for f32 q/k/v/y.
#include "gdn_chunk_vg.h"

namespace gdn {
hipError_t launch_chunk_vg_f32(const FwdArgs &a, hipStream_t s) { return launch_chunk_vg_typed<float>(a, s); }
}  // namespace gdn
