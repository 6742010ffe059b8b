// gdn_chunk_f16.hip -- chunk kernel instantiations for f16 q/k/v/y.
#include "gdn_chunk_dispatch.h"

namespace gdn {
hipError_t launch_chunk_f16(const FwdArgs &a, hipStream_t s) { return launch_chunk_typed<_Float16>(a, s); }
}  // namespace gdn
