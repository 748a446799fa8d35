// Absorbed-MLA decode (placeholder until the kernels land).
#include "da_internal.h"

namespace da {
hipError_t launch_mla_decode(const MlaArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace da
