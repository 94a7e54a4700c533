// gemm.hip -- matrix-core OWQ linear for larger M (gfx950). Placeholder: the
// decode kernel handles every M until the MFMA kernel is in place.
#include <cstdint>
#include <cstdlib>

#include "owq_launch.h"

namespace owq {

int64_t gemm_min_m() { return INT64_MAX; }

hipError_t launch_gemm(const LinearDesc&, int64_t, hipStream_t) { return hipErrorNotSupported; }

}  // namespace owq
