// Backward ring step (placeholder until the MFMA kernel lands).
#include "ra_internal.h"

namespace ra {

int bwd_block_n(int /*dtype*/, int /*D*/) { return 128; }

hipError_t launch_bwd(int, int, const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ra
