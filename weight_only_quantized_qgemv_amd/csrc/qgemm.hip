// qgemm.hip — prefill path (M > 16). Placeholder routing through the GEMV in
// chunks until the MFMA kernel lands.
#include "launch.hpp"

namespace qp {

hipError_t launch_qgemm(const GemvArgs& a, hipStream_t stream) { return launch_qgemv(a, stream); }

} // namespace qp
