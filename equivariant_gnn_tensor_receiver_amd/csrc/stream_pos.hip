// The position-gradient stream, compiled once per feature dtype:
//   -DTP_FT=<float|uint16_t> -DTP_HESS=<0|1> -DTP_LAUNCHER=<name>
// (TP_HESS: the position derivative of the force loss instead of the gradient)
// (fp32 features reach the kernel as pre-split bf16 hi / lo planes)
#include "stream_pos.h"

namespace tpconv {

hipError_t TP_LAUNCHER(int lmax, int K, const StreamArgs& a, int64_t /*items*/, hipStream_t s) {
  return launch_pos<std::is_same<TP_FT, float>::value, TP_HESS != 0>(lmax, K, a, s);
}

}  // namespace tpconv
