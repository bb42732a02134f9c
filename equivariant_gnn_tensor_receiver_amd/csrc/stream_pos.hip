// The position-gradient stream, compiled once per feature dtype:
//   -DTP_FT=<float|uint16_t> -DTP_LAUNCHER=<name>
// (fp32 features reach the kernel as pre-split bf16 hi / lo planes)
#include "stream_pos.h"

namespace tpconv {

hipError_t TP_LAUNCHER(int lmax, int K, const StreamArgs& a, int64_t /*items*/, hipStream_t s) {
  return launch_pos<std::is_same<TP_FT, float>::value>(lmax, K, a, s);
}

}  // namespace tpconv
