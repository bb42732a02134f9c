// The accumulating edge streams as per-node products on the matrix cores,
// compiled once per (mode, feature planes):
//   -DTP_MODE=<kFwd|kJvp|kSnd|kSndT> -DTP_LO=<0|1> -DTP_LAUNCHER=<name>
// (TP_LO: fp32 features reach the kernel as pre-split bf16 hi / lo planes;
// otherwise the features are bf16)
#include "stream_gf.h"

namespace tpconv {

hipError_t TP_LAUNCHER(int lmax, int K, const StreamArgs& a, int64_t /*items*/, hipStream_t s) {
  return launch_gf<TP_MODE, TP_LO != 0>(lmax, K, a, s);
}

}  // namespace tpconv
