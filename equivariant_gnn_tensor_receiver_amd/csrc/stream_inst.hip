// One instantiation set of the edge-stream kernel, selected at compile time:
//   -DTP_MODE=<StreamMode> -DTP_FT=<float|uint16_t> -DTP_LAUNCHER=<name>
// The build compiles this file once per (mode, feature dtype) so that the
// instantiations compile in parallel.
#include "stream_impl.h"

namespace tpconv {

hipError_t TP_LAUNCHER(int lmax, int K, const StreamArgs& a, int64_t items, hipStream_t s) {
  return launch_stream_mode<TP_MODE, TP_FT>(lmax, K, a, items, s);
}

}  // namespace tpconv
