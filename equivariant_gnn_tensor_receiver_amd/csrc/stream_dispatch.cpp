// Host dispatch of the edge-stream kernels to their per-(mode, dtype) instantiations.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

#define TP_DECL(name) hipError_t name(int lmax, int K, const StreamArgs& a, int64_t items, hipStream_t s);
TP_DECL(launch_stream_fwd_f32)
TP_DECL(launch_stream_fwd_bf16)
TP_DECL(launch_stream_jvp_f32)
TP_DECL(launch_stream_jvp_bf16)
TP_DECL(launch_stream_bpos_f32)
TP_DECL(launch_stream_bpos_bf16)
TP_DECL(launch_stream_hess_f32)
TP_DECL(launch_stream_hess_bf16)
TP_DECL(launch_stream_snd_f32)
TP_DECL(launch_stream_sndt_f32)
#undef TP_DECL

hipError_t launch_stream(int mode, int lmax, int K, bool bf16, const StreamArgs& a, int64_t items,
                         hipStream_t s) {
  TimingScope ts(mode == kBwdHess ? (int)kcStreamHess : kcStreamFwd + mode, s);
  switch (mode) {
    case kFwd: return bf16 ? launch_stream_fwd_bf16(lmax, K, a, items, s) : launch_stream_fwd_f32(lmax, K, a, items, s);
    case kJvp: return bf16 ? launch_stream_jvp_bf16(lmax, K, a, items, s) : launch_stream_jvp_f32(lmax, K, a, items, s);
    case kBwdPos:
      return bf16 ? launch_stream_bpos_bf16(lmax, K, a, items, s) : launch_stream_bpos_f32(lmax, K, a, items, s);
    case kBwdHess:
      return bf16 ? launch_stream_hess_bf16(lmax, K, a, items, s) : launch_stream_hess_f32(lmax, K, a, items, s);
    case kSnd: return launch_stream_snd_f32(lmax, K, a, items, s);
    case kSndT: return launch_stream_sndt_f32(lmax, K, a, items, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpconv
