// Forward pass without any allocation: the receiver state S lives in a
// file-scope device array instead of caller-provided workspace, for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// Every GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  The host-side name of the array is not a
// device address, so its address on the current device is looked up once per
// device (hipGetSymbolAddress) and only that pointer is handed to kernels.
// All calls on one GPU share the array: calls that overlap on one GPU race.
// The forward stream writes every entry of S (nodes without edges get zeros),
// so nothing has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/tpconv.h"

namespace tpconv {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // TPCONV_STATIC_SCRATCH_BYTES
static_assert(kScratchBytes == TPCONV_STATIC_SCRATCH_BYTES, "header and library disagree on the scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Address of this device's copy of `scratch`, looked up on the first call on
// the device (with that device current).  nullptr on failure.
void* scratch_on_current_device() {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[d]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[d] = p;
  }
  return g_ptr[d];
}

}  // namespace
}  // namespace tpconv

extern "C" tpconv_status tpconv_forward_static(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                                               const void* x, const void* W, float* out, void* stream) {
  if (!plan || !g || g->num_nodes < 0) return TPCONV_ERROR_INVALID_VALUE;
  size_t need = 0;
  tpconv_status st = tpconv_workspace_size(plan, TPCONV_OP_FORWARD, g->num_nodes, g->num_edges, &need);
  if (st != TPCONV_SUCCESS) return st;
  if (need > tpconv::kScratchBytes) return TPCONV_ERROR_SCRATCH;
  void* ws = tpconv::scratch_on_current_device();
  if (!ws) return TPCONV_ERROR_DEVICE;
  return tpconv_forward(plan, g, pos, x, W, out, nullptr, ws, tpconv::kScratchBytes, stream);
}
