// Per-kernel event timing: a table of (class, start, stop) event pairs that is
// filled while timing is enabled and summed on read.  Events are recycled
// through a pool so steady-state timing allocates nothing.
#include "timing.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace tpconv {
namespace {

struct Record {
  int cls;
  hipEvent_t start, stop;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_all() {
  for (auto& r : g_records) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace

TimingScope::TimingScope(int cls, hipStream_t s) : cls_(cls), s_(s) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  if (start_ && hipEventRecord(start_, s_) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

TimingScope::~TimingScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, s_) != hipSuccess) {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
    return;
  }
  g_records.push_back({cls_, start_, stop});
}

bool timing_enabled() { return g_enabled.load(); }

bool timing_set(bool enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_records)
    if (hipEventSynchronize(r.stop) != hipSuccess) return false;
  recycle_all();
  g_enabled.store(enable);
  return true;
}

bool timing_read(int cls, long long* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  long long n = 0;
  double ms = 0.0;
  for (auto& r : g_records) {
    if (r.cls != cls) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return false;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return false;
    ++n;
    ms += t;
  }
  *launches = n;
  *total_ms = ms;
  return true;
}

}  // namespace tpconv
