// Event-pair profiling of the contraction kernels (host code). When enabled,
// every wq_matmul_add_rmsnorm / mx_quant_matmul_inplace_add call records a
// pair of HIP events on its stream around its contraction kernel (the MFMA
// tile, the decode weight stream or the generic tile), so a caller can time
// that kernel alone, on the stream it runs on, without a profiler.
// This is a measurement aid and the library's only process-wide state: with
// profiling off (the default) a launch reads one atomic flag and takes no
// lock.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "wq.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kMaxPairs = 4096;

struct Profile {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;   // 2 * kMaxPairs events, created on first enable
  int used = 0;                 // pairs recorded since the last enable / read
  int64_t launches = 0;         // launches seen (including any past kMaxPairs)
};

Profile& prof() {
  static Profile p;
  return p;
}

}  // namespace

void prof_begin(hipStream_t s) {
  Profile& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on) return;
  ++p.launches;
  if (p.used < kMaxPairs) (void)hipEventRecord(p.ev[2 * p.used], s);
}

void prof_end(hipStream_t s) {
  Profile& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || p.used >= kMaxPairs) return;
  (void)hipEventRecord(p.ev[2 * p.used + 1], s);
  ++p.used;
}

}  // namespace wq

extern "C" wq_status wq_profile_enable(int enable) {
  wq::Profile& p = wq::prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (enable && p.ev.empty()) {
    p.ev.resize(2 * wq::kMaxPairs);
    for (auto& e : p.ev)
      if (hipEventCreate(&e) != hipSuccess) {
        p.ev.clear();
        return WQ_ERR_LAUNCH;
      }
  }
  p.on = enable != 0;
  p.used = 0;
  p.launches = 0;
  return WQ_OK;
}

extern "C" wq_status wq_profile_read(float* times_ms, int64_t capacity, int64_t* launches) {
  if (!launches || (capacity > 0 && !times_ms)) return WQ_ERR_NULLPTR;
  wq::Profile& p = wq::prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (int i = 0; i < p.used; ++i) {
    if (hipEventSynchronize(p.ev[2 * i + 1]) != hipSuccess) return WQ_ERR_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) return WQ_ERR_LAUNCH;
    if (i < capacity) times_ms[i] = ms;
  }
  *launches = p.used;
  p.used = 0;
  p.launches = 0;
  return WQ_OK;
}
