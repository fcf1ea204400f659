// wq_matmul_add_rmsnorm_noalloc: the fused weight-quantized matmul +
// AddRmsNorm for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops that forbid allocation). The kernels of
// wq_matmul_add_rmsnorm run unchanged; their workspace is a file-scope device
// array of kNoallocScratchBytes instead of a caller buffer.
//
// The array exists once per GPU the library runs on and lives until the
// process ends. In host code its name is only a stand-in for the symbol:
// the device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is ever passed to
// a kernel. Every call on one GPU shares the array; the kernels need no
// initial contents (each call writes what it reads), and calls that overlap
// on one GPU (different streams, no ordering) race on it.
#include <atomic>
#include <mutex>

#include "wq_internal.h"

namespace {

constexpr size_t kNoallocScratchBytes = WQ_NOALLOC_MAX_WORKSPACE;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's copy of the array (nullptr if the
// lookup fails).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    p = q;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" wq_status wq_matmul_add_rmsnorm_noalloc(
    const void* x1, int64_t m, int64_t k, wq_dtype act_dtype, const void* x2, int64_t n,
    wq_dtype w_dtype, wq_layout x2_layout, int transpose_x2, const void* antiquant_scale,
    int64_t scale_rows, int64_t scale_cols, const void* antiquant_offset,
    int64_t antiquant_group_size, const void* bias, const void* residual, const void* gamma,
    double epsilon, void* y, void* norm_out, hipStream_t stream) {
  // the size rule comes first, so that a call the array cannot serve never
  // touches the device (wq_matmul_add_rmsnorm_workspace_size is pure host)
  if (m > 0 && k > 0 && n > 0 &&
      wq_matmul_add_rmsnorm_workspace_size(m, k, n) > kNoallocScratchBytes)
    return WQ_ERR_WORKSPACE;
  // every other rule is the workspace call's; a device whose array cannot be
  // located passes no workspace (WQ_ERR_WORKSPACE for any non-empty problem)
  void* ws = device_scratch();
  return wq_matmul_add_rmsnorm(x1, m, k, act_dtype, x2, n, w_dtype, x2_layout, transpose_x2,
                               antiquant_scale, scale_rows, scale_cols, antiquant_offset,
                               antiquant_group_size, bias, residual, gamma, epsilon, y, norm_out,
                               ws, ws ? kNoallocScratchBytes : 0, stream);
}
