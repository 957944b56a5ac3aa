// gns_gram_batched_noalloc: gns_gram_batched for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a file-scope device
// array of fixed size that each GPU holds from the library's first use on it
// until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gns.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // GNS_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GNS_NOALLOC_SCRATCH_BYTES, "header and library agree on the size");

// One copy per GPU, at its own address on each.  In host code this name is
// only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (the current device's),
// looked up on the first call on that device; nullptr on failure.
void *scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" gns_status gns_gram_batched_noalloc(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                                               gns_dtype io_dtype, gns_dtype compute_dtype,
                                               const double *coeffs, int T, const int *restart_after,
                                               int n_restart, const int64_t *row_idx, int64_t k,
                                               unsigned opts, void *stream) {
  // no library streams or events (creating them may allocate), no timing
  // runs and no synchronous checks: everything runs on `stream` with the size
  // rule's tiles
  if (opts & (GNS_OPT_TILE_AUTOTUNE | GNS_OPT_DEBUG_CHECKS)) return GNS_E_FLAGS;
  opts |= GNS_OPT_ONE_STREAM;
  const int64_t rows = row_idx ? k : n;
  const size_t need = batch > 0 ? gns_gram_workspace_bytes(compute_dtype, batch, rows, m) : 0;
  if (batch <= 0 || need == 0 || need > kScratchBytes) {
    // validation only (no workspace: nothing is enqueued): argument errors
    // are reported exactly as gns_gram_batched reports them, and a problem
    // whose workspace exceeds the array is GNS_E_WORKSPACE
    const gns_status st = gns_gram_batched(X, out, batch, n, m, io_dtype, compute_dtype, coeffs, T, restart_after,
                                           n_restart, row_idx, k, opts, nullptr, 0, stream);
    return (st == GNS_OK && batch > 0) ? GNS_E_WORKSPACE : st;
  }
  void *ws = scratch_for_current_device();
  if (!ws) return GNS_E_HIP;
  return gns_gram_batched(X, out, batch, n, m, io_dtype, compute_dtype, coeffs, T, restart_after, n_restart,
                          row_idx, k, opts, ws, kScratchBytes, stream);
}
