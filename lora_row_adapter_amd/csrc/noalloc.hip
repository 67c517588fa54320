// noalloc.hip -- lora_linear_sliced_noalloc: the multi-slice layer for callers
// that cannot allocate device memory (code under HIP-graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Instead of a caller's
// workspace it uses `scratch`, a file-scope device array of fixed size that
// every GPU the library runs on holds until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device copy: its
// device address is fetched once per device with hipGetSymbolAddress (with
// that device current) and only that address is handed to kernels.
#include <mutex>

#include "kernels.hpp"

namespace lora {
namespace {

constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;

}  // namespace
}  // namespace lora

// Plan regions, shrink partials and the split-K pairs' partials and words of
// one call.  Zero at load; the split-K words tolerate any contents, and the
// plan writes every region it reads.
static __device__ __align__(256) uint8_t scratch[lora::kScratchBytes];

namespace lora {
namespace {

constexpr int kMaxDev = 64;
std::mutex g_mu;
void *g_ptr[kMaxDev];
bool g_tried[kMaxDev];

// Device address of this device's scratch (nullptr on failure); looked up on
// the first call per device and kept.
void *scratch_ptr(int dev) {
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_tried[dev]) {
    g_tried[dev] = true;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace lora

extern "C" {

lora_status_t lora_linear_sliced_noalloc(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                         int64_t ldx, const void *W, int64_t ldw,
                                         int32_t n_slices, const lora_slice_t *slices,
                                         const int32_t *adapter_ids, void *y, int64_t ldy,
                                         int32_t path, uint32_t flags, void *stream) {
  if (M == 0) {
    return lora::linear_sliced_impl(dtype, M, k, x, ldx, W, ldw, nullptr, n_slices, slices,
                                    adapter_ids, y, ldy, nullptr, 0, path, flags, stream, true);
  }
  // size of the workspace this call needs (host arithmetic only)
  const size_t need = lora_workspace_bytes_sliced(M, k, dtype, n_slices, slices);
  if (need == 0) return LORA_ERR_ARG;  // invalid slices, dtype or sizes
  if (need > lora::kScratchBytes) return LORA_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= lora::kMaxDev) return LORA_ERR_HIP;
  void *ws = lora::scratch_ptr(dev);
  if (ws == nullptr) return LORA_ERR_HIP;
  return lora::linear_sliced_impl(dtype, M, k, x, ldx, W, ldw, nullptr, n_slices, slices,
                                  adapter_ids, y, ldy, ws, lora::kScratchBytes, path, flags, stream,
                                  true);
}

}  // extern "C"
