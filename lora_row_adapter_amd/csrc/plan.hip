// plan.hip -- the plan kernel (for lora_plan and for base GEMMs that cannot
// carry the plan in their own launch) and the page-table translation kernel.
#include <mutex>
#include <unordered_map>

#include "plan_body.hpp"

namespace lora {

namespace {

// The layer runs this kernel on a side stream beside its base GEMM, whose
// split-K workgroups hold three waves of 160 VGPRs per SIMD: it keeps
// running there only while it needs at most 32 VGPRs (at 40 it waited for
// the GEMM to finish and the 70B q+v step lost ~10%).
template <int NT>
__global__ __launch_bounds__(NT) void k_plan(PlanArgs a, uint32_t lds_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t plan_lds[];
  plan_detail::plan_body<NT>(a, plan_lds, lds_bytes);
}

__global__ __launch_bounds__(256) void k_translate(AdapterRef ar, int32_t S, int64_t n_pages,
                                                   const int32_t *adapter, const int64_t *off,
                                                   int64_t n, int64_t *phys) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t a = adapter[i];
  const int64_t o = off[i];
  int64_t out = -1;
  if (a >= 0 && a < S && o >= 0) {
    const int64_t lp = o >> ar.page_shift;
    if (lp < ar.max_pages) {
      const int64_t p = ar.page_table[(int64_t)a * ar.max_pages + lp];
      if (p >= 0 && p < n_pages) out = (p << ar.page_shift) + (o & (ar.page_bytes - 1));
    }
  }
  phys[i] = out;
}

}  // namespace

// LDS sized to the batch: the small-adapter-count plan for up to 64
// adapters, else the counting sort where its per-wave histograms fit in
// kMaxLds, else the bitonic sort (each with 1024 threads for batches of more
// than 1024 rows, else 256)
static void plan_shape(const PlanArgs &a, size_t kMaxLds, int *nt, size_t *lds) {
  const bool large = (1 << a.row_bits) > 1024;
  if (a.S <= 64) {
    *nt = large ? kPlanThreads : 256;
    *lds = plan_detail::plan_small_lds(a.M, *nt);
    if (*lds <= kMaxLds) return;
  }
  const size_t c1024 = plan_detail::plan_count_lds(a.M, a.S, kPlanThreads);
  const size_t c256 = plan_detail::plan_count_lds(a.M, a.S, 256);
  if (large && c1024 <= kMaxLds) {
    *nt = kPlanThreads;
    *lds = c1024;
  } else if (c256 <= kMaxLds) {
    *nt = 256;
    *lds = c256;
  } else {
    *nt = large ? kPlanThreads : 256;
    *lds = plan_detail::plan_sort_lds(a.row_bits);
  }
}

hipError_t launch_plan(const PlanArgs &a, hipStream_t st, size_t max_lds) {
  int nt;
  size_t lds;
  plan_shape(a, max_lds, &nt, &lds);
  if (nt == 256)
    hipLaunchKernelGGL(k_plan<256>, dim3(1), dim3(256), lds, st, a, (uint32_t)lds);
  else
    hipLaunchKernelGGL(k_plan<kPlanThreads>, dim3(1), dim3(kPlanThreads), lds, st, a,
                       (uint32_t)lds);
  return hipGetLastError();
}

bool kernel_attributes(const void *fn, hipFuncAttributes *out) {
  static std::mutex mu;
  static std::unordered_map<const void *, hipFuncAttributes> cache;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find(fn);
  if (it == cache.end()) {
    hipFuncAttributes at{};
    if (hipFuncGetAttributes(&at, fn) != hipSuccess) return false;
    it = cache.emplace(fn, at).first;
  }
  *out = it->second;
  return true;
}

bool plan_footprint(const PlanArgs &a, KernelFootprint *out) {
  int nt;
  size_t lds;
  plan_shape(a, kPlanLdsBeside, &nt, &lds);
  hipFuncAttributes at{};
  if (!kernel_attributes(nt == 256 ? (const void *)k_plan<256> : (const void *)k_plan<kPlanThreads>, &at))
    return false;
  out->threads = nt;
  out->vgprs = at.numRegs;
  out->lds = at.sharedSizeBytes + lds;
  return true;
}

bool fits_beside(const KernelFootprint &a, const KernelFootprint &b) {
  auto waves_per_simd = [](int threads) { return ((threads + 63) / 64 + 3) / 4; };
  auto alloc = [](int v) { return (v + 7) / 8 * 8; };
  const int vg = waves_per_simd(a.threads) * alloc(a.vgprs) + waves_per_simd(b.threads) * alloc(b.vgprs);
  return vg <= 512 && a.lds + b.lds <= 160 * 1024;
}

hipError_t launch_translate(const AdapterRef &ar, int32_t S, int64_t n_pages,
                            const int32_t *adapter, const int64_t *off, int64_t n,
                            int64_t *phys, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_translate, dim3((unsigned)blocks), dim3(256), 0, st, ar, S, n_pages,
                     adapter, off, n, phys);
  return hipGetLastError();
}

}  // namespace lora
