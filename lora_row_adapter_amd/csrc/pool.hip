// pool.hip -- device side of the adapter pool manager.
//
// "S-LoRA: ...", section "Unified paging": each adapter finds its weights
// through a list of fixed-size blocks of one pool.  The manager decides the
// placement on the host; these kernels carry it out on the caller's stream:
//
//   k_pool_rows  writes the page-table rows and ranks of a batch of adapters
//                (loaded ones get their pages, evicted ones -1).  The values
//                travel in the kernel arguments, so no host buffer has to
//                outlive the call.
//   k_pool_pull  copies the adapters' weights into their pages, reading the
//                caller's pinned host memory directly over the host link
//                (one workgroup per chunk of at most 64 KiB inside one page;
//                the destination page comes from the row written just
//                before).  One launch replaces one DMA copy per page run:
//                separate copies pay a fixed cost each, which for the
//                adapters of a batch costs more than the transfer itself.
//
// "Your LoRA Adapters Are Thrashing Your GPUs", section 03 "The True Cost of
// an Adapter Swap": the weight transfer over the host link is the part of a
// swap that moves data; it is what k_pool_pull does.
#include "kernels.hpp"

namespace lora {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_pool_fill(int32_t *p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

// One workgroup per row piece: columns j0 .. j0 + n_vals - 1 from v, and for
// the last piece of a row -1 in every later column and the rank.
__global__ __launch_bounds__(256) void k_pool_rows(PoolRowsArgs a) {
  const PoolRow r = a.row[blockIdx.x];
  int32_t *row = a.page_table + (int64_t)r.adapter * a.max_pages;
  const int jend = r.last ? a.max_pages : r.j0 + r.n_vals;
  for (int j = r.j0 + (int)threadIdx.x; j < jend; j += 256)
    row[j] = j - r.j0 < r.n_vals ? a.v[r.v0 + (j - r.j0)] : -1;
  if (threadIdx.x == 0 && r.last) a.ranks[r.adapter] = r.rank;
}

// dst[i] = src[i] for i < n bytes; 16-byte vectors when everything is
// 16-byte aligned, else 2-byte elements (every size here is a multiple of 2).
__device__ inline void pull_range(const uint8_t *src, uint8_t *dst, int64_t n) {
  if ((((uintptr_t)src | (uintptr_t)dst | (uintptr_t)n) & 15) == 0) {
    const u32x4_t *s = reinterpret_cast<const u32x4_t *>(src);
    u32x4_t *d = reinterpret_cast<u32x4_t *>(dst);
    const int64_t n16 = n >> 4;
    for (int64_t i = threadIdx.x; i < n16; i += 4 * 256) {
      u32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i + u * 256 < n16) v[u] = __builtin_nontemporal_load(s + i + u * 256);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i + u * 256 < n16) d[i + u * 256] = v[u];
    }
  } else {
    const uint16_t *s = reinterpret_cast<const uint16_t *>(src);
    uint16_t *d = reinterpret_cast<uint16_t *>(dst);
    for (int64_t i = threadIdx.x; i < (n >> 1); i += 256) d[i] = s[i];
  }
}

__global__ __launch_bounds__(256) void k_pool_pull(PoolPullArgs a) {
  const int c = blockIdx.x;
  int di = 0;
  for (int j = 1; j < a.n_desc; ++j)
    if (a.d[j].chunk0 <= c) di = j;
  const PoolPullDesc D = a.d[di];
  const int64_t L0 = (int64_t)(c - D.chunk0) << a.log2_chunk;
  if (L0 >= D.total) return;
  const int64_t L1 = min(L0 + ((int64_t)1 << a.log2_chunk), D.total);
  const int32_t pg = a.page_table[(int64_t)D.adapter * a.max_pages + (L0 >> a.log2_page)];
  if (pg < 0) return;  // cannot happen: the row was written just before
  // device address of logical byte L0 (the chunk lies inside one page)
  uint8_t *dst = a.pool + ((int64_t)pg << a.log2_page) + (L0 & (((int64_t)1 << a.log2_page) - 1));
  // logical bytes [0, a_bytes) come from A, [a_bytes, total) from B
  if (L0 < D.a_bytes) {
    const int64_t e = min(L1, D.a_bytes);
    pull_range(D.a + L0, dst, e - L0);
  }
  if (L1 > D.a_bytes) {
    const int64_t s = max(L0, D.a_bytes);
    pull_range(D.b + (s - D.a_bytes), dst + (s - L0), L1 - s);
  }
}

hipError_t launch_pool_fill(int32_t *p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(k_pool_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_pool_rows(const PoolRowsArgs &a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pool_rows, dim3(a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pool_pull(const PoolPullArgs &a, hipStream_t st) {
  if (a.n_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pool_pull, dim3(a.n_chunks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
