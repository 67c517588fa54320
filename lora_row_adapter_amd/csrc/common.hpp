// common.hpp -- device-side types and helpers shared by the HIP kernels of
// liblora_row (gfx950).  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

// ---------------------------------------------------------------------------
// Tunables fixed at build time (the host lays out workspaces with them).
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxRows = 8192;  // LORA_PLAN_MAX_ROWS
constexpr int kRowsPerGatherItem = 16;  // rows per shrink/expand work item (gather path)
constexpr int kRowsPerSgmvItem = 64;    // rows per work item (SGMV path)
constexpr int kMaxKSplit = 16;          // k-splits of the shrink (fp32 partials)
constexpr int kMaxRank = 256;
constexpr int kMaxSlices = 4;           // projections sharing x in one call (e.g. q, k, v, o)

// Header words at the start of a workspace (int32).
enum HdrWord {
  kHdrBadIds = 0,
  kHdrBadRanks = 1,
  kHdrBadPages = 2,
  kHdrAdapted = 3,
  kHdrSegments = 4,
  kHdrItemsGather = 5,
  kHdrItemsSgmv = 6,
  kHdrRows = 7,
  // Split-K pairs of the base GEMM whose second workgroup stopped waiting for
  // the first one's partial (bounded wait; the tile is then wrong).  Sticky:
  // the plan never writes it, the GEMM only adds to it.
  kHdrSyncExpired = 8,
  kHdrWords = 64
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Cache-policy bit of buffer accesses: device (agent) scope, coherent across
// the XCDs' L2 caches.
constexpr int kCpolSc1 = 16;

// bf16 <-> fp32.  bf16 is the upper half of an fp32; widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round-to-nearest-even narrowing (NaN kept quiet): gfx950's
// v_cvt_pk_bf16_f32.  Checked on the device against the integer form
// (add 0x7fff plus the kept lsb, NaNs quieted) on all 2^32 fp32 patterns:
// identical.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values in one instruction: lo in bits 0-15, hi in bits 16-31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Work item of the LoRA kernels: `nrows` consecutive entries of the sorted
// row permutation starting at `pos`, all using adapter `adapter`.
struct Item {
  int32_t adapter;
  int32_t pos;
  int32_t nrows;
  int32_t seg;
};

// Beside each 16-row work item: the adapter's rank in every slice and the
// item's rows (perm[pos .. pos + nrows)), so a kernel reads them together
// with the item instead of one dependent load after another.
struct ItemRows {
  int32_t r[kMaxSlices];
  int32_t rows[kRowsPerGatherItem];
};

// Where one adapter's A and B live.  SLOTS: A [S, R, k] and B [S, d, R];
// POOL: logical space [A r x k | B d x r] cut into pages.
struct AdapterRef {
  const uint8_t *A;        // SLOTS
  const uint8_t *B;        // SLOTS
  const uint8_t *pool;     // POOL
  const int32_t *page_table;
  int64_t page_bytes;
  int32_t page_shift;
  int32_t max_pages;
  int32_t max_rank;
  int32_t pooled;
  int64_t k;
  int64_t d;
  int32_t elem_bytes;
};

// Byte address of A_s[j][kk] (a vector starting there never crosses a page
// as long as it is aligned to its own size and the page size is a multiple).
__device__ __forceinline__ const uint8_t *adapter_a_ptr(const AdapterRef &ar, int s, int r,
                                                        int64_t j, int64_t kk) {
  if (!ar.pooled) {
    return ar.A + (((int64_t)s * ar.max_rank + j) * ar.k + kk) * ar.elem_bytes;
  }
  int64_t off = (j * ar.k + kk) * ar.elem_bytes;
  int64_t page = ar.page_table[(int64_t)s * ar.max_pages + (off >> ar.page_shift)];
  return ar.pool + (page << ar.page_shift) + (off & (ar.page_bytes - 1));
}

// Byte address of B_s[n][j].
__device__ __forceinline__ const uint8_t *adapter_b_ptr(const AdapterRef &ar, int s, int r,
                                                        int64_t n, int64_t j) {
  if (!ar.pooled) {
    return ar.B + (((int64_t)s * ar.d + n) * ar.max_rank + j) * ar.elem_bytes;
  }
  int64_t off = ((int64_t)r * ar.k + n * r + j) * ar.elem_bytes;
  int64_t page = ar.page_table[(int64_t)s * ar.max_pages + (off >> ar.page_shift)];
  return ar.pool + (page << ar.page_shift) + (off & (ar.page_bytes - 1));
}

// One projection of a multi-slice call: its adapters, scales and the
// columns [col0, col0 + d) of y it owns.
struct SliceRef {
  AdapterRef ar;
  const int32_t *ranks;
  const float *scales;
  int64_t d;
  int64_t col0;
};

// Index of the fp32 shrink partial of (k split q, sorted position p, slice s,
// rank j): one [rows][slices][R] block per split, so a reader that needs the
// item's rows for every split reads ksplit contiguous runs.
__device__ __forceinline__ int64_t tpart_index(int q, int64_t p, int s, int j, int64_t rows,
                                               int n_slices, int R) {
  return ((q * rows + p) * n_slices + s) * (int64_t)R + j;
}

// t[p, s, j..j+3] = the four k-split sums, in split order (R % 4 == 0).
__device__ __forceinline__ float4 tpart_sum4(const float *tpart, int64_t p, int s, int j,
                                             int ksplit, int64_t rows, int n_slices, int R) {
  float4 v[kMaxKSplit];
#pragma unroll
  for (int q = 0; q < kMaxKSplit; ++q)
    v[q] = q < ksplit ? *reinterpret_cast<const float4 *>(
                            tpart + tpart_index(q, p, s, j, rows, n_slices, R))
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc = v[0];
#pragma unroll
  for (int q = 1; q < kMaxKSplit; ++q) {
    acc.x += v[q].x;
    acc.y += v[q].y;
    acc.z += v[q].z;
    acc.w += v[q].w;
  }
  return acc;
}

// Scalar form for any R.
__device__ __forceinline__ float tpart_sum1(const float *tpart, int64_t p, int s, int j,
                                            int ksplit, int64_t rows, int n_slices, int R) {
  float v[kMaxKSplit];
#pragma unroll
  for (int q = 0; q < kMaxKSplit; ++q)
    v[q] = q < ksplit ? tpart[tpart_index(q, p, s, j, rows, n_slices, R)] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int q = 1; q < kMaxKSplit; ++q) acc += v[q];
  return acc;
}

}  // namespace lora
