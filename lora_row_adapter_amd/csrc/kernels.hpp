// kernels.hpp -- host-side launchers of the HIP kernels (internal to liblora_row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_row.h"
#include "common.hpp"

namespace lora {

// Byte offsets of the workspace regions, laid out for `rows` rows (<= the
// plan limit), S adapters and max rank R.  Every region is 256-byte aligned.
struct WsLayout {
  int64_t rows = 0;
  int64_t seg_cap = 0;
  int64_t items_g_cap = 0;
  int64_t items_s_cap = 0;
  int32_t R = 0;  // fp32 partial row width: max rank rounded up to 4
  size_t hdr = 0, perm = 0, seg_adapter = 0, seg_start = 0, seg_len = 0;
  size_t items_g = 0, items_gx = 0, items_s = 0, tpart = 0, total = 0;
};
WsLayout ws_layout(int64_t rows, int32_t S, int32_t R, int32_t n_slices);

// Per-slice validity data the plan checks for each adapter.
struct PlanSlice {
  const int32_t *ranks;
  int32_t R;
  // pool checks (page_table == nullptr for slots)
  const int32_t *page_table;
  int32_t max_pages;
  int64_t n_pages;
  int64_t page_bytes;
  int64_t bytes_per_rank;  // (k + d) * elem_bytes
};

struct PlanArgs {
  const int32_t *ids;
  int32_t M;
  int32_t S;
  int32_t row_bits;  // log2 of the sort width
  int32_t n_slices;
  PlanSlice sl[kMaxSlices];
  // outputs
  uint8_t *ws;
  WsLayout L;
};

struct LoraArgs {
  int32_t dtype;  // 0 f32, 1 bf16
  int64_t k;
  const void *x;
  int64_t ldx;
  void *y;
  int64_t ldy;
  int32_t y_vec;    // y base 16-byte aligned and ldy a multiple of 16 bytes
  int32_t n_slices;
  int32_t R;        // max rank over slices (partials row width)
  SliceRef sl[kMaxSlices];
  int32_t col_blk[kMaxSlices + 1];  // prefix of expand column blocks per slice
  uint8_t *ws;
  WsLayout L;
  int32_t ksplit;
  int64_t kchunk;  // k per split (multiple of 256)
  // > 0: this call's base GEMM computed t into split 0 of the partials,
  // indexed by row (no shrink launch); the expand reads that t
  int32_t fused_cap;
};

// max_lds: dynamic LDS the plan may take -- kPlanLdsBeside when it runs
// beside a GEMM, kPlanLdsAlone when it has the CU to itself (the 1024-thread
// counting sort then serves more adapters)
constexpr size_t kPlanLdsBeside = 65536, kPlanLdsAlone = 152 * 1024;
hipError_t launch_plan(const PlanArgs &a, hipStream_t st, size_t max_lds = kPlanLdsBeside);

// Resources of one workgroup of a kernel: threads, VGPRs per lane (arch +
// accumulation registers), LDS bytes (static + dynamic).
struct KernelFootprint {
  int threads = 0;
  int vgprs = 0;
  size_t lds = 0;
};
// hipFuncGetAttributes of a kernel, cached (the library is built for one
// architecture, so the attributes do not depend on the device).
bool kernel_attributes(const void *fn, hipFuncAttributes *out);
// What launch_plan would launch for these arguments.
bool plan_footprint(const PlanArgs &a, KernelFootprint *out);
// What launch_gemm (fused = false) or launch_gemm_fused (true) would launch.
bool gemm_footprint(int32_t dtype, int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw,
                    void *gws, size_t gws_bytes, bool fused, KernelFootprint *out);
// Whether a workgroup of `b` fits on a CU beside one workgroup of `a`
// (gfx950: 4 SIMDs of 512 VGPRs per lane, VGPRs allocated in blocks of 8,
// 160 KiB of LDS).
bool fits_beside(const KernelFootprint &a, const KernelFootprint &b);
hipError_t launch_translate(const AdapterRef &ar, int32_t S, int64_t n_pages,
                            const int32_t *adapter, const int64_t *off, int64_t n,
                            int64_t *phys, hipStream_t st);
// The shrink folded into the base GEMM (bf16, adapters in slots).  The
// (slice, adapter, rank) triples with rank < that adapter's rank (clamped
// to [0, max_rank]), in that order, form the columns of t_all = x A_cat^T;
// column tile tn of the GEMM computes columns [16 tn, 16 tn + 16) of t_all
// from 16 extra rows of its W stage, and columns [cap + 16 tn, + 16) -- if
// the ranks sum past cap -- in a second pass after its k loop; it writes
// t[slice][row][rank] (split 0 of the partials layout, indexed by the row
// itself) for the rows whose adapter owns the column.  The caller keeps
// n_slices * S * max_rank <= 2 * cap.
struct FusedT {
  int32_t cap;     // 16 x column tiles of the launch; 0: not fused
  int32_t n_slices, S;
  const uint8_t *A[kMaxSlices];   // slot A [S][R][k] of each slice, or its pool
  int32_t R[kMaxSlices];          // max_rank of each slice (rank stride of slot A)
  // pool slices (page_table != nullptr): A_s row j starts at logical byte
  // j * 2k of adapter s, inside one page (the page size is a multiple of
  // 2k); an entry outside [0, n_pages) or a page past max_pages makes the
  // row read x instead (the plan counts such rows as bad pages, so their t
  // is never used)
  const int32_t *page_table[kMaxSlices];
  int32_t max_pages[kMaxSlices];
  int32_t page_shift[kMaxSlices];
  int64_t n_pages[kMaxSlices];
  const int32_t *ranks[kMaxSlices];
  const int32_t *ids;             // adapter id of each row
  float *tpart;                   // partials region of the workspace
  int64_t rows;                   // its row stride (WsLayout::rows)
  int32_t Rw;                     // its row width (WsLayout::R)
};
constexpr int kFusedMaxEntries = 256;  // n_slices * S the fused path scans
// Base GEMM y = x W^T (bf16 operands: MFMA tiles; fp32: VALU).  gws: the
// GEMM's region of the workspace (split-K partials), 256-byte aligned, or
// nullptr; shapes with gemm_ws_bytes(M, k, d) > 0 run split-K pairs when it
// holds that many bytes, else the unsplit tiles (another summation order).
// expired: where split-K pairs count expired waits (nullptr: word
// kHdrSyncExpired of the GEMM region's own 256-byte header).
// plan: run this plan inside the launch (only where gemm_runs_plan says
// the launch can carry it; else nullptr).
hipError_t launch_gemm(int32_t dtype, int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                       const void *W, int64_t ldw, void *y, int64_t ldy, void *gws,
                       size_t gws_bytes, hipStream_t st, int32_t *expired = nullptr,
                       const PlanArgs *plan = nullptr);
// Whether the base GEMM launch of this shape (and GEMM region, and fold)
// carries the layer's plan: split-K pairs (the first-arriving workgroup of
// pair 0 runs it), or MFMA tiles whose kernel fits twice on a CU (one more
// workgroup runs it beside the tiles).  launch_gemm(_fused) with a plan
// where this is false fails with hipErrorInvalidValue.
bool gemm_runs_plan(int32_t dtype, int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw,
                    void *gws, size_t gws_bytes, bool fused);
// Bound of the split-K pairs' wait in polls for later launches (< 0: the
// default); a test hook that makes every wait expire at once with 0 (an
// expired wait is counted; that tile is wrong).
void set_sync_spin_limit(int32_t polls);
// Bytes of GEMM workspace the split-K launch of this shape uses (0: none).
size_t gemm_ws_bytes(int64_t M, int64_t k, int64_t d);
// Capacity (t_all columns) a fused launch of this shape would have; 0 when
// the shape's tile cannot carry the extra rows.
int32_t gemm_fused_cap(int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw);
// The base GEMM with the shrink folded in (ft.cap == gemm_fused_cap(...)).
hipError_t launch_gemm_fused(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                             const void *W, int64_t ldw, void *y, int64_t ldy, const FusedT &ft,
                             void *gws, size_t gws_bytes, hipStream_t st,
                             int32_t *expired = nullptr, const PlanArgs *plan = nullptr);
// Base GEMM with a quantized weight (bf16 x and y).
struct QGemmArgs {
  int32_t fmt;  // 1 INT8 (per-row scales), 2 INT4 (per-row, per-k-group scales)
  int M, N, K;
  const uint16_t *x;
  int64_t ldx;            // elements
  const uint8_t *q;
  int64_t ldq;            // bytes
  const float *scales;    // INT8 [N]; INT4 [N, ngroups]
  int32_t group;          // INT4 k-group (multiple of 64)
  int32_t ngroups;        // INT4: K / group; INT8: 1
  uint16_t *y;
  int64_t ldy;
  int tiles_m, tiles_n;
  int vec_store;
};
hipError_t launch_gemm_q(const QGemmArgs &a, hipStream_t st);
hipError_t launch_shrink_gather(const LoraArgs &a, hipStream_t st);
hipError_t launch_expand_gather(const LoraArgs &a, hipStream_t st);
// A rows per stage the LDS-staged SGMV shrink takes for this launch (per
// slice: the largest max_rank, else the sum over slices, each rounded up to
// 16; as 16, 32, 64 or 128), or 0 where it cannot run (fp32, x past 32-bit
// offsets, more than 128 rows).
int shrink_dma_rows(const LoraArgs &a, bool per_slice);
hipError_t launch_shrink_sgmv(const LoraArgs &a, int rows_per_item, bool per_slice,
                              hipStream_t st);
hipError_t launch_expand_sgmv(const LoraArgs &a, int rows_per_item, hipStream_t st);
constexpr int kMaxRankMfma = 64;

// Adapter pool manager.  Kernel arguments carry the page lists and the
// copy descriptors (each struct stays under 4 KiB).
constexpr int kPoolRowsMax = 32;     // rows per k_pool_rows launch
constexpr int kPoolRowVals = 768;    // page entries per k_pool_rows launch
struct PoolRow {    // columns [j0, j0 + n_vals) of one row, from v[v0 ...]
  int32_t adapter;
  int32_t rank;      // -1: evicted
  int32_t n_vals;
  int32_t v0;
  int32_t j0;
  int32_t last;      // last piece of the row: columns after it get -1, the rank is written
};
struct PoolRowsArgs {
  int32_t *page_table;
  int32_t *ranks;
  int32_t max_pages;
  int32_t n_rows;
  PoolRow row[kPoolRowsMax];
  int32_t v[kPoolRowVals];
};
constexpr int kPoolPullMax = 64;  // adapters per k_pool_pull launch
struct PoolPullDesc {
  const uint8_t *a;  // device-visible address of host A (rank x k)
  const uint8_t *b;  // device-visible address of host B (d x rank)
  int64_t a_bytes;
  int64_t total;     // a_bytes + b_bytes
  int32_t adapter;
  int32_t chunk0;    // first chunk (workgroup) of this adapter
};
struct PoolPullArgs {
  uint8_t *pool;
  const int32_t *page_table;
  int32_t max_pages;
  int32_t log2_page;
  int32_t log2_chunk;  // <= log2_page
  int32_t n_desc;
  int32_t n_chunks;
  PoolPullDesc d[kPoolPullMax];
};
// Merged weight of one adapter: Wo = W + coef * scales[adapter] * B A.
struct MergeArgs {
  int32_t dtype;  // 0 f32, 1 bf16
  int64_t d, k;
  const uint8_t *W;
  int64_t ldw;    // elements
  uint8_t *Wo;
  int64_t ldo;
  AdapterRef ar;
  const int32_t *ranks;
  const float *scales;
  int32_t adapter;
  float coef;
  int32_t rp;      // bf16 LDS rank capacity: max_rank rounded up to 32
  int64_t n_pages; // pool: pages in the pool
};
hipError_t launch_merge(const MergeArgs &m, hipStream_t st);

hipError_t launch_pool_fill(int32_t *p, int64_t n, int32_t v, hipStream_t st);
hipError_t launch_pool_rows(const PoolRowsArgs &a, hipStream_t st);
hipError_t launch_pool_pull(const PoolPullArgs &a, hipStream_t st);

// The multi-slice layer behind lora_linear_sliced(_q) (the C ABI's types;
// defined in lora_api.cpp).  self_contained: create no library resource --
// the plan runs on the caller's stream and no launch is timed.
lora_status_t linear_sliced_impl(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                 int64_t ldx, const void *W, int64_t ldw, const lora_qweight_t *qw,
                                 int32_t n_slices, const lora_slice_t *slices,
                                 const int32_t *adapter_ids, void *y, int64_t ldy, void *workspace,
                                 size_t workspace_bytes, int32_t path, uint32_t flags, void *stream,
                                 bool self_contained);

}  // namespace lora
