// lora_api.cpp -- host side of the C ABI declared in include/lora_row.h:
// argument validation, workspace layout, step dispatch and the optional
// per-kernel event timer.  Every compute step runs in the HIP kernels; this
// file only checks arguments and launches them on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/lora_row.h"
#include "kernels.hpp"

namespace lora {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int64_t rows, int32_t S, int32_t R) {
  WsLayout L;
  L.rows = std::max<int64_t>(1, rows);
  L.R = R;
  L.seg_cap = std::max<int64_t>(1, std::min<int64_t>(L.rows, S));
  L.items_g_cap = (L.rows + kRowsPerGatherItem - 1) / kRowsPerGatherItem + L.seg_cap;
  L.items_s_cap = (L.rows + kRowsPerSgmvItem - 1) / kRowsPerSgmvItem + L.seg_cap;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.hdr = take(kHdrWords * sizeof(int32_t));
  L.perm = take((size_t)L.rows * sizeof(int32_t));
  L.seg_adapter = take((size_t)L.seg_cap * sizeof(int32_t));
  L.seg_start = take((size_t)L.seg_cap * sizeof(int32_t));
  L.seg_len = take((size_t)L.seg_cap * sizeof(int32_t));
  L.items_g = take((size_t)L.items_g_cap * sizeof(Item));
  L.items_s = take((size_t)L.items_s_cap * sizeof(Item));
  L.tpart = take((size_t)kMaxKSplit * L.rows * R * sizeof(float));
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Optional per-kernel timing (lora_profile_*).
// ---------------------------------------------------------------------------
namespace prof {
constexpr int kRing = 8192;
std::mutex mu;
std::atomic<int> enabled{0};
std::vector<hipEvent_t> ev0, ev1;
std::vector<int> cls;
int used = 0;
int64_t dropped = 0;
double ms[LORA_K_COUNT] = {};
int64_t launches[LORA_K_COUNT] = {};

// Returns the slot index to record into, or -1 (not profiling / ring full).
int begin(int c, hipStream_t st) {
  if (!enabled.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> g(mu);
  if (ev0.empty()) {
    ev0.resize(kRing);
    ev1.resize(kRing);
    cls.resize(kRing);
    for (int i = 0; i < kRing; ++i) {
      if (hipEventCreate(&ev0[i]) != hipSuccess || hipEventCreate(&ev1[i]) != hipSuccess) {
        ev0.clear();
        ev1.clear();
        return -1;
      }
    }
  }
  if (used >= kRing) {
    ++dropped;
    return -1;
  }
  const int i = used++;
  cls[i] = c;
  if (hipEventRecord(ev0[i], st) != hipSuccess) return -1;
  return i;
}
void end(int i, hipStream_t st) {
  if (i < 0) return;
  (void)hipEventRecord(ev1[i], st);
}
}  // namespace prof

template <typename F>
static hipError_t timed(int c, hipStream_t st, F &&launch) {
  const int slot = prof::begin(c, st);
  const hipError_t e = launch();
  prof::end(slot, st);
  return e;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static int row_bits_for(int64_t rows) {
  int b = 1;
  while ((int64_t(1) << b) < rows) ++b;
  return b;
}

static lora_status_t check_adapters(const lora_adapters_t *ad, int64_t rows_cap) {
  if (ad == nullptr || ad->ranks == nullptr) return LORA_ERR_ARG;
  if (ad->n_adapters < 1) return LORA_ERR_ARG;
  if (ad->max_rank < 1 || ad->max_rank > kMaxRank) return LORA_ERR_RANK;
  const int rb = row_bits_for(std::max<int64_t>(2, std::min<int64_t>(rows_cap, kPlanMaxRows)));
  if (((uint64_t)ad->n_adapters << rb) >= 0xFFFFFFFFull) return LORA_ERR_SHAPE;
  if (ad->kind == LORA_ADAPTERS_SLOTS) {
    if (ad->A == nullptr || ad->B == nullptr) return LORA_ERR_ARG;
    if (!aligned16(ad->A) || !aligned16(ad->B)) return LORA_ERR_SHAPE;
  } else if (ad->kind == LORA_ADAPTERS_POOL) {
    if (ad->pool == nullptr || ad->page_table == nullptr) return LORA_ERR_ARG;
    if (!aligned16(ad->pool)) return LORA_ERR_SHAPE;
    const int64_t P = ad->page_bytes;
    if (P < 256 || (P & (P - 1)) != 0 || P > (int64_t(1) << 40)) return LORA_ERR_PAGE;
    if (ad->n_pages < 1 || ad->max_pages < 1) return LORA_ERR_PAGE;
    if (ad->n_pages > (int64_t(1) << 31)) return LORA_ERR_PAGE;
  } else {
    return LORA_ERR_ARG;
  }
  return LORA_OK;
}

static AdapterRef make_ref(const lora_adapters_t *ad, int64_t k, int64_t d, int32_t eb) {
  AdapterRef r{};
  r.A = (const uint8_t *)ad->A;
  r.B = (const uint8_t *)ad->B;
  r.pool = (const uint8_t *)ad->pool;
  r.page_table = ad->page_table;
  r.page_bytes = ad->page_bytes;
  int sh = 0;
  if (ad->kind == LORA_ADAPTERS_POOL)
    while ((int64_t(1) << sh) < ad->page_bytes) ++sh;
  r.page_shift = sh;
  r.max_pages = ad->max_pages;
  r.max_rank = ad->max_rank;
  r.pooled = ad->kind == LORA_ADAPTERS_POOL;
  r.k = k;
  r.d = d;
  r.elem_bytes = eb;
  return r;
}

static lora_status_t check_gemm_args(lora_dtype_t dt, int64_t M, int64_t k, int64_t d,
                                     const void *x, int64_t ldx, const void *W, int64_t ldw,
                                     const void *y, int64_t ldy) {
  if (dt != LORA_DTYPE_F32 && dt != LORA_DTYPE_BF16) return LORA_ERR_DTYPE;
  if (M < 0 || k < 1 || d < 1) return LORA_ERR_SHAPE;
  if (M > INT32_MAX || k > INT32_MAX || d > INT32_MAX) return LORA_ERR_SHAPE;
  if (M == 0) return LORA_OK;
  if (x == nullptr || W == nullptr || y == nullptr) return LORA_ERR_ARG;
  if (ldx < k || ldw < k || ldy < d) return LORA_ERR_SHAPE;
  const int64_t vec = dt == LORA_DTYPE_BF16 ? 8 : 4;
  if (k % vec || ldx % vec || ldw % vec) return LORA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(W)) return LORA_ERR_SHAPE;
  return LORA_OK;
}

}  // namespace lora

using namespace lora;

extern "C" {

int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

const char *lora_status_str(lora_status_t s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_ERR_ARG: return "invalid argument";
    case LORA_ERR_SHAPE: return "unsupported shape, leading dimension or alignment";
    case LORA_ERR_DTYPE: return "unsupported dtype";
    case LORA_ERR_RANK: return "max_rank out of range (1..256)";
    case LORA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case LORA_ERR_PAGE: return "invalid pool geometry";
    case LORA_ERR_HIP: return "HIP runtime error";
    case LORA_ERR_UNSUPPORTED: return "not implemented in this build";
  }
  return "unknown status";
}

size_t lora_workspace_bytes(int64_t max_rows, int64_t d, int64_t k, lora_dtype_t dtype,
                            const lora_adapters_t *adapters) {
  if (max_rows < 0 || d < 1 || k < 1) return 0;
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return 0;
  if (check_adapters(adapters, max_rows) != LORA_OK) return 0;
  const int64_t rows = std::min<int64_t>(std::max<int64_t>(max_rows, 1), kPlanMaxRows);
  return ws_layout(rows, adapters->n_adapters, adapters->max_rank).total;
}

lora_status_t lora_gemm(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                        int64_t ldx, const void *W, int64_t ldw, void *y, int64_t ldy,
                        void *stream) {
  lora_status_t s = check_gemm_args(dtype, M, k, d, x, ldx, W, ldw, y, ldy);
  if (s != LORA_OK || M == 0) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(LORA_K_GEMM, st, [&] {
    return launch_gemm(dtype, M, k, d, x, ldx, W, ldw, y, ldy, st);
  });
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

static lora_status_t run_plan(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype,
                              const lora_adapters_t *ad, const int32_t *ids, uint8_t *ws,
                              const WsLayout &L, hipStream_t st) {
  PlanArgs p{};
  p.ids = ids;
  p.ranks = ad->ranks;
  p.M = (int32_t)M;
  p.S = ad->n_adapters;
  p.R = ad->max_rank;
  p.row_bits = row_bits_for(std::max<int64_t>(M, 2));
  if (ad->kind == LORA_ADAPTERS_POOL) {
    p.page_table = ad->page_table;
    p.max_pages = ad->max_pages;
    p.n_pages = ad->n_pages;
    p.page_bytes = ad->page_bytes;
    p.bytes_per_rank = (k + d) * (dtype == LORA_DTYPE_BF16 ? 2 : 4);
  }
  p.ws = ws;
  p.L = L;
  hipError_t e = timed(LORA_K_PLAN, st, [&] { return launch_plan(p, st); });
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status_t lora_plan(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype,
                        const lora_adapters_t *adapters, const int32_t *adapter_ids,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return LORA_ERR_DTYPE;
  if (M < 0 || M > kPlanMaxRows || k < 1 || d < 1) return LORA_ERR_SHAPE;
  lora_status_t s = check_adapters(adapters, M);
  if (s != LORA_OK) return s;
  if (workspace == nullptr || (M > 0 && adapter_ids == nullptr)) return LORA_ERR_ARG;
  if (((uintptr_t)workspace & 255u) != 0) return LORA_ERR_WORKSPACE;
  const WsLayout L = ws_layout(std::max<int64_t>(M, 1), adapters->n_adapters, adapters->max_rank);
  if (workspace_bytes < L.total) return LORA_ERR_WORKSPACE;
  // M == 0 runs too: the kernel then writes an empty plan (zero counts).
  return run_plan(M, k, d, dtype, adapters, adapter_ids, (uint8_t *)workspace, L, (hipStream_t)stream);
}

lora_status_t lora_plan_view(const void *workspace, size_t workspace_bytes, int64_t M,
                             const lora_adapters_t *adapters, lora_plan_view_t *out) {
  if (workspace == nullptr || out == nullptr) return LORA_ERR_ARG;
  if (M < 0 || M > kPlanMaxRows) return LORA_ERR_SHAPE;
  lora_status_t s = check_adapters(adapters, M);
  if (s != LORA_OK) return s;
  const WsLayout L = ws_layout(std::max<int64_t>(M, 1), adapters->n_adapters, adapters->max_rank);
  if (workspace_bytes < L.total) return LORA_ERR_WORKSPACE;
  const uint8_t *w = (const uint8_t *)workspace;
  out->counters = (const int32_t *)(w + L.hdr);
  out->perm = (const int32_t *)(w + L.perm);
  out->seg_adapter = (const int32_t *)(w + L.seg_adapter);
  out->seg_start = (const int32_t *)(w + L.seg_start);
  out->seg_len = (const int32_t *)(w + L.seg_len);
  out->capacity_rows = L.rows;
  return LORA_OK;
}

lora_status_t lora_linear(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                          int64_t ldx, const void *W, int64_t ldw,
                          const lora_adapters_t *adapters, const int32_t *adapter_ids,
                          const float *scales, void *y, int64_t ldy, void *workspace,
                          size_t workspace_bytes, int32_t path, uint32_t flags, void *stream) {
  lora_status_t s = check_gemm_args(dtype, M, k, d, x, ldx, W, ldw, y, ldy);
  if (s != LORA_OK) return s;
  if (path != LORA_PATH_AUTO && path != LORA_PATH_GATHER && path != LORA_PATH_SGMV) return LORA_ERR_ARG;
  if ((flags & ~LORA_FLAG_REUSE_PLAN) != 0) return LORA_ERR_ARG;
  s = check_adapters(adapters, M);
  if (s != LORA_OK) return s;
  if (M == 0) return LORA_OK;
  if (adapter_ids == nullptr || scales == nullptr || workspace == nullptr) return LORA_ERR_ARG;
  if (((uintptr_t)workspace & 255u) != 0) return LORA_ERR_WORKSPACE;
  if ((flags & LORA_FLAG_REUSE_PLAN) && M > kPlanMaxRows) return LORA_ERR_ARG;
  const int64_t first = std::min<int64_t>(M, kPlanMaxRows);
  if (workspace_bytes < ws_layout(first, adapters->n_adapters, adapters->max_rank).total)
    return LORA_ERR_WORKSPACE;
  if (path == LORA_PATH_SGMV) return LORA_ERR_UNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  const int32_t eb = dtype == LORA_DTYPE_BF16 ? 2 : 4;
  const AdapterRef ar = make_ref(adapters, k, d, eb);
  uint8_t *ws = (uint8_t *)workspace;

  for (int64_t c0 = 0; c0 < M; c0 += kPlanMaxRows) {
    const int64_t Mc = std::min<int64_t>(kPlanMaxRows, M - c0);
    const WsLayout L = ws_layout(Mc, adapters->n_adapters, adapters->max_rank);
    const uint8_t *xc = (const uint8_t *)x + c0 * ldx * eb;
    uint8_t *yc = (uint8_t *)y + c0 * ldy * eb;
    if (!(flags & LORA_FLAG_REUSE_PLAN)) {
      s = run_plan(Mc, k, d, dtype, adapters, adapter_ids + c0, ws, L, st);
      if (s != LORA_OK) return s;
    }
    hipError_t e = timed(LORA_K_GEMM, st, [&] {
      return launch_gemm(dtype, Mc, k, d, xc, ldx, W, ldw, yc, ldy, st);
    });
    if (e != hipSuccess) return LORA_ERR_HIP;

    LoraArgs a{};
    a.dtype = dtype;
    a.k = k;
    a.d = d;
    a.x = xc;
    a.ldx = ldx;
    a.y = yc;
    a.ldy = ldy;
    a.scales = scales;
    a.ar = ar;
    a.ws = ws;
    a.L = L;
    // k splits: aim for ~1024 shrink workgroups on the 256 CUs.
    const int64_t est_items = (Mc + kRowsPerGatherItem - 1) / kRowsPerGatherItem +
                              std::min<int64_t>({(int64_t)adapters->n_adapters, Mc, 64});
    int64_t ks = std::max<int64_t>(1, std::min<int64_t>(kMaxKSplit, (1024 + est_items - 1) / est_items));
    int64_t kchunk = (k + ks - 1) / ks;
    kchunk = (kchunk + 255) / 256 * 256;
    ks = (k + kchunk - 1) / kchunk;
    a.ksplit = (int32_t)ks;
    a.kchunk = kchunk;
    e = timed(LORA_K_SHRINK, st, [&] { return launch_shrink_gather(a, st); });
    if (e != hipSuccess) return LORA_ERR_HIP;
    e = timed(LORA_K_EXPAND, st, [&] { return launch_expand_gather(a, st); });
    if (e != hipSuccess) return LORA_ERR_HIP;
  }
  return LORA_OK;
}

lora_status_t lora_translate(const lora_adapters_t *adapters, const int32_t *adapter,
                             const int64_t *logical_off, int64_t n, int64_t *phys_off,
                             void *stream) {
  lora_status_t s = check_adapters(adapters, 1);
  if (s != LORA_OK) return s;
  if (adapters->kind != LORA_ADAPTERS_POOL) return LORA_ERR_ARG;
  if (n < 0) return LORA_ERR_SHAPE;
  if (n == 0) return LORA_OK;
  if (adapter == nullptr || logical_off == nullptr || phys_off == nullptr) return LORA_ERR_ARG;
  const AdapterRef ar = make_ref(adapters, 0, 0, 1);
  hipError_t e = launch_translate(ar, adapters->n_adapters, adapters->n_pages, adapter,
                                  logical_off, n, phys_off, (hipStream_t)stream);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status_t lora_check(const void *workspace, void *stream, int64_t *n_bad_ids,
                         int64_t *n_bad_ranks, int64_t *n_bad_pages) {
  if (workspace == nullptr) return LORA_ERR_ARG;
  int32_t h[3] = {0, 0, 0};
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(h, workspace, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess)
    return LORA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LORA_ERR_HIP;
  if (n_bad_ids) *n_bad_ids = h[kHdrBadIds];
  if (n_bad_ranks) *n_bad_ranks = h[kHdrBadRanks];
  if (n_bad_pages) *n_bad_pages = h[kHdrBadPages];
  return LORA_OK;
}

lora_status_t lora_profile_enable(int32_t on) {
  prof::enabled.store(on ? 1 : 0);
  return LORA_OK;
}

lora_status_t lora_profile_read(lora_profile_t *out, int32_t reset) {
  std::lock_guard<std::mutex> g(prof::mu);
  for (int i = 0; i < prof::used; ++i) {
    if (hipEventSynchronize(prof::ev1[i]) != hipSuccess) return LORA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, prof::ev0[i], prof::ev1[i]) != hipSuccess) return LORA_ERR_HIP;
    prof::ms[prof::cls[i]] += ms;
    prof::launches[prof::cls[i]] += 1;
  }
  prof::used = 0;
  if (out) {
    for (int c = 0; c < LORA_K_COUNT; ++c) {
      out->ms[c] = prof::ms[c];
      out->launches[c] = prof::launches[c];
    }
    out->dropped = prof::dropped;
  }
  if (reset) {
    for (int c = 0; c < LORA_K_COUNT; ++c) {
      prof::ms[c] = 0.0;
      prof::launches[c] = 0;
    }
    prof::dropped = 0;
  }
  return LORA_OK;
}

}  // extern "C"
