// lora_api.cpp -- host side of the C ABI declared in include/lora_row.h:
// argument validation, workspace layout, step dispatch and the optional
// per-kernel event timer.  Every compute step runs in the HIP kernels; this
// file only checks arguments and launches them on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "lora_row.h"
#include "kernels.hpp"

namespace lora {

// MFMA shrink: one workgroup per slice (more parallelism) rather than one
// for all slices (x read once).

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int64_t rows, int32_t S, int32_t R, int32_t n_slices) {
  WsLayout L;
  L.rows = std::max<int64_t>(1, rows);
  L.R = (std::max<int32_t>(R, 1) + 3) & ~3;  // partial row width (float4 runs)
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
  L.items_gx = take((size_t)L.items_g_cap * sizeof(ItemRows));
  L.items_s = take((size_t)L.items_s_cap * sizeof(Item));
  L.tpart = take((size_t)kMaxKSplit * L.rows * n_slices * L.R * sizeof(float));
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
      // timing only: no system-scope fence (it would write back caches and
      // perturb the work being timed)
      if (hipEventCreateWithFlags(&ev0[i], hipEventDisableSystemFence) != hipSuccess ||
          hipEventCreateWithFlags(&ev1[i], hipEventDisableSystemFence) != hipSuccess) {
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

// ---------------------------------------------------------------------------
// Side stream for the plan: the plan depends only on the ids, the GEMM only
// on x and W, so the plan runs beside the GEMM and the caller's stream waits
// for it before the shrink.  One non-blocking stream (default priority) and
// a ring of events per device, created on first use and kept.  (Launching
// the GEMM unordered behind the plan on the caller's stream was measured not
// to overlap them.)
// ---------------------------------------------------------------------------
namespace side {
constexpr int kMaxDev = 64;
constexpr int kEvents = 16;
std::mutex mu;
struct Dev {
  bool tried = false, ok = false;
  hipStream_t s = nullptr;
  hipEvent_t ev[kEvents];
  int next = 0;
};
Dev devs[kMaxDev];

bool get(hipStream_t *s, hipEvent_t *fork, hipEvent_t *join) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDev) return false;
  std::lock_guard<std::mutex> g(mu);
  Dev &D = devs[d];
  if (!D.tried) {
    D.tried = true;
    if (hipStreamCreateWithFlags(&D.s, hipStreamNonBlocking) != hipSuccess) return false;
    for (int i = 0; i < kEvents; ++i)
      // device-scope release: the waiting stream is on the same device (a
      // system-scope release would write caches back on every record)
      if (hipEventCreateWithFlags(&D.ev[i], hipEventDisableTiming | hipEventReleaseToDevice) !=
          hipSuccess)
        return false;
    D.ok = true;
  }
  if (!D.ok) return false;
  *s = D.s;
  *fork = D.ev[D.next];
  *join = D.ev[D.next + 1];
  D.next = (D.next + 2) % kEvents;
  return true;
}
}  // namespace side


template <typename F>
static hipError_t timed(int c, hipStream_t st, F &&launch) {
  const int slot = prof::begin(c, st);
  const hipError_t e = launch();
  prof::end(slot, st);
  return e;
}
// timed() unless the call must not create the profiler's events
template <typename F>
static hipError_t maybe_timed(bool untimed, int c, hipStream_t st, F &&launch) {
  return untimed ? launch() : timed(c, st, launch);
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

// Quantized base weight: host checks and kernel arguments.
static lora_status_t check_qweight(const lora_qweight_t *W, int64_t k, int64_t d) {
  if (W == nullptr || W->q == nullptr || W->scales == nullptr) return LORA_ERR_ARG;
  if (W->format != LORA_W_INT8 && W->format != LORA_W_INT4) return LORA_ERR_DTYPE;
  if (!aligned16(W->q) || W->ldq % 16 != 0) return LORA_ERR_SHAPE;
  if (W->format == LORA_W_INT8 && W->ldq < k) return LORA_ERR_SHAPE;
  if (W->format == LORA_W_INT4) {
    if (W->ldq < k / 2) return LORA_ERR_SHAPE;
    if (W->group < 64 || W->group % 64 != 0 || k % W->group != 0) return LORA_ERR_SHAPE;
  }
  // byte offsets inside one tile's rows and scales stay below 2^32
  const int64_t ng = W->format == LORA_W_INT4 ? k / W->group : 1;
  if ((uint64_t)144 * W->ldq >= (1ull << 32) || (uint64_t)144 * ng * 4 >= (1ull << 32))
    return LORA_ERR_SHAPE;
  (void)d;
  return LORA_OK;
}

static lora_status_t check_q_gemm_args(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                                       const lora_qweight_t *W, const void *y, int64_t ldy) {
  if (M < 0 || k < 1 || d < 1) return LORA_ERR_SHAPE;
  if (M > INT32_MAX || k > INT32_MAX || d > INT32_MAX) return LORA_ERR_SHAPE;
  lora_status_t s = check_qweight(W, k, d);
  if (s != LORA_OK) return s;
  if (M == 0) return LORA_OK;
  if (x == nullptr || y == nullptr) return LORA_ERR_ARG;
  if (ldx < k || ldy < d) return LORA_ERR_SHAPE;
  if (k % 64 != 0 || ldx % 8 != 0 || !aligned16(x)) return LORA_ERR_SHAPE;
  if ((uint64_t)256 * ldx * 2 >= (1ull << 32)) return LORA_ERR_SHAPE;
  return LORA_OK;
}

static QGemmArgs make_q_args(const lora_qweight_t *W, int64_t M, int64_t k, int64_t d,
                             const void *x, int64_t ldx, void *y, int64_t ldy) {
  QGemmArgs a{};
  a.fmt = W->format == LORA_W_INT8 ? 1 : 2;
  a.M = (int)M;
  a.N = (int)d;
  a.K = (int)k;
  a.x = (const uint16_t *)x;
  a.ldx = ldx;
  a.q = (const uint8_t *)W->q;
  a.ldq = W->ldq;
  a.scales = W->scales;
  a.group = W->format == LORA_W_INT4 ? W->group : 64;
  a.ngroups = W->format == LORA_W_INT4 ? (int32_t)(k / W->group) : 1;
  a.y = (uint16_t *)y;
  a.ldy = ldy;
  a.vec_store = ((ldy % 8) == 0 && ((uintptr_t)y & 15) == 0) ? 1 : 0;
  return a;
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
    case LORA_ERR_UNSUPPORTED: return "not implemented by this library";
  }
  return "unknown status";
}

// Validate a slice list; fills S (common adapter count) and R (max rank).
static lora_status_t check_slices(int32_t n_slices, const lora_slice_t *slices, int64_t rows_cap,
                                  int32_t *S_out, int32_t *R_out, int64_t *d_total) {
  if (slices == nullptr || n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_ERR_ARG;
  int32_t R = 0;
  int64_t dt = 0;
  for (int q = 0; q < n_slices; ++q) {
    const lora_status_t s = check_adapters(&slices[q].adapters, rows_cap);
    if (s != LORA_OK) return s;
    if (slices[q].adapters.n_adapters != slices[0].adapters.n_adapters) return LORA_ERR_ARG;
    if (slices[q].d < 1 || slices[q].d > INT32_MAX) return LORA_ERR_SHAPE;
    R = std::max(R, slices[q].adapters.max_rank);
    dt += slices[q].d;
  }
  if (dt > INT32_MAX) return LORA_ERR_SHAPE;
  *S_out = slices[0].adapters.n_adapters;
  *R_out = R;
  *d_total = dt;
  return LORA_OK;
}

// The base GEMM's region follows the plan's regions of a chunk of Mc rows.
static size_t gemm_region_bytes(int64_t Mc, int64_t k, lora_dtype_t dtype, int64_t d_total) {
  return dtype == LORA_DTYPE_BF16 ? gemm_ws_bytes(Mc, k, d_total) : 0;
}

size_t lora_workspace_bytes_sliced(int64_t max_rows, int64_t k, lora_dtype_t dtype,
                                   int32_t n_slices, const lora_slice_t *slices) {
  if (max_rows < 0 || k < 1) return 0;
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return 0;
  int32_t S = 0, R = 0;
  int64_t dt = 0;
  if (check_slices(n_slices, slices, max_rows, &S, &R, &dt) != LORA_OK) return 0;
  const int64_t rows = std::min<int64_t>(std::max<int64_t>(max_rows, 1), kPlanMaxRows);
  // any batch of at most max_rows rows: chunks of up to `rows` rows, each
  // with its plan regions and the GEMM region of its row count
  size_t need = ws_layout(rows, S, R, n_slices).total + gemm_region_bytes(rows, k, dtype, dt);
  for (int64_t mc = 256; mc < rows; mc += 256)
    need = std::max(need, ws_layout(rows, S, R, n_slices).total + gemm_region_bytes(mc, k, dtype, dt));
  return need;
}

size_t lora_workspace_bytes(int64_t max_rows, int64_t d, int64_t k, lora_dtype_t dtype,
                            const lora_adapters_t *adapters) {
  if (adapters == nullptr) return 0;
  lora_slice_t s{};
  s.d = d;
  s.scales = nullptr;
  s.adapters = *adapters;
  return lora_workspace_bytes_sliced(max_rows, k, dtype, 1, &s);
}

size_t lora_gemm_workspace_bytes(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype) {
  if (M < 0 || k < 1 || d < 1) return 0;
  return gemm_region_bytes(M, k, dtype, d);
}

lora_status_t lora_gemm(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                        int64_t ldx, const void *W, int64_t ldw, void *y, int64_t ldy,
                        void *workspace, size_t workspace_bytes, void *stream) {
  lora_status_t s = check_gemm_args(dtype, M, k, d, x, ldx, W, ldw, y, ldy);
  if (s != LORA_OK || M == 0) return s;
  if (workspace != nullptr && ((uintptr_t)workspace & 255u) != 0) return LORA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(LORA_K_GEMM, st, [&] {
    return launch_gemm(dtype, M, k, d, x, ldx, W, ldw, y, ldy,
                       workspace_bytes > 0 ? workspace : nullptr, workspace_bytes, st);
  });
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status_t lora_gemm_q(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                          const lora_qweight_t *W, void *y, int64_t ldy, void *stream) {
  lora_status_t s = check_q_gemm_args(M, k, d, x, ldx, W, y, ldy);
  if (s != LORA_OK || M == 0) return s;
  hipStream_t st = (hipStream_t)stream;
  const QGemmArgs a = make_q_args(W, M, k, d, x, ldx, y, ldy);
  hipError_t e = timed(LORA_K_GEMM, st, [&] { return launch_gemm_q(a, st); });
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

static PlanArgs make_plan_args(int64_t M, int64_t k, lora_dtype_t dtype, int32_t n_slices,
                               const lora_slice_t *slices, const int32_t *ids, uint8_t *ws,
                               const WsLayout &L) {
  PlanArgs p{};
  p.ids = ids;
  p.M = (int32_t)M;
  p.S = slices[0].adapters.n_adapters;
  p.row_bits = row_bits_for(std::max<int64_t>(M, 2));
  p.n_slices = n_slices;
  const int64_t eb = dtype == LORA_DTYPE_BF16 ? 2 : 4;
  for (int q = 0; q < n_slices; ++q) {
    const lora_adapters_t &ad = slices[q].adapters;
    PlanSlice &ps = p.sl[q];
    ps.ranks = ad.ranks;
    ps.R = ad.max_rank;
    if (ad.kind == LORA_ADAPTERS_POOL) {
      ps.page_table = ad.page_table;
      ps.max_pages = ad.max_pages;
      ps.n_pages = ad.n_pages;
      ps.page_bytes = ad.page_bytes;
      ps.bytes_per_rank = (k + slices[q].d) * eb;
    }
  }
  p.ws = ws;
  p.L = L;
  return p;
}

static lora_status_t run_plan(int64_t M, int64_t k, lora_dtype_t dtype, int32_t n_slices,
                              const lora_slice_t *slices, const int32_t *ids, uint8_t *ws,
                              const WsLayout &L, hipStream_t st,
                              size_t max_lds = kPlanLdsBeside, bool untimed = false) {
  const PlanArgs p = make_plan_args(M, k, dtype, n_slices, slices, ids, ws, L);
  hipError_t e = maybe_timed(untimed, LORA_K_PLAN, st, [&] { return launch_plan(p, st, max_lds); });
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

static lora_status_t plan_common(int64_t M, int64_t k, lora_dtype_t dtype, int32_t n_slices,
                                 const lora_slice_t *slices, const int32_t *adapter_ids,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return LORA_ERR_DTYPE;
  if (M < 0 || M > kPlanMaxRows || k < 1) return LORA_ERR_SHAPE;
  int32_t S = 0, R = 0;
  int64_t dt = 0;
  lora_status_t s = check_slices(n_slices, slices, M, &S, &R, &dt);
  if (s != LORA_OK) return s;
  if (workspace == nullptr || (M > 0 && adapter_ids == nullptr)) return LORA_ERR_ARG;
  if (((uintptr_t)workspace & 255u) != 0) return LORA_ERR_WORKSPACE;
  const WsLayout L = ws_layout(std::max<int64_t>(M, 1), S, R, n_slices);
  if (workspace_bytes < L.total) return LORA_ERR_WORKSPACE;
  // M == 0 runs too: the kernel then writes an empty plan (zero counts).
  return run_plan(M, k, dtype, n_slices, slices, adapter_ids, (uint8_t *)workspace, L,
                  (hipStream_t)stream);
}

lora_status_t lora_plan(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype,
                        const lora_adapters_t *adapters, const int32_t *adapter_ids,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (adapters == nullptr) return LORA_ERR_ARG;
  lora_slice_t sl{};
  sl.d = d;
  sl.adapters = *adapters;
  if (d < 1) return LORA_ERR_SHAPE;
  return plan_common(M, k, dtype, 1, &sl, adapter_ids, workspace, workspace_bytes, stream);
}

lora_status_t lora_plan_view(const void *workspace, size_t workspace_bytes, int64_t M,
                             const lora_adapters_t *adapters, lora_plan_view_t *out) {
  if (workspace == nullptr || out == nullptr) return LORA_ERR_ARG;
  if (M < 0 || M > kPlanMaxRows) return LORA_ERR_SHAPE;
  lora_status_t s = check_adapters(adapters, M);
  if (s != LORA_OK) return s;
  const WsLayout L = ws_layout(std::max<int64_t>(M, 1), adapters->n_adapters, adapters->max_rank, 1);
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

}  // extern "C"

namespace lora {
// The layer over several slices; the base weight is dense (W, ldw) or, with
// qw != nullptr, quantized (bf16 only).  self_contained: use no library
// resource that may need creating -- the plan runs on the caller's stream
// (no side stream or fork/join events) and no launch is timed.
lora_status_t linear_sliced_impl(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                 int64_t ldx, const void *W, int64_t ldw, const lora_qweight_t *qw,
                                 int32_t n_slices, const lora_slice_t *slices,
                                 const int32_t *adapter_ids, void *y, int64_t ldy, void *workspace,
                                 size_t workspace_bytes, int32_t path, uint32_t flags, void *stream,
                                 bool self_contained) {
  int32_t S = 0, R = 0;
  int64_t d_total = 0;
  if (slices == nullptr || n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_ERR_ARG;
  lora_status_t s = check_slices(n_slices, slices, M, &S, &R, &d_total);
  if (s != LORA_OK) return s;
  s = qw ? check_q_gemm_args(M, k, d_total, x, ldx, qw, y, ldy)
         : check_gemm_args(dtype, M, k, d_total, x, ldx, W, ldw, y, ldy);
  if (s != LORA_OK) return s;
  if (path != LORA_PATH_AUTO && path != LORA_PATH_GATHER && path != LORA_PATH_SGMV) return LORA_ERR_ARG;
  if ((flags & ~(LORA_FLAG_REUSE_PLAN | LORA_FLAG_SEPARATE_SHRINK)) != 0) return LORA_ERR_ARG;
  if (M == 0) return LORA_OK;
  if (adapter_ids == nullptr || workspace == nullptr) return LORA_ERR_ARG;
  for (int q = 0; q < n_slices; ++q)
    if (slices[q].scales == nullptr) return LORA_ERR_ARG;
  if (((uintptr_t)workspace & 255u) != 0) return LORA_ERR_WORKSPACE;
  if ((flags & LORA_FLAG_REUSE_PLAN) && M > kPlanMaxRows) return LORA_ERR_ARG;
  const int64_t first = std::min<int64_t>(M, kPlanMaxRows);
  if (workspace_bytes < ws_layout(first, S, R, n_slices).total) return LORA_ERR_WORKSPACE;

  // kernel family: MFMA tiles need bf16 operands and ranks <= 64
  const bool mfma_ok = dtype == LORA_DTYPE_BF16 && R <= kMaxRankMfma;
  bool use_mfma;
  if (path == LORA_PATH_SGMV) {
    if (!mfma_ok) return LORA_ERR_UNSUPPORTED;
    use_mfma = true;
  } else if (path == LORA_PATH_GATHER) {
    use_mfma = false;
  } else {
    use_mfma = mfma_ok;
  }

  hipStream_t st = (hipStream_t)stream;
  const int32_t eb = dtype == LORA_DTYPE_BF16 ? 2 : 4;
  uint8_t *ws = (uint8_t *)workspace;

  LoraArgs a{};
  a.dtype = dtype;
  a.k = k;
  a.ldx = ldx;
  a.ldy = ldy;
  a.y_vec = ((uintptr_t)y % 16 == 0 && (ldy * eb) % 16 == 0) ? 1 : 0;
  a.n_slices = n_slices;
  a.R = R;
  a.ws = ws;
  int64_t col0 = 0;
  for (int q = 0; q < n_slices; ++q) {
    SliceRef &sr = a.sl[q];
    sr.ar = make_ref(&slices[q].adapters, k, slices[q].d, eb);
    sr.ranks = slices[q].adapters.ranks;
    sr.scales = slices[q].scales;
    sr.d = slices[q].d;
    sr.col0 = col0;
    col0 += slices[q].d;
  }

  for (int64_t c0 = 0; c0 < M; c0 += kPlanMaxRows) {
    const int64_t Mc = std::min<int64_t>(kPlanMaxRows, M - c0);
    const WsLayout L = ws_layout(Mc, S, R, n_slices);
    // the GEMM's region: what the workspace holds past this chunk's plan
    // regions (a workspace sized by lora_workspace_bytes(_sliced) holds
    // what every chunk's GEMM uses)
    void *gws = workspace_bytes > L.total ? (void *)(ws + L.total) : nullptr;
    const size_t gws_bytes = workspace_bytes > L.total ? workspace_bytes - L.total : 0;
    const uint8_t *xc = (const uint8_t *)x + c0 * ldx * eb;
    uint8_t *yc = (uint8_t *)y + c0 * ldy * eb;

    a.x = xc;
    a.y = yc;
    a.L = L;
    // rows per MFMA work item: 64-row segment tiles when asked for (SGMV)
    // or when adapters are expected to hold long runs of rows (prefill);
    // else 16, which gives decode batches more workgroups
    const int64_t segs = std::min<int64_t>((int64_t)S, Mc);
    const int rpi = (use_mfma && (path == LORA_PATH_SGMV ||
                            Mc / std::max<int64_t>(segs, 1) >= 128))
                  ? kRowsPerSgmvItem
                  : kRowsPerGatherItem;

    // k splits: aim for ~600 shrink workgroups on the 256 CUs (measured
    // best for decode batches: more splits add partials for the expand to
    // sum, fewer leave CUs idle).  The MFMA shrink covers all slices in one
    // workgroup; the gather shrink takes one per slice and 16-rank block.
    const int64_t est_items = (Mc + rpi - 1) / rpi + std::min<int64_t>(segs, 64);
    const int64_t jblk = (R + 15) / 16;
    // one workgroup for every slice's rank blocks (x rows read once for all
    // projections) where the LDS-staged shrink holds them all, else one per
    // slice (more workgroups)
    const bool per_slice = !(use_mfma && n_slices > 1 && shrink_dma_rows(a, false) > 0);
    const int64_t per_split = std::max<int64_t>(
        1, use_mfma ? est_items * (per_slice ? n_slices : 1)
                    : est_items * n_slices * std::min<int64_t>(jblk, 2));
    int64_t ks = std::max<int64_t>(1, std::min<int64_t>(kMaxKSplit, (600 + per_split - 1) / per_split));
    int64_t kchunk = (k + ks - 1) / ks;
    kchunk = (kchunk + 255) / 256 * 256;
    ks = (k + kchunk - 1) / kchunk;
    a.ksplit = (int32_t)ks;
    a.kchunk = kchunk;

    // Folded shrink: the base GEMM carries the stacked A rows (slots only:
    // each A row is one contiguous run) when its tile shape has room for
    // every rank in at most two passes (the second is a fallback for rank
    // sums past the first pass's capacity).
    int32_t fcap = 0;
    if (!qw && dtype == LORA_DTYPE_BF16 && use_mfma && !(flags & LORA_FLAG_SEPARATE_SHRINK) &&
        (int64_t)n_slices * S <= kFusedMaxEntries && S <= 256) {
      // slots, or pools whose pages hold whole A rows (each row one
      // contiguous run the GEMM's loads can take)
      bool rows_ok = true;
      int64_t worst = 0;
      for (int q = 0; q < n_slices; ++q) {
        const lora_adapters_t &ad = slices[q].adapters;
        rows_ok = rows_ok && (ad.kind == LORA_ADAPTERS_SLOTS
                                  ? ((uintptr_t)ad.A & 15u) == 0
                                  : ad.page_bytes % (2 * k) == 0);
        worst += (int64_t)S * ad.max_rank;
      }
      const int32_t cap = rows_ok ? gemm_fused_cap(Mc, k, d_total, ldx, ldw) : 0;
      if (cap > 0 && worst <= 2 * (int64_t)cap) fcap = cap;
    }
    a.fused_cap = fcap;
    FusedT ft{};
    if (fcap > 0) {
      ft.cap = fcap;
      ft.n_slices = n_slices;
      ft.S = S;
      for (int q = 0; q < n_slices; ++q) {
        const lora_adapters_t &ad = slices[q].adapters;
        const bool pooled = ad.kind == LORA_ADAPTERS_POOL;
        ft.A[q] = (const uint8_t *)(pooled ? ad.pool : ad.A);
        ft.R[q] = ad.max_rank;
        ft.ranks[q] = ad.ranks;
        ft.page_table[q] = pooled ? ad.page_table : nullptr;
        ft.max_pages[q] = pooled ? ad.max_pages : 0;
        int sh = 0;
        while (pooled && (int64_t(1) << sh) < ad.page_bytes) ++sh;
        ft.page_shift[q] = sh;
        ft.n_pages[q] = pooled ? ad.n_pages : 0;
      }
      ft.ids = adapter_ids + c0;
      ft.tpart = (float *)(ws + L.tpart);
      ft.rows = L.rows;
      ft.Rw = L.R;
    }
    // The plan needs only the ids, the GEMM only x and W: with a side
    // stream the plan runs beside the GEMM and the caller's stream waits
    // for it before the shrink.  (A shrink on the side stream as well gets
    // only the GEMM's leftover CU resources and finishes later than after
    // it.)  Later calls on the caller's stream are ordered after this call
    // by the fork event, so the workspace is never rewritten while read.
    // The plan runs beside the GEMM only where one of its workgroups fits on a
    // CU next to one of the GEMM's (registers and LDS); otherwise it would
    // wait for GEMM workgroups to finish and then hold up the shrink, so it
    // runs on the caller's stream ahead of the GEMM.
    hipStream_t ps = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    const bool reuse = (flags & LORA_FLAG_REUSE_PLAN) != 0;
    // Where the base GEMM launch can carry the plan, it does (no plan
    // launch, side stream or events: the fork and join cost ~6.5 us each on
    // the stream at the 70B q+v step)
    const bool in_gemm = !reuse && !qw &&
                         gemm_runs_plan(dtype, Mc, k, d_total, ldx, ldw, gws, gws_bytes, fcap > 0);
    PlanArgs gplan{};
    if (in_gemm) gplan = make_plan_args(Mc, k, dtype, n_slices, slices, adapter_ids + c0, ws, L);
    bool beside = !self_contained && !in_gemm;
    if (!reuse && !qw && beside) {
      KernelFootprint pf, gf;
      const PlanArgs pa = make_plan_args(Mc, k, dtype, n_slices, slices, adapter_ids + c0, ws, L);
      beside = plan_footprint(pa, &pf) &&
               gemm_footprint(dtype, Mc, k, d_total, ldx, ldw, gws, gws_bytes, fcap > 0, &gf) &&
               fits_beside(gf, pf);
    }
    const bool fork = !reuse && beside && !self_contained && side::get(&ps, &ev_fork, &ev_join);
    if (!reuse && !in_gemm) {
      if (fork) {
        if (hipEventRecord(ev_fork, st) != hipSuccess || hipStreamWaitEvent(ps, ev_fork, 0) != hipSuccess)
          return LORA_ERR_HIP;
      }
      s = run_plan(Mc, k, dtype, n_slices, slices, adapter_ids + c0, ws, L, fork ? ps : st,
                   fork || beside ? kPlanLdsBeside : kPlanLdsAlone, self_contained);
      if (s != LORA_OK) return s;
      if (fork && hipEventRecord(ev_join, ps) != hipSuccess) return LORA_ERR_HIP;
    }
    hipError_t e = maybe_timed(self_contained, LORA_K_GEMM, st, [&] {
      if (qw) return launch_gemm_q(make_q_args(qw, Mc, k, d_total, xc, ldx, yc, ldy), st);
      // expired split-K waits are counted in the plan header, where
      // lora_check reads them
      int32_t *expired = reinterpret_cast<int32_t *>(ws + L.hdr) + kHdrSyncExpired;
      const PlanArgs *pp = in_gemm ? &gplan : nullptr;
      if (fcap > 0)
        return launch_gemm_fused(Mc, k, d_total, xc, ldx, W, ldw, yc, ldy, ft, gws, gws_bytes, st,
                                 expired, pp);
      return launch_gemm(dtype, Mc, k, d_total, xc, ldx, W, ldw, yc, ldy, gws, gws_bytes, st,
                         expired, pp);
    });
    if (e != hipSuccess) return LORA_ERR_HIP;
    if (fork && hipStreamWaitEvent(st, ev_join, 0) != hipSuccess) return LORA_ERR_HIP;

    if (use_mfma) {
      if (fcap == 0) {  // else the base GEMM computed t
        e = maybe_timed(self_contained, LORA_K_SGMV_SHRINK, st, [&] { return launch_shrink_sgmv(a, rpi, per_slice, st); });
        if (e != hipSuccess) return LORA_ERR_HIP;
      }
      e = maybe_timed(self_contained, LORA_K_SGMV_EXPAND, st, [&] { return launch_expand_sgmv(a, rpi, st); });
      if (e != hipSuccess) return LORA_ERR_HIP;
    } else {
      e = maybe_timed(self_contained, LORA_K_SHRINK, st, [&] { return launch_shrink_gather(a, st); });
      if (e != hipSuccess) return LORA_ERR_HIP;
      e = maybe_timed(self_contained, LORA_K_EXPAND, st, [&] { return launch_expand_gather(a, st); });
      if (e != hipSuccess) return LORA_ERR_HIP;
    }
  }
  return LORA_OK;
}

}  // namespace lora

extern "C" {

lora_status_t lora_linear_sliced(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                 int64_t ldx, const void *W, int64_t ldw, int32_t n_slices,
                                 const lora_slice_t *slices, const int32_t *adapter_ids, void *y,
                                 int64_t ldy, void *workspace, size_t workspace_bytes,
                                 int32_t path, uint32_t flags, void *stream) {
  return linear_sliced_impl(dtype, M, k, x, ldx, W, ldw, nullptr, n_slices, slices, adapter_ids,
                            y, ldy, workspace, workspace_bytes, path, flags, stream, false);
}

lora_status_t lora_linear_sliced_q(int64_t M, int64_t k, const void *x, int64_t ldx,
                                   const lora_qweight_t *W, int32_t n_slices,
                                   const lora_slice_t *slices, const int32_t *adapter_ids, void *y,
                                   int64_t ldy, void *workspace, size_t workspace_bytes,
                                   int32_t path, uint32_t flags, void *stream) {
  if (W == nullptr) return LORA_ERR_ARG;
  return linear_sliced_impl(LORA_DTYPE_BF16, M, k, x, ldx, nullptr, 0, W, n_slices, slices,
                            adapter_ids, y, ldy, workspace, workspace_bytes, path, flags, stream,
                            false);
}

lora_status_t lora_linear(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                          int64_t ldx, const void *W, int64_t ldw,
                          const lora_adapters_t *adapters, const int32_t *adapter_ids,
                          const float *scales, void *y, int64_t ldy, void *workspace,
                          size_t workspace_bytes, int32_t path, uint32_t flags, void *stream) {
  if (adapters == nullptr) return LORA_ERR_ARG;
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return LORA_ERR_DTYPE;
  if (d < 1) return LORA_ERR_SHAPE;
  lora_slice_t sl{};
  sl.d = d;
  sl.scales = scales;
  sl.adapters = *adapters;
  if (M > 0 && scales == nullptr) return LORA_ERR_ARG;
  return lora_linear_sliced(dtype, M, k, x, ldx, W, ldw, 1, &sl, adapter_ids, y, ldy, workspace,
                            workspace_bytes, path, flags, stream);
}

lora_status_t lora_merge(lora_dtype_t dtype, int64_t d, int64_t k, const void *W, int64_t ldw,
                         const lora_adapters_t *adapters, int32_t adapter, const float *scales,
                         float coef, void *W_out, int64_t ldo, void *stream) {
  if (dtype != LORA_DTYPE_F32 && dtype != LORA_DTYPE_BF16) return LORA_ERR_DTYPE;
  if (d < 1 || k < 1 || d > INT32_MAX || k > INT32_MAX) return LORA_ERR_SHAPE;
  if (W == nullptr || W_out == nullptr || scales == nullptr) return LORA_ERR_ARG;
  lora_status_t s = check_adapters(adapters, 1);
  if (s != LORA_OK) return s;
  if (adapter < 0 || adapter >= adapters->n_adapters) return LORA_ERR_ARG;
  if (ldw < k || ldo < k) return LORA_ERR_SHAPE;
  const int64_t vec = dtype == LORA_DTYPE_BF16 ? 8 : 4;
  if (k % vec || ldw % vec || ldo % vec || !aligned16(W) || !aligned16(W_out)) return LORA_ERR_SHAPE;
  // in place is allowed; any other overlap is not
  const int64_t eb = dtype == LORA_DTYPE_BF16 ? 2 : 4;
  const uint8_t *wb = (const uint8_t *)W, *ob = (const uint8_t *)W_out;
  const int64_t wspan = ((d - 1) * ldw + k) * eb, ospan = ((d - 1) * ldo + k) * eb;
  if (wb != ob && wb < ob + ospan && ob < wb + wspan) return LORA_ERR_ARG;
  if (wb == ob && ldw != ldo) return LORA_ERR_ARG;
  MergeArgs m{};
  m.dtype = dtype == LORA_DTYPE_BF16 ? 1 : 0;
  m.d = d;
  m.k = k;
  m.W = wb;
  m.ldw = ldw;
  m.Wo = (uint8_t *)W_out;
  m.ldo = ldo;
  m.ar = make_ref(adapters, k, d, (int32_t)eb);
  m.ranks = adapters->ranks;
  m.scales = scales;
  m.adapter = adapter;
  m.coef = coef;
  m.rp = (adapters->max_rank + 31) & ~31;
  m.n_pages = adapters->n_pages;
  return launch_merge(m, (hipStream_t)stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
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
                         int64_t *n_bad_ranks, int64_t *n_bad_pages, int64_t *n_sync_expired) {
  if (workspace == nullptr) return LORA_ERR_ARG;
  int32_t h[kHdrSyncExpired + 1] = {};
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(h, workspace, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess)
    return LORA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LORA_ERR_HIP;
  if (n_bad_ids) *n_bad_ids = h[kHdrBadIds];
  if (n_bad_ranks) *n_bad_ranks = h[kHdrBadRanks];
  if (n_bad_pages) *n_bad_pages = h[kHdrBadPages];
  if (n_sync_expired) *n_sync_expired = h[kHdrSyncExpired];
  return LORA_OK;
}

lora_status_t lora_test_sync_spin_limit(int32_t polls) {
  set_sync_spin_limit(polls);
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
