// plan_body.hpp -- the plan step as a device function, run either by its
// own kernel or by a workgroup of the base GEMM's launch.
//
// Plan ("Adapter Residency When One Replica Serves Many Fine-Tunes", section
// "Batch composition under many adapters": sort a batch's rows by adapter
// before the forward pass so every adapter's rows are contiguous; "S-LoRA:
// what the paper actually says ...", section "Batched LoRA computation": the
// corrections run as one segmented operation over the adapter-sorted rows).
//
// One workgroup does the whole plan for up to 8192 rows:
//   1. classify each row (none / adapted / bad id / bad rank / bad page) --
//      where a table of the adapters fits in LDS, each adapter's ranks and
//      pages are checked once and the rows' ids (16-byte loads) are looked
//      up in it;
//   2. order the adapted rows by (adapter, row) -- a stable counting sort
//      over the adapters where LDS holds a histogram per wave, else a
//      bitonic sort of the keys (adapter << row_bits) | row;
//   3. write perm, the segment table and the gather / SGMV work-item lists
//      (segments cut into row blocks).
// The (adapter, row) order is unique, so both sorts give the same result.
// Integer atomics only (exact counts); nothing depends on thread timing.
#pragma once

#include "kernels.hpp"

namespace lora {
namespace plan_detail {

constexpr uint32_t kSentinel = 0xFFFFFFFFu;

// Exclusive scan of one value per thread over an NT-thread block.
// `wsum` is LDS scratch of >= NT / 64 + 1 values; returns the exclusive
// prefix and writes the block total to *total (every thread sees it).
template <int NT, typename T = int>
__device__ __forceinline__ T block_exclusive_scan(T v, T *wsum, T *total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = (lane < NT / 64) ? wsum[lane] : T(0);
    T inc = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      T y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < NT / 64) wsum[lane] = inc - w;
    if (lane == NT / 64 - 1) wsum[NT / 64] = inc;
  }
  __syncthreads();
  *total = wsum[NT / 64];
  return x - v + wsum[wave];
}

// The fields of a slice the row checks read, staged in LDS once per plan
// (plan_stage_slices): the checks then read them from LDS, and the kernel
// arguments are read at fixed indexes only, by one thread -- few of them
// stay live in scalar registers through the plan.
struct PlanSliceL {
  const int32_t *ranks;
  const int32_t *page_table;  // nullptr: slots
  int64_t n_pages, page_bytes, bytes_per_rank;
  int32_t R, max_pages;
};
__device__ __forceinline__ void plan_stage_slices(const PlanArgs &a, PlanSliceL *sl) {
  if (threadIdx.x != 0) return;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q) {
    if (q >= a.n_slices) break;
    const PlanSlice &g = a.sl[q];
    sl[q] = PlanSliceL{g.ranks, g.page_table, g.n_pages, g.page_bytes, g.bytes_per_rank, g.R,
                       g.max_pages};
  }
}  // the caller's barrier publishes them

// The class of a row with adapter id `id` whose rank in slice q is rk[q]:
// the adapter if the row is adapted, else -1 (no adapter), -2 (id outside
// [-1, S)), -3 (a slice's rank outside [0, R]) or -4 (a slice's pages
// outside its table or pool).
__device__ __forceinline__ int plan_class_id(const PlanArgs &a, const PlanSliceL *sls, int id,
                                             const int rk[kMaxSlices]) {
  if (id == -1) return -1;  // no adapter
  if (id < -1 || id >= a.S) return -2;
  // every slice's rank must be in range, then every slice's pages
  bool rank_ok = true, page_ok = true;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q) {
    if (q >= a.n_slices) break;
    const PlanSliceL &sl = sls[q];
    const int r = rk[q];
    if (r < 0 || r > sl.R) {
      rank_ok = false;
      continue;
    }
    if (sl.page_table != nullptr) {
      const int64_t bytes = (int64_t)r * sl.bytes_per_rank;
      const int64_t pages = (bytes + sl.page_bytes - 1) / sl.page_bytes;
      if (pages > sl.max_pages) page_ok = false;
      for (int64_t j = 0; page_ok && j < pages; ++j) {
        const int32_t pg = sl.page_table[(int64_t)id * sl.max_pages + j];
        if (pg < 0 || (int64_t)pg >= sl.n_pages) page_ok = false;
      }
    }
  }
  if (!rank_ok) return -3;
  if (!page_ok) return -4;
  return id;
}

// The ranks of adapter `id` (taken as adapter 0 outside [0, S)) in every
// slice.
__device__ __forceinline__ void plan_ranks_of(const PlanArgs &a, const PlanSliceL *sls, int id,
                                              int rk[kMaxSlices]) {
  const int idc = (id >= 0 && id < a.S) ? id : 0;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q) rk[q] = q < a.n_slices ? sls[q].ranks[idc] : 0;
}

// Row m's class (plan_class_id).  Without `sls` (the lean plan run inside a
// GEMM kernel whose registers are spoken for) the slices are walked with a
// loop over the arguments themselves, one slice's fields live at a time.
__device__ __forceinline__ int plan_class(const PlanArgs &a, const PlanSliceL *sls, int m) {
  const int id = a.ids[m];
  if (sls != nullptr) {
    int rk[kMaxSlices];
    plan_ranks_of(a, sls, id, rk);
    return plan_class_id(a, sls, id, rk);
  }
  if (id == -1) return -1;
  if (id < -1 || id >= a.S) return -2;
  bool rank_ok = true, page_ok = true;
  for (int q = 0; q < a.n_slices; ++q) {
    const PlanSlice &sl = a.sl[q];
    const int r = sl.ranks[id];
    if (r < 0 || r > sl.R) {
      rank_ok = false;
      continue;
    }
    if (sl.page_table != nullptr) {
      const int64_t pages = ((int64_t)r * sl.bytes_per_rank + sl.page_bytes - 1) / sl.page_bytes;
      if (pages > sl.max_pages) page_ok = false;
      for (int64_t j = 0; page_ok && j < pages; ++j) {
        const int32_t pg = sl.page_table[(int64_t)id * sl.max_pages + j];
        if (pg < 0 || (int64_t)pg >= sl.n_pages) page_ok = false;
      }
    }
  }
  return !rank_ok ? -3 : (!page_ok ? -4 : id);
}

// Row m's adapter if the row is adapted, else -1; a bad row is counted in
// cnt[0] bad id, cnt[1] bad rank or cnt[2] bad page (rare: counted per
// row); cnt[3] adapted rows is counted by the callers, per wave.  With
// `cls` the class is read from cls[m] (LDS, plan_classes), else found here.
__device__ __forceinline__ int plan_row(const PlanArgs &a, const PlanSliceL *sls, const int *cls,
                                        int m, int *cnt) {
  const int c = cls ? cls[m] : plan_class(a, sls, m);
  if (c < -1) {
    atomicAdd(&cnt[min(-2 - c, 2)], 1);
    return -1;
  }
  return c;
}

// Validity of every adapter into vt[0, S) (LDS bytes): 0 when each slice's
// rank of the adapter is in [0, R] and its pages lie in the table and the
// pool, 1 for a bad rank, 2 for a bad page, so a row's class follows from its
// id alone (plan_class_vt).  U adapters per thread at a time: their ranks in
// every slice are loaded before the first is waited for.
template <int NT, int U>
__device__ __forceinline__ void plan_validate(const PlanArgs &a, const PlanSliceL *sls, int8_t *vt) {
  for (int base = threadIdx.x; base < a.S; base += NT * U) {
    int rk[U][kMaxSlices];
#pragma unroll
    for (int u = 0; u < U; ++u) plan_ranks_of(a, sls, min(base + NT * u, a.S - 1), rk[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base + NT * u;
      if (s < a.S) {
        const int c = plan_class_id(a, sls, s, rk[u]);  // s, -3 or -4
        vt[s] = (int8_t)(c >= 0 ? 0 : -2 - c);
      }
    }
  }
}

// plan_class of a row with adapter id `id`, from the validity table.
__device__ __forceinline__ int plan_class_vt(int id, int S, const int8_t *vt) {
  if (id == -1) return -1;
  if (id < -1 || id >= S) return -2;
  const int v = vt[id];
  return v == 0 ? id : -2 - v;
}

// The classes of all M rows into cls[0, M) (LDS, int or int8_t entries;
// room for M rounded up to 4): the ids are read with 16-byte buffer loads
// (four per thread issued before the first is waited for; the buffer's bound
// turns reads past the last row into zeros, which are not stored), and the
// validity table vt (LDS, S bytes) is built while the first of them are in
// flight.  Ends with a barrier.
template <int NT, typename C>
__device__ __forceinline__ void plan_classes(const PlanArgs &a, const PlanSliceL *sls, int8_t *vt,
                                             C *cls) {
  constexpr int U = 4;
  const int M = a.M;
  const int n16 = (M + 3) / 4;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(a.ids), 0, M * 4, 0x00020000);
  u32x4_t v[U];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_bit_cast(u32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, (c0 + u * NT) * 16, 0, 0));
  };
  load(threadIdx.x);
  plan_validate<NT, 2>(a, sls, vt);
  __syncthreads();
  for (int c0 = threadIdx.x; c0 < n16; c0 += NT * U) {
    if (c0 != (int)threadIdx.x) load(c0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int m = 4 * (c0 + u * NT);
      if (m >= M) continue;
      int c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = m + e < M ? plan_class_vt((int)v[u][e], a.S, vt) : -1;
      if constexpr (sizeof(C) == 1) {
        *reinterpret_cast<uint32_t *>(cls + m) = (uint32_t)(c[0] & 0xff) | (uint32_t)(c[1] & 0xff) << 8 |
                                                 (uint32_t)(c[2] & 0xff) << 16 | (uint32_t)c[3] << 24;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (m + e < M) cls[m + e] = c[e];
      }
    }
  }
  __syncthreads();
}

// Bitonic plan.  `plan_lds` holds plan_sort_lds(row_bits) bytes: the sort
// keys [n2] then segment starts [n2] (uint16).
template <int NT>
__device__ __forceinline__ void plan_bitonic(const PlanArgs &a, const PlanSliceL *sls,
                                             uint8_t *plan_lds) {
  uint32_t *keys = reinterpret_cast<uint32_t *>(plan_lds);
  uint16_t *sstart = reinterpret_cast<uint16_t *>(plan_lds + ((size_t)4 << a.row_bits));
  __shared__ int wsum[32];
  __shared__ int cnt[4];

  const int tid = threadIdx.x;
  const int M = a.M;
  const int n2 = 1 << a.row_bits;
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.L.hdr);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + a.L.perm);
  int32_t *seg_adapter = reinterpret_cast<int32_t *>(a.ws + a.L.seg_adapter);
  int32_t *seg_start = reinterpret_cast<int32_t *>(a.ws + a.L.seg_start);
  int32_t *seg_len = reinterpret_cast<int32_t *>(a.ws + a.L.seg_len);
  Item *items_g = reinterpret_cast<Item *>(a.ws + a.L.items_g);
  ItemRows *items_gx = reinterpret_cast<ItemRows *>(a.ws + a.L.items_gx);
  Item *items_s = reinterpret_cast<Item *>(a.ws + a.L.items_s);

  if (tid < 4) cnt[tid] = 0;
  __syncthreads();

  // 1. classify (the active lanes of a wave are a prefix: lane 0 counts
  //    the wave's adapted rows)
  for (int m = tid; m < n2; m += NT) {
    uint32_t key = kSentinel;
    if (m < M) {
      const int id = plan_row(a, sls, nullptr, m, cnt);
      if (id >= 0) key = ((uint32_t)id << a.row_bits) | (uint32_t)m;
    }
    const uint64_t valid = __ballot(key != kSentinel);
    if ((tid & 63) == 0 && valid != 0) atomicAdd(&cnt[3], (int)__popcll(valid));
    keys[m] = key;
  }
  __syncthreads();

  // 2. bitonic sort, ascending, n2 keys (n2 a power of two)
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t ka = keys[lo], kb = keys[hi];
        if ((ka > kb) == up) {
          keys[lo] = kb;
          keys[hi] = ka;
        }
      }
      __syncthreads();
    }
  }

  // 3. segments
  const int n_ad = cnt[3];
  const uint32_t rmask = (1u << a.row_bits) - 1u;
  const int chunk = (n2 + NT - 1) / NT;
  const int i0 = tid * chunk;
  int heads = 0;
  for (int i = i0; i < i0 + chunk; ++i) {
    if (i < n_ad) heads += (i == 0 || (keys[i] >> a.row_bits) != (keys[i - 1] >> a.row_bits));
  }
  int n_seg = 0;
  int run = block_exclusive_scan<NT>(heads, wsum, &n_seg);
  for (int i = i0; i < i0 + chunk; ++i) {
    if (i < n_ad) {
      const bool head = (i == 0 || (keys[i] >> a.row_bits) != (keys[i - 1] >> a.row_bits));
      run += head;
      perm[i] = (int32_t)(keys[i] & rmask);
      if (head) {
        const int s = (int)(keys[i] >> a.row_bits);
        sstart[run - 1] = (uint16_t)i;
        seg_start[run - 1] = i;
        seg_adapter[run - 1] = s;
      }
    }
  }
  __syncthreads();

  // segment lengths and work-item counts
  const int schunk = (n_seg + NT - 1) / NT;
  const int s0 = tid * schunk;
  int ng = 0, ns = 0;
  for (int s = s0; s < s0 + schunk && s < n_seg; ++s) {
    const int len = ((s + 1 < n_seg) ? (int)sstart[s + 1] : n_ad) - (int)sstart[s];
    seg_len[s] = len;
    ng += (len + kRowsPerGatherItem - 1) / kRowsPerGatherItem;
    ns += (len + kRowsPerSgmvItem - 1) / kRowsPerSgmvItem;
  }
  int n_items_g = 0, n_items_s = 0;
  int og = block_exclusive_scan<NT>(ng, wsum, &n_items_g);
  int os = block_exclusive_scan<NT>(ns, wsum, &n_items_s);
  for (int s = s0; s < s0 + schunk && s < n_seg; ++s) {
    const int st = sstart[s];
    const int len = ((s + 1 < n_seg) ? (int)sstart[s + 1] : n_ad) - st;
    const int ad = (int)(keys[st] >> a.row_bits);
    int rk[kMaxSlices];
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)
      rk[q] = q < a.n_slices ? (sls ? sls[q].ranks[ad] : a.sl[q].ranks[ad]) : 0;
    for (int p = 0; p < len; p += kRowsPerGatherItem) {
      Item it;
      it.adapter = ad;
      it.pos = st + p;
      it.nrows = min(kRowsPerGatherItem, len - p);
      it.seg = s;
      ItemRows &ix = items_gx[og];
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q) ix.r[q] = rk[q];
      for (int q = 0; q < it.nrows; ++q) ix.rows[q] = (int32_t)(keys[st + p + q] & rmask);
      items_g[og++] = it;
    }
    for (int p = 0; p < len; p += kRowsPerSgmvItem) {
      Item it;
      it.adapter = ad;
      it.pos = st + p;
      it.nrows = min(kRowsPerSgmvItem, len - p);
      it.seg = s;
      items_s[os++] = it;
    }
  }
  if (tid == 0) {
    hdr[kHdrBadIds] = cnt[0];
    hdr[kHdrBadRanks] = cnt[1];
    hdr[kHdrBadPages] = cnt[2];
    hdr[kHdrAdapted] = n_ad;
    hdr[kHdrSegments] = n_seg;
    hdr[kHdrItemsGather] = n_items_g;
    hdr[kHdrItemsSgmv] = n_items_s;
    hdr[kHdrRows] = M;
  }
}



// LDS bytes of each form of the plan.
__host__ __device__ constexpr size_t plan_align16(size_t v) { return (v + 15) & ~(size_t)15; }
__host__ __device__ constexpr size_t plan_sort_lds(int row_bits) { return (size_t)6 << row_bits; }
constexpr int kPlanRowBitsMax = 13;  // sort width of the largest batch
static_assert((1 << kPlanRowBitsMax) == kPlanMaxRows, "kPlanMaxRows rows");
__host__ __device__ constexpr size_t plan_count_lds(int M, int S, int NT) {
  return plan_align16((size_t)M * 4) + plan_align16((size_t)S * 4) * (2 + NT / 64) +
         plan_align16((size_t)S) + plan_align16((size_t)S) * (NT / 64);
}

// Runs of equal adapters among a wave's 64 rows (b: the lane's adapter, or
// -1): whether the lane starts a run, and the run's length (valid at its
// first lane).  A run ends where the next lane's adapter differs.
__device__ __forceinline__ bool plan_run(int b, int lane, int *len) {
  const int up = __shfl_up(b, 1, 64);
  const int dn = __shfl_down(b, 1, 64);
  const int prev = lane == 0 ? -1 : up;
  const int next = lane == 63 ? -1 : dn;
  const uint64_t ends = __ballot(b >= 0 && next != b);
  *len = (int)__builtin_ctzll(ends >> lane) + 1;  // at a run's first lane its end is at or after it
  return b >= 0 && prev != b;
}

// Counting-sort plan.  `lds` holds plan_count_lds(M, S, NT) bytes: the
// rows' classes, then adapters [M], a histogram [S] (then each adapter's
// first sorted position), each adapter's first gather item [S], per-wave
// counts [NT / 64][S], the adapters' validity table [S] (bytes) and a
// per-wave scratch table [NT / 64][S] (bytes).
// Wave w owns the rows [w * RPW, (w + 1) * RPW): the per-wave counts give
// each (wave, adapter) its first sorted position, and the wave then places
// its rows in row order, so equal adapters keep row order (stable).
// Both passes work on runs of equal adapters within 64 rows (consecutive
// rows of one sequence share an adapter): one count and one position per
// run instead of a ballot loop over the distinct adapters.
template <int NT>
__device__ __forceinline__ void plan_counting(const PlanArgs &a, const PlanSliceL *sls,
                                              uint8_t *lds) {
  constexpr int NW = NT / 64;
  __shared__ uint64_t wsum64[32];
  __shared__ int cnt[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = a.M;
  const int S = a.S;
  int *binv = reinterpret_cast<int *>(lds);
  int *hist = reinterpret_cast<int *>(lds + plan_align16((size_t)M * 4));
  int *ibase = hist + plan_align16((size_t)S * 4) / 4;
  int *cntw = ibase + plan_align16((size_t)S * 4) / 4;
  int8_t *vt = reinterpret_cast<int8_t *>(cntw + plan_align16((size_t)S * 4) / 4 * NW);
  int8_t *dupt = vt + plan_align16((size_t)S);  // [NW][S]: a run's lane, per wave
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.L.hdr);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + a.L.perm);
  int32_t *seg_adapter = reinterpret_cast<int32_t *>(a.ws + a.L.seg_adapter);
  int32_t *seg_start = reinterpret_cast<int32_t *>(a.ws + a.L.seg_start);
  int32_t *seg_len = reinterpret_cast<int32_t *>(a.ws + a.L.seg_len);
  Item *items_g = reinterpret_cast<Item *>(a.ws + a.L.items_g);
  ItemRows *items_gx = reinterpret_cast<ItemRows *>(a.ws + a.L.items_gx);
  Item *items_s = reinterpret_cast<Item *>(a.ws + a.L.items_s);
  const int RPW = ((M + NW - 1) / NW + 63) & ~63;  // rows per wave, whole 64-row chunks

  if (tid < 4) cnt[tid] = 0;
  for (int s = tid; s < S; s += NT) hist[s] = 0;
  for (int i = tid; i < NW * S; i += NT) cntw[i] = 0;
  if (sls != nullptr)
    plan_classes<NT>(a, sls, vt, binv);  // ends with a barrier
  else
    __syncthreads();

  // 1. classify; histogram per adapter and per (wave range, adapter).  The
  //    64 rows a wave classifies at once lie in one wave range (RPW is a
  //    multiple of 64); each run of one adapter among them is counted with
  //    one atomic by its first lane (per-row atomics on a few hot adapters
  //    serialized: 24 us for 8192 rows of 8 adapters)
  for (int mb = wave * 64; mb < M; mb += NT) {
    const int m = mb + lane;
    const int b = m < M ? plan_row(a, sls, sls ? binv : nullptr, m, cnt) : -1;
    if (m < M) binv[m] = b;
    const int wr = mb / RPW;
    int len;
    if (plan_run(b, lane, &len)) {
      atomicAdd(&hist[b], len);
      atomicAdd(&cntw[wr * S + b], len);
    }
  }
  __syncthreads();

  // 2. segments and items per adapter; each thread owns a run of adapters
  const int bper = (S + NT - 1) / NT;
  const int s0 = min(S, tid * bper);
  const int s1 = min(S, s0 + bper);
  int nrow = 0, nseg = 0, ng = 0, ns = 0;
  for (int s = s0; s < s1; ++s) {
    const int h = hist[s];
    nrow += h;
    nseg += h > 0;
    ng += (h + kRowsPerGatherItem - 1) / kRowsPerGatherItem;
    ns += (h + kRowsPerSgmvItem - 1) / kRowsPerSgmvItem;
  }
  // the four counts as 16-bit fields of one 64-bit scan: each total is at
  // most M <= 8192 (every segment and item holds at least one row), so no
  // field carries into the next
  uint64_t tot4 = 0;
  const uint64_t ex4 = block_exclusive_scan<NT, uint64_t>(
      (uint64_t)nrow | (uint64_t)nseg << 16 | (uint64_t)ng << 32 | (uint64_t)ns << 48, wsum64, &tot4);
  int orow = (int)(ex4 & 0xFFFF), oseg = (int)((ex4 >> 16) & 0xFFFF);
  int og = (int)((ex4 >> 32) & 0xFFFF), os = (int)(ex4 >> 48);
  const int n_ad = (int)(tot4 & 0xFFFF), n_seg = (int)((tot4 >> 16) & 0xFFFF);
  const int n_items_g = (int)((tot4 >> 32) & 0xFFFF), n_items_s = (int)(tot4 >> 48);
  for (int s = s0; s < s1; ++s) {
    const int h = hist[s];
    hist[s] = orow;  // from here on: the adapter's first sorted position
    ibase[s] = og;
    if (h > 0) {
      seg_adapter[oseg] = s;
      seg_start[oseg] = orow;
      seg_len[oseg] = h;
      int rk[kMaxSlices];
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q)
        rk[q] = q < a.n_slices ? (sls ? sls[q].ranks[s] : a.sl[q].ranks[s]) : 0;
      for (int p = 0; p < h; p += kRowsPerGatherItem) {
        Item it;
        it.adapter = s;
        it.pos = orow + p;
        it.nrows = min(kRowsPerGatherItem, h - p);
        it.seg = oseg;
#pragma unroll
        for (int q = 0; q < kMaxSlices; ++q) items_gx[og].r[q] = rk[q];
        items_g[og++] = it;
      }
      for (int p = 0; p < h; p += kRowsPerSgmvItem) {
        Item it;
        it.adapter = s;
        it.pos = orow + p;
        it.nrows = min(kRowsPerSgmvItem, h - p);
        it.seg = oseg;
        items_s[os++] = it;
      }
      ++oseg;
    }
    // first sorted position of each wave's rows of adapter s (the counts
    // read before the first is overwritten: no chain of LDS round trips)
    int cw[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) cw[w] = cntw[w * S + s];
    int run = orow;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cntw[w * S + s] = run;
      run += cw[w];
    }
    orow += h;
  }
  __syncthreads();

  // 3. stable placement: each wave walks its rows in order, 64 at a time;
  //    the lanes of one adapter take consecutive positions in lane order.
  //    Every lane reads its adapter's next position (and first position and
  //    first item) once per 64 rows, so the loop over the distinct adapters
  //    of the 64 rows waits on no LDS read; its leader lane moves the next
  //    position on, which the wave's next 64 rows read (in order).
  const int wend = min(M, (wave + 1) * RPW);
  int8_t *dupw = dupt + (size_t)wave * plan_align16((size_t)S);
  for (int base = wave * RPW; base < wend; base += 64) {
    const int m = base + lane;
    const int b = m < wend ? binv[m] : -1;
    const int bc = b >= 0 ? b : 0;
    const int start = hist[bc];
    const int item0 = ibase[bc];
    int len;
    const bool head = plan_run(b, lane, &len);
    const uint64_t heads = __ballot(head);
    if (heads == 0) continue;
    // Two runs of one adapter among these rows (each run's first lane
    // writes its lane number at the adapter's entry; a lane that reads back
    // another's shares its adapter): the general loop below.  Else each run
    // takes the next positions of its adapter at once.
    // (volatile: the read must see the other lanes' writes, not be
    // forwarded from this lane's own store; a wave's LDS accesses complete
    // in order)
    volatile int8_t *dupv = dupw;
    if (head) dupv[b] = (int8_t)lane;
    const bool dup = head && dupv[b] != (int8_t)lane;
    if (__ballot(dup) == 0) {
      int rbase = 0;
      if (head) {
        rbase = cntw[wave * S + b];
        cntw[wave * S + b] = rbase + len;
      }
      // the lane's run starts at the highest run start at or below it
      const uint64_t upto = heads & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
      const int h = 63 - (int)__builtin_clzll(upto | 1ull);
      const int hb = __shfl(rbase, h, 64);
      if (b >= 0) {
        const int pos = hb + (lane - h);
        perm[pos] = m;
        const int rel = pos - start;
        items_gx[item0 + rel / kRowsPerGatherItem].rows[rel % kRowsPerGatherItem] = m;
      }
      continue;
    }
    const int first = cntw[wave * S + bc];
    uint64_t pending = __ballot(b >= 0);
    while (pending != 0) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int lb = __builtin_amdgcn_readlane(b, leader);
      const uint64_t mask = __ballot(b == lb);
      if (b == lb) {
        const int pos = first + __popcll(mask & ((1ull << lane) - 1ull));
        perm[pos] = m;
        const int rel = pos - start;
        items_gx[item0 + rel / kRowsPerGatherItem].rows[rel % kRowsPerGatherItem] = m;
        if (lane == leader) cntw[wave * S + lb] = first + __popcll(mask);
      }
      pending &= ~mask;
    }
  }

  if (tid == 0) {
    hdr[kHdrBadIds] = cnt[0];
    hdr[kHdrBadRanks] = cnt[1];
    hdr[kHdrBadPages] = cnt[2];
    hdr[kHdrAdapted] = n_ad;
    hdr[kHdrSegments] = n_seg;
    hdr[kHdrItemsGather] = n_items_g;
    hdr[kHdrItemsSgmv] = n_items_s;
    hdr[kHdrRows] = M;
  }
}

// Byte i of a packed class word, sign-extended.
__device__ __forceinline__ int plan_cls_byte(uint32_t w, int i) {
  return (int)(w << (24 - 8 * i)) >> 24;
}

// Plan for batches of at most 64 adapters, where one wave holds a value per
// adapter (lane s: adapter s).  `lds` holds plan_small_lds(M, NT) bytes: the
// row classes [M] (bytes), the sorted rows [M + 16], the rows of each
// adapter in each wave's row range [NW][64], per-adapter tables [9][64] and
// the adapters' validity [64] (bytes).
//   0. the classes of all rows (plan_classes);
//   A. each wave takes a contiguous range of rows (RPW, whole blocks of
//      64 * RL rows, RL consecutive rows per lane: 4 where every wave has
//      whole blocks, so a long run of one adapter takes a quarter of the
//      steps, else 1, so short ranges of many adapters spread over all
//      waves) and counts them per adapter with RL ballots per distinct
//      adapter of a block, into lane s's register;
//   B. wave 0: per adapter the row total, its first sorted position, first
//      16- and 64-row work items and segment (four wave-wide exclusive
//      scans, run side by side), the first position of each wave's rows,
//      the segment table, and the adapter's rank in every slice;
//   C. each wave walks its range again: the rows of adapter s in a block
//      take consecutive positions after the wave's running offset (a
//      register of lane s, read with readlane and moved on by lane s), and
//      are written to the sorted rows in LDS;
//   D. every thread copies the sorted rows out to perm with 16-byte stores,
//      and the waves write the work items, adapter by adapter, each item's
//      rows read back from LDS -- 16-byte stores throughout, instead of
//      scattered 4-byte stores per row and adapter.
// Stable by construction: the waves' ranges are in row order, and so are a
// block's rows in (lane, row) order.  No LDS atomics except the rare bad-row
// counts.
__host__ __device__ constexpr size_t plan_small_lds(int M, int NT) {
  return plan_align16((size_t)M) + plan_align16((size_t)(M + 16) * 4) + (size_t)(NT / 64) * 64 * 4 +
         9 * 64 * 4 + 64;
}

template <int NT, int RL>
__device__ __forceinline__ void plan_small(const PlanArgs &a, const PlanSliceL *sls, uint8_t *lds) {
  static_assert(RL == 1 || RL == 4, "1 or 4 rows per lane");
  constexpr int NW = NT / 64;
  static_assert(kMaxSlices == 4, "four rank columns in the tables");
  static_assert(kRowsPerGatherItem == 16 && kRowsPerSgmvItem % 16 == 0, "16-row item rows");
  static_assert(sizeof(Item) == 16 && sizeof(ItemRows) == 80 && offsetof(ItemRows, rows) == 16,
                "items, their rank columns and rows are written as 16-byte stores");
  __shared__ int cnt[4];   // bad ids, bad ranks, bad pages
  __shared__ int tot[4];   // adapted rows, 16-row items, 64-row items, segments
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = a.M;
  const int S = a.S;
  int8_t *cls = reinterpret_cast<int8_t *>(lds);
  int *permL = reinterpret_cast<int *>(lds + plan_align16((size_t)M));
  int *cntw = reinterpret_cast<int *>(lds + plan_align16((size_t)M) + plan_align16((size_t)(M + 16) * 4));
  // per adapter: [0] first sorted position [64] first 16-row item [128]
  // first 64-row item [192] rows [256] segment [320 + 64 q] rank in slice q
  int *tab = cntw + NW * 64;
  int8_t *vt = reinterpret_cast<int8_t *>(tab + 9 * 64);
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.L.hdr);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + a.L.perm);
  int32_t *seg_adapter = reinterpret_cast<int32_t *>(a.ws + a.L.seg_adapter);
  int32_t *seg_start = reinterpret_cast<int32_t *>(a.ws + a.L.seg_start);
  int32_t *seg_len = reinterpret_cast<int32_t *>(a.ws + a.L.seg_len);
  Item *items_g = reinterpret_cast<Item *>(a.ws + a.L.items_g);
  ItemRows *items_gx = reinterpret_cast<ItemRows *>(a.ws + a.L.items_gx);
  Item *items_s = reinterpret_cast<Item *>(a.ws + a.L.items_s);
  constexpr int BLK = 64 * RL;  // rows per block
  const int RPW = ((M + NW - 1) / NW + BLK - 1) / BLK * BLK;
  const int r0 = min(M, wave * RPW);
  const int r1 = min(M, r0 + RPW);

  // wave 0 loads the ranks of adapter `lane` first: their latency overlaps A
  int rk[kMaxSlices];
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q)
    rk[q] = (wave == 0 && q < a.n_slices && lane < S) ? sls[q].ranks[lane] : 0;

  if (tid < 4) cnt[tid] = 0;
  plan_classes<NT>(a, sls, vt, cls);  // ends with a barrier

  // this lane's RL rows of the block at `base`: classes, -1 past r1
  auto block = [&](int base, int c[RL]) {
    const int m0 = base + RL * lane;
    if constexpr (RL == 4) {
      const uint32_t w = m0 < r1 ? *reinterpret_cast<const uint32_t *>(cls + m0) : 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = m0 + i < r1 ? plan_cls_byte(w, i) : -1;
    } else {
      c[0] = m0 < r1 ? (int)cls[m0] : -1;
    }
  };
  // first class >= 0 among c[0..RL) (-1 if none)
  auto first_of = [](const int c[RL]) {
    int f = c[RL - 1];
#pragma unroll
    for (int i = RL - 2; i >= 0; --i) f = c[i] >= 0 ? c[i] : f;
    return f;
  };

  // A. per-adapter counts of this wave's range; bad rows become -1
  int mine = 0;
  for (int base = r0; base < r1; base += BLK) {
    int c[RL];
    block(base, c);
    bool bad = false;
#pragma unroll
    for (int i = 0; i < RL; ++i) bad = bad || c[i] < -1;
    if (bad) {  // rare: count, and store the rows as unadapted
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        if (c[i] < -1) {
          atomicAdd(&cnt[min(-2 - c[i], 2)], 1);
          c[i] = -1;
          cls[base + RL * lane + i] = -1;
        }
      }
    }
    for (;;) {
      const int f = first_of(c);
      const uint64_t pf = __ballot(f >= 0);
      if (pf == 0) break;
      const int s = __builtin_amdgcn_readlane(f, __ffsll((unsigned long long)pf) - 1);
      int n = 0;
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        n += __popcll(__ballot(c[i] == s));
        if (c[i] == s) c[i] = -1;
      }
      if (lane == s) mine += n;
    }
  }
  cntw[wave * 64 + lane] = mine;
  __syncthreads();

  // B. per adapter (wave 0, lane s)
  if (wave == 0) {
    int h = 0;
    for (int w = 0; w < NW; ++w) h += cntw[w * 64 + lane];
    const int v[4] = {h, (h + kRowsPerGatherItem - 1) / kRowsPerGatherItem,
                      (h + kRowsPerSgmvItem - 1) / kRowsPerSgmvItem, h > 0 ? 1 : 0};
    int inc[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __shfl_up(inc[i], o, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane >= o) inc[i] += y[i];
    }
    const int start = inc[0] - v[0];
    const int seg = inc[3] - v[3];
    int run = start;
    for (int w = 0; w < NW; ++w) {
      const int c = cntw[w * 64 + lane];
      cntw[w * 64 + lane] = run;
      run += c;
    }
    tab[lane] = start;
    tab[64 + lane] = inc[1] - v[1];
    tab[128 + lane] = inc[2] - v[2];
    tab[192 + lane] = h;
    tab[256 + lane] = seg;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) tab[320 + 64 * q + lane] = rk[q];
    if (h > 0) {
      seg_adapter[seg] = lane;
      seg_start[seg] = start;
      seg_len[seg] = h;
    }
    if (lane == 63) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] = inc[i];
    }
  }
  __syncthreads();

  // C. sorted positions into LDS
  {
    int off = cntw[wave * 64 + lane];
    const uint64_t below = (1ull << lane) - 1ull;
    for (int base = r0; base < r1; base += BLK) {
      int c[RL];
      block(base, c);
      int pos[RL];
      bool valid[RL];
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        pos[i] = 0;
        valid[i] = c[i] >= 0;
      }
      for (;;) {
        const int f = first_of(c);
        const uint64_t pf = __ballot(f >= 0);
        if (pf == 0) break;
        const int s = __builtin_amdgcn_readlane(f, __ffsll((unsigned long long)pf) - 1);
        uint64_t mk[RL];
        int before = 0, n = 0;
#pragma unroll
        for (int i = 0; i < RL; ++i) {
          mk[i] = __ballot(c[i] == s);
          before += __popcll(mk[i] & below);
          n += __popcll(mk[i]);
        }
        const int first = __builtin_amdgcn_readlane(off, s) + before;
        int k = 0;
#pragma unroll
        for (int i = 0; i < RL; ++i) {
          if (c[i] == s) {
            pos[i] = first + k++;
            c[i] = -1;
          }
        }
        if (lane == s) off += n;
      }
#pragma unroll
      for (int i = 0; i < RL; ++i)
        if (valid[i]) permL[pos[i]] = base + RL * lane + i;
    }
  }
  __syncthreads();

  // D. perm and the work items, with 16-byte stores
  const int n_ad = tot[0];
  for (int e = 4 * tid; e < n_ad; e += 4 * NT) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(permL + e);
    if (e + 3 < n_ad) {
      *reinterpret_cast<u32x4_t *>(perm + e) = v;
    } else {
      for (int i = 0; i < 4 && e + i < n_ad; ++i) perm[e + i] = (int)v[i];
    }
  }
  for (int s = wave; s < S; s += NW) {
    const int h = tab[192 + s];
    if (h == 0) continue;
    const int start = tab[s], ib = tab[64 + s], sb = tab[128 + s], seg = tab[256 + s];
    const u32x4_t r = {(unsigned)tab[320 + s], (unsigned)tab[384 + s], (unsigned)tab[448 + s],
                       (unsigned)tab[512 + s]};
    for (int j = lane; j * kRowsPerGatherItem < h; j += 64) {
      const int rel = j * kRowsPerGatherItem;
      const u32x4_t it = {(unsigned)s, (unsigned)(start + rel),
                          (unsigned)min(kRowsPerGatherItem, h - rel), (unsigned)seg};
      *reinterpret_cast<u32x4_t *>(items_g + ib + j) = it;
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(items_gx + ib + j);
      dst[0] = r;
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int *src = permL + start + rel + 4 * b4;  // past the segment: unused entries
        dst[1 + b4] = u32x4_t{(unsigned)src[0], (unsigned)src[1], (unsigned)src[2], (unsigned)src[3]};
      }
    }
    for (int j = lane; j * kRowsPerSgmvItem < h; j += 64) {
      const int rel = j * kRowsPerSgmvItem;
      const u32x4_t it = {(unsigned)s, (unsigned)(start + rel),
                          (unsigned)min(kRowsPerSgmvItem, h - rel), (unsigned)seg};
      *reinterpret_cast<u32x4_t *>(items_s + sb + j) = it;
    }
  }

  if (tid == 0) {
    hdr[kHdrBadIds] = cnt[0];
    hdr[kHdrBadRanks] = cnt[1];
    hdr[kHdrBadPages] = cnt[2];
    hdr[kHdrAdapted] = n_ad;
    hdr[kHdrSegments] = tot[3];
    hdr[kHdrItemsGather] = tot[1];
    hdr[kHdrItemsSgmv] = tot[2];
    hdr[kHdrRows] = M;
  }
}

// The whole plan, run by one workgroup of NT threads, in `lds_bytes` of LDS
// at `lds` (the caller guarantees room for at least the bitonic form).
template <int NT>
__device__ __forceinline__ void plan_body(const PlanArgs &a, uint8_t *lds, size_t lds_bytes) {
  __shared__ PlanSliceL sls[kMaxSlices];
  plan_stage_slices(a, sls);
  __syncthreads();
  if (a.S <= 64 && plan_small_lds(a.M, NT) <= lds_bytes) {
    if (a.M >= NT * 4)  // every wave has whole blocks of 256 rows
      plan_small<NT, 4>(a, sls, lds);
    else
      plan_small<NT, 1>(a, sls, lds);
  } else if (plan_count_lds(a.M, a.S, NT) <= lds_bytes) {
    plan_counting<NT>(a, sls, lds);
  } else {
    plan_bitonic<NT>(a, sls, lds);
  }
}

// The lean plan, for a workgroup of a GEMM kernel whose registers its own
// loop has spoken for: the counting or bitonic sort with each row's class
// found on its own (the slices walked with a loop), so the plan adds little
// register pressure to the kernel.
template <int NT>
__device__ __forceinline__ void plan_body_lean(const PlanArgs &a, uint8_t *lds, size_t lds_bytes) {
  if (plan_count_lds(a.M, a.S, NT) <= lds_bytes)
    plan_counting<NT>(a, nullptr, lds);
  else
    plan_bitonic<NT>(a, nullptr, lds);
}

}  // namespace plan_detail
}  // namespace lora
