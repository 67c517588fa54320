// plan_body.hpp -- the plan step as a device function, run either by its
// own kernel or by one extra workgroup of the base GEMM's launch.
//
// Plan ("Adapter Residency When One Replica Serves Many Fine-Tunes", section
// "Batch composition under many adapters": sort a batch's rows by adapter
// before the forward pass so every adapter's rows are contiguous; "S-LoRA:
// what the paper actually says ...", section "Batched LoRA computation": the
// corrections run as one segmented operation over the adapter-sorted rows).
//
// One workgroup does the whole plan for up to 8192 rows:
//   1. classify each row (none / adapted / bad id / bad rank / bad page);
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

// Exclusive scan of one int per thread over an NT-thread block.
// `wsum` is LDS scratch of >= NT / 64 + 1 ints; returns the exclusive prefix
// and writes the block total to *total (every thread sees it).
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int *total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < NT / 64) ? wsum[lane] : 0;
    int inc = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < NT / 64) wsum[lane] = inc - w;
    if (lane == NT / 64 - 1) wsum[NT / 64] = inc;
  }
  __syncthreads();
  *total = wsum[NT / 64];
  return x - v + wsum[wave];
}

// Row m's adapter if the row is adapted, else -1; counts the row's class in
// cnt[0] bad id, cnt[1] bad rank, cnt[2] bad page (rare: counted per row);
// cnt[3] adapted rows is counted by the callers that need it, per wave.
__device__ __forceinline__ int plan_classify(const PlanArgs &a, int m, int *cnt) {
  const int id = a.ids[m];
  if (id == -1) return -1;  // no adapter
  if (id < -1 || id >= a.S) {
    atomicAdd(&cnt[0], 1);
    return -1;
  }
  // every slice's rank must be in range, then every slice's pages
  bool rank_ok = true, page_ok = true;
  for (int q = 0; q < a.n_slices; ++q) {
    const PlanSlice &sl = a.sl[q];
    const int r = sl.ranks[id];
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
  if (!rank_ok) {
    atomicAdd(&cnt[1], 1);
    return -1;
  }
  if (!page_ok) {
    atomicAdd(&cnt[2], 1);
    return -1;
  }
  return id;
}

// Bitonic plan.  `plan_lds` holds plan_sort_lds(row_bits) bytes: the sort
// keys [n2] then segment starts [n2] (uint16).
template <int NT>
__device__ __forceinline__ void plan_bitonic(const PlanArgs &a, uint8_t *plan_lds) {
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
      const int id = plan_classify(a, m, cnt);
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
    for (int q = 0; q < kMaxSlices; ++q) rk[q] = q < a.n_slices ? a.sl[q].ranks[ad] : 0;
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
__host__ __device__ constexpr size_t plan_count_lds(int M, int S, int NT) {
  return plan_align16((size_t)M * 4) + plan_align16((size_t)S * 4) * (2 + NT / 64);
}

// Counting-sort plan.  `lds` holds plan_count_lds(M, S, NT) bytes: the
// rows' adapters [M], a histogram [S] (then each adapter's first sorted
// position), each adapter's first gather item [S] and per-wave counts
// [NT / 64][S].
// Wave w owns the rows [w * RPW, (w + 1) * RPW): the per-wave counts give
// each (wave, adapter) its first sorted position, and the wave then places
// its rows in row order, so equal adapters keep row order (stable).
template <int NT>
__device__ __forceinline__ void plan_counting(const PlanArgs &a, uint8_t *lds) {
  constexpr int NW = NT / 64;
  __shared__ int wsum[32];
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
  __syncthreads();

  // 1. classify; histogram per adapter and per (wave range, adapter).  The
  //    64 rows a wave classifies at once lie in one wave range (RPW is a
  //    multiple of 64), so each distinct adapter among them is counted with
  //    one atomic by its lowest lane (per-row atomics on a few hot adapters
  //    serialized: 24 us for 8192 rows of 8 adapters)
  for (int mb = wave * 64; mb < M; mb += NT) {
    const int m = mb + lane;
    const int b = m < M ? plan_classify(a, m, cnt) : -1;
    if (m < M) binv[m] = b;
    const int wr = mb / RPW;
    uint64_t pending = __ballot(b >= 0);
    while (pending != 0) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int lb = __shfl(b, leader, 64);
      const uint64_t mask = __ballot(b == lb);
      if (lane == leader) {
        const int c = __popcll(mask);
        atomicAdd(&hist[lb], c);
        atomicAdd(&cntw[wr * S + lb], c);
      }
      pending &= ~mask;
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
  int n_ad = 0, n_seg = 0, n_items_g = 0, n_items_s = 0;
  int orow = block_exclusive_scan<NT>(nrow, wsum, &n_ad);
  int oseg = block_exclusive_scan<NT>(nseg, wsum, &n_seg);
  int og = block_exclusive_scan<NT>(ng, wsum, &n_items_g);
  int os = block_exclusive_scan<NT>(ns, wsum, &n_items_s);
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
      for (int q = 0; q < kMaxSlices; ++q) rk[q] = q < a.n_slices ? a.sl[q].ranks[s] : 0;
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
    // first sorted position of each wave's rows of adapter s
    int run = orow;
    for (int w = 0; w < NW; ++w) {
      const int c = cntw[w * S + s];
      cntw[w * S + s] = run;
      run += c;
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
  for (int base = wave * RPW; base < wend; base += 64) {
    const int m = base + lane;
    const int b = m < wend ? binv[m] : -1;
    const int bc = b >= 0 ? b : 0;
    const int first = cntw[wave * S + bc];
    const int start = hist[bc];
    const int item0 = ibase[bc];
    uint64_t pending = __ballot(b >= 0);
    while (pending != 0) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int lb = __shfl(b, leader, 64);
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

// The whole plan, run by one workgroup of NT threads, in `lds_bytes` of LDS
// at `lds` (the caller guarantees room for at least the bitonic form).
template <int NT>
__device__ __forceinline__ void plan_body(const PlanArgs &a, uint8_t *lds, size_t lds_bytes) {
  if (plan_count_lds(a.M, a.S, NT) <= lds_bytes)
    plan_counting<NT>(a, lds);
  else
    plan_bitonic<NT>(a, lds);
}

}  // namespace plan_detail
}  // namespace lora
