// lora_sgmv.hip -- segmented (SGMV-style) LoRA correction on MFMA tiles.
//
// "Your LoRA Adapters Are Thrashing Your GPUs", section 09 (Punica's
// segmented gather matrix-vector kernels: one launch for all adapters of a
// mixed batch) and "S-LoRA: what the paper actually says ...", section
// "Batched LoRA computation" (rows sorted by adapter so each adapter's rows
// form a contiguous segment; one kernel walks all segments).  Where a
// segment has enough rows, the two small products are dense contractions
// and run on the matrix cores here.
//
// Work items come from the plan: up to RB (16 or 64) consecutive rows of
// one adapter's segment.  bf16 only (the matrix cores' operand type).
//
// shrink: t[p, j] = sum_k A_s[j, k] x[perm[p], k]
//   grid (item, slice or all slices, k split).  A workgroup covers the
//   16-rank blocks of one slice, or of every slice (then each x row is
//   fetched once for all projections, with fewer workgroups).
//   16 x 16 output blocks (rows x ranks) on v_mfma_f32_16x16x32_bf16; x rows
//   are gathered through perm straight into the A operand (16 bytes per
//   lane), A_s rows into the B operand.  The 4 waves take alternate 32-wide k
//   steps of the split; their partial blocks are summed in wave order through
//   LDS.  Output: fp32 partials, one per k split (summed in split order by
//   the expand).
// expand: y[perm[p], n] += scale_s * sum_j B_s[n, j] t[p, j]
//   grid: (item, 256-column block of any slice), each column block kept on
//   one XCD across items.  t (the sum of the k-split partials, in split
//   order) is split into bf16 hi + lo parts (t = hi + lo to ~16 mantissa
//   bits), so two MFMAs per block keep t's precision; B_s rows feed the B
//   operand (ranks are contiguous in both slot and pool layouts).  Then
//   y = y + scale * acc, rounded once.  Rows without an adapter are never
//   touched.
#include "kernels.hpp"

namespace lora {

namespace {

constexpr int RMAX_MFMA = 64; // largest max_rank these kernels take
// Stages of the LDS-staged shrink per (rows per item, A rows per stage):
// measured on MI355X, fewer stages (more workgroups per CU) where a
// workgroup streams little
template <int RB, int AROWS>
constexpr int kShrinkStages = RB == 16 ? 3 : (AROWS == 16 ? 5 : AROWS == 128 ? 3 : 4);
constexpr int kExpandCols16 = 256;  // expand columns per workgroup, 16-row items (512 measured slower)

__device__ __forceinline__ bf16x8_t ld16(const void *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

__device__ __forceinline__ bf16x8_t zero8() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
}

// Row of A_s as seen by one lane: a 16-rank block of one slice.  For slot
// storage `base` is the row start; for a pool each 16-byte vector goes
// through the page table (a vector never crosses a page).
struct ARow {
  const uint8_t *base;  // slots: &A_s[j][0]; pool: pool base
  const int32_t *pt;    // pool: page-table row of the adapter; slots: nullptr
  int64_t off;          // pool: logical byte offset of A_s[j][0]
  int32_t shift;
  int64_t mask;
};

__device__ __forceinline__ ARow make_arow(const AdapterRef &ar, int s, int64_t j) {
  ARow w;
  if (!ar.pooled) {
    w.base = ar.A + ((int64_t)s * ar.max_rank + j) * ar.k * ar.elem_bytes;
    w.pt = nullptr;
    w.off = 0;
  } else {
    w.base = ar.pool;
    w.pt = ar.page_table + (int64_t)s * ar.max_pages;
    w.off = j * ar.k * ar.elem_bytes;
  }
  w.shift = ar.page_shift;
  w.mask = ar.page_bytes - 1;
  return w;
}

// A pooled row whose bytes for k in [kbeg, kend) lie in one page becomes a
// slot-style row (base + 2 kk): one page-table load per lane before the k
// loop instead of one ahead of every vector.  (k and the bounds are
// multiples of 8, so the last vector ends at byte 2 kend - 1.)
__device__ __forceinline__ void arow_resolve(ARow &w, int64_t kbeg, int64_t kend) {
  if (w.pt == nullptr || kend <= kbeg) return;
  const int64_t o0 = w.off + kbeg * 2;
  const int64_t idx = o0 >> w.shift;
  if (idx != ((w.off + kend * 2 - 1) >> w.shift)) return;
  const int64_t pg = w.pt[idx];
  w.base = reinterpret_cast<const uint8_t *>(reinterpret_cast<uintptr_t>(w.base) +
                                             (pg - idx) * (int64_t(1) << w.shift) + w.off);
  w.pt = nullptr;
}

__device__ __forceinline__ const uint8_t *arow_ptr(const ARow &w, int64_t kk) {
  if (w.pt == nullptr) return w.base + kk * 2;
  const int64_t off = w.off + kk * 2;
  return w.base + ((int64_t)w.pt[off >> w.shift] << w.shift) + (off & w.mask);
}

// The item's rank blocks over all slices, in slice order: block v is
// (slice, 16-rank block) with 16 * block < r_slice.  rk: the adapter's rank
// in every slice.  Returns the count and, for v, its slice / block / rank.
__device__ __forceinline__ int vblock_count(const LoraArgs &a, const int (&rk)[kMaxSlices]) {
  int n = 0;
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q)
    if (q < a.n_slices) n += (rk[q] + 15) >> 4;
  return n;
}
__device__ __forceinline__ void vblock_find(const LoraArgs &a, const int (&rk)[kMaxSlices], int v,
                                            int &slice, int &jb, int &r) {
  slice = 0;
  jb = v;
  r = rk[0];
  bool found = false;
#pragma unroll
  for (int q = 0; q + 1 < kMaxSlices; ++q) {
    if (found || q + 1 >= a.n_slices) continue;
    const int nb = (r + 15) >> 4;
    if (jb < nb) {
      found = true;
      continue;
    }
    jb -= nb;
    slice = q + 1;
    r = rk[q + 1];
  }
}

// The adapter's rank in every slice: from the 16-row item's record
// (FROM_ITEM), else from the slices' rank arrays.
template <bool FROM_ITEM>
__device__ __forceinline__ void item_ranks(const LoraArgs &a, const ItemRows *ix, int adapter,
                                           int (&rk)[kMaxSlices]) {
#pragma unroll
  for (int q = 0; q < kMaxSlices; ++q) {
    if constexpr (FROM_ITEM)
      rk[q] = q < a.n_slices ? ix->r[q] : 0;
    else
      rk[q] = q < a.n_slices ? a.sl[q].ranks[adapter] : 0;
  }
}

// Row of sorted position it.pos + row: from the 16-row item's record, else
// from perm.
template <bool FROM_ITEM>
__device__ __forceinline__ int item_row(const ItemRows *ix, const int32_t *perm, const Item &it,
                                        int row) {
  if constexpr (FROM_ITEM)
    return ix->rows[row];
  else
    return perm[it.pos + row];
}

// Rank blocks [v0, v0 + G) of one item over one k split: MFMA partial
// blocks per wave (alternate 32-wide k steps), summed in wave order through
// LDS, written as this split's fp32 partials.
template <int RB, int G, int U>
__device__ __forceinline__ void shrink_blocks(const LoraArgs &a, const Item &it,
                                              const int (&rk)[kMaxSlices], int v0, int nvb,
                                              int64_t kbeg, int64_t kend,
                                              const int64_t (&xoff)[RB / 16],
                                              const bool (&xv)[RB / 16],
                                              f32x4_t (*red)[4][64]) {
  constexpr int RBK = RB / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kl = (lane >> 4) * 8;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(a.x);

  ARow arow[G];
  bool jv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    jv[g] = false;
    arow[g] = ARow{nullptr, nullptr, 0, 0, 0};
    if (v0 + g < nvb) {
      int slice, jb, r;
      vblock_find(a, rk, v0 + g, slice, jb, r);
      const int j = jb * 16 + (lane & 15);
      jv[g] = j < r;
      arow[g] = make_arow(a.sl[slice].ar, it.adapter, jv[g] ? j : 0);
      arow_resolve(arow[g], kbeg, kend);
    }
  }

  f32x4_t acc[RBK][G];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[rb][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // U k steps per round: all their loads are issued before their MFMAs
  for (int64_t kb0 = kbeg + wave * 32; kb0 < kend; kb0 += 128 * U) {
    bf16x8_t xf[U][RBK], af[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kc = kb0 + 128 * u + kl;
      const bool kin = kc < kend;
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
        xf[u][rb] = (xv[rb] && kin) ? ld16(xb + xoff[rb] + kc) : zero8();
#pragma unroll
      for (int g = 0; g < G; ++g)
        af[u][g] = (jv[g] && kin) ? ld16(arow_ptr(arow[g], kc)) : zero8();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (v0 + g < nvb)
            acc[rb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u][rb], af[u][g], acc[rb][g], 0, 0, 0);
  }

  float *tpart = reinterpret_cast<float *>(a.ws + a.L.tpart);
  // four output blocks per round through LDS; wave w sums block w
#pragma unroll
  for (int c0 = 0; c0 < RBK * G; c0 += 4) {
    if (v0 + (c0 % G) >= nvb) continue;  // uniform: the whole chunk is past the end
    __syncthreads();  // the previous round's reads of red are done
#pragma unroll
    for (int b = 0; b < 4; ++b) red[wave][b][lane] = acc[(c0 + b) / G][(c0 + b) % G];
    __syncthreads();
    const int blk = c0 + wave;
    const int rb = blk / G;
    const int g = blk % G;
    if (v0 + g < nvb) {
      int slice, jb, r;
      vblock_find(a, rk, v0 + g, slice, jb, r);
      const f32x4_t sum = ((red[0][wave][lane] + red[1][wave][lane]) + red[2][wave][lane]) +
                          red[3][wave][lane];
      const int j = jb * 16 + (lane & 15);
      if (j < r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb * 16 + ((lane >> 4) << 2) + i;
          if (row < it.nrows)
            tpart[tpart_index(blockIdx.z, it.pos + row, slice, j, a.L.rows, a.n_slices, a.L.R)] =
                sum[i];
        }
      }
    }
  }
}

// grid (item, slice or all slices, k split).  PER_SLICE: one slice per
// workgroup, at most 4 rank blocks (ranks <= 64), so only the 4-block path
// is compiled and it alone sets the register budget (64-row items: 422 ->
// 212 VGPRs, two waves per SIMD; with one k step per load round the
// 8192-row prefill shrink went 31.4 -> 23.4 us, 2 or 4 steps 24.8 / 25.2 us).
constexpr int kShrinkSteps64 = 1;
template <int RB, bool PER_SLICE>
__global__ __launch_bounds__(256) void k_shrink_mfma(LoraArgs a) {
  constexpr int RBK = RB / 16;
  __shared__ f32x4_t red[4][4][64];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  // the item slot exists up to the list's capacity: read it beside the count
  const Item it =
      reinterpret_cast<const Item *>(a.ws + (RB == 16 ? a.L.items_g : a.L.items_s))[item];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + item;
  if (item >= hdr[RB == 16 ? kHdrItemsGather : kHdrItemsSgmv]) return;
  int rk[kMaxSlices];
  item_ranks<RB == 16>(a, ix, it.adapter, rk);
  // grid.y == 1: every slice's rank blocks (x rows read once for all);
  // grid.y == n_slices: slice blockIdx.y's blocks only (more workgroups)
  int vlo = 0, vhi = vblock_count(a, rk);
  if (gridDim.y > 1) {
    vlo = 0;
    int nb = 0;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) {
      if (q < (int)blockIdx.y) vlo += (rk[q] + 15) >> 4;
      if (q == (int)blockIdx.y) nb = (rk[q] + 15) >> 4;
    }
    vhi = vlo + nb;
  }
  if (vhi == vlo) return;
  const int64_t kbeg = (int64_t)blockIdx.z * a.kchunk;
  if (kbeg >= a.k) return;
  const int64_t kend = min(a.k, kbeg + a.kchunk);
  const int32_t *perm = reinterpret_cast<const int32_t *>(a.ws + a.L.perm);
  const int lane = threadIdx.x & 63;

  int64_t xoff[RBK];
  bool xv[RBK];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const int row = rb * 16 + (lane & 15);
    xv[rb] = row < it.nrows;
    xoff[rb] = xv[rb] ? (int64_t)item_row<RB == 16>(ix, perm, it, row) * a.ldx : 0;
  }

  // block groups sized so that few blocks keep several k steps of loads
  // in flight; up to 8 blocks (two projections of rank 64) share one read
  // of the x rows, more take another pass over them
  if (PER_SLICE || vhi - vlo <= 4) {
    shrink_blocks<RB, 4, RB == 64 ? kShrinkSteps64 : 4>(a, it, rk, vlo, vhi, kbeg, kend, xoff, xv, red);
  } else if constexpr (!PER_SLICE) {
    for (int v0 = vlo; v0 < vhi; v0 += 8)
      shrink_blocks<RB, 8, RB == 16 ? 2 : 1>(a, it, rk, v0, vhi, kbeg, kend, xoff, xv, red);
  }
}

// Keep the first `keep` bf16 elements of a 16-byte fragment, zero the rest
// (ranks at or past r: slot padding may hold anything).  Branch-free.
__device__ __forceinline__ bf16x8_t keep_first(bf16x8_t v, int keep) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  const uint32_t q[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t msk = 2 * i + 1 < keep ? 0xffffffffu : (2 * i < keep ? 0xffffu : 0u);
    o[i] = q[i] & msk;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// FAST: y 16-byte aligned with every slice's columns a multiple of 8 wide
// and at a multiple of 8, and either every slice in slots with max_rank % 8
// == 0 (16-byte B rows) or (POOL) every slice in a pool, where an item whose
// rank is a multiple of 8 takes the same B loads through the page table.
// Then the B fragments, the item's row numbers, the y runs
// and the k-split partials are all loaded unconditionally at clamped
// addresses and masked by selects afterwards, so they leave back to back
// (loads under a branch -- even a uniform one -- or behind a slot/pool
// address branch each sat in their own block behind a full wait: 18.5 ->
// 16.2 us at the 70B q+v shapes).  The shrink keeps its masked loads: it is
// bound by the address path of the vector memory unit, where clamped lanes
// cost as much as real ones (measured slower with clamping).
// RMX: the largest padded rank the instantiation takes (32 or RMAX_MFMA).
// The plan drops rows whose rank exceeds max_rank, so every item's rank is
// at most the slices' largest max_rank, which selects RMX on the host: at
// ranks up to 32 the B fragments and registers of the second k step go.
template <int RB, int ECB, bool FAST, int RMX, bool POOL>
__device__ __forceinline__ void expand_body(const LoraArgs &a) {
  constexpr int RBK = RB / 16;
  constexpr int KP = RMX + 8;  // padded LDS row (bf16)
  constexpr int CB = ECB / 64;       // 16-column blocks per wave
  constexpr int CPR = ECB / 8;       // 16-byte y chunks per row
  constexpr int CPT = 16 * CPR / 256;  // 16-byte y chunks per thread per 16-row pass
  constexpr int YLD = ECB + 4;       // transposed-output LDS row (fp32)
  constexpr int YCH = CPT * RBK;     // 16-byte y chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t th[RB * KP];
  __shared__ __attribute__((aligned(16))) uint16_t tl[RB * KP];
  __shared__ __attribute__((aligned(16))) float ys[16 * YLD];

  // Workgroup b runs on XCD b % 8.  A column block stays on one XCD for
  // every item, so the items of one adapter -- which read the same B rows
  // -- share that XCD's L2 instead of each fetching B (whole 128-byte lines
  // even for a small rank) from memory.  XCD x takes the blocks of columns
  // [x d / 8, (x + 1) d / 8): the base GEMM's tile order gives each XCD the
  // same eighth of y's columns, so the y rows this kernel updates are still
  // in that XCD's L2.
  const int ncb = a.col_blk[a.n_slices];
  const int per_xcd = (ncb + 7) >> 3;
  const int b = blockIdx.x;
  const int q = b >> 3;
  const int item = q / per_xcd;
  const int xcd = b & 7;
  const int cbk = ((xcd * ncb) >> 3) + (q - item * per_xcd);
  if (cbk >= (((xcd + 1) * ncb) >> 3)) return;
  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  // the item slot exists up to the list's capacity, so it is read beside
  // the count instead of after it
  const Item it =
      reinterpret_cast<const Item *>(a.ws + (RB == 16 ? a.L.items_g : a.L.items_s))[item];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + item;
  if (item >= hdr[RB == 16 ? kHdrItemsGather : kHdrItemsSgmv]) return;
  int slice = 0;
  while (slice + 1 < a.n_slices && cbk >= a.col_blk[slice + 1]) ++slice;
  const SliceRef &sl = a.sl[slice];
  int r;
  if constexpr (RB == 16)
    r = ix->r[slice];
  else
    r = sl.ranks[it.adapter];
  if (r == 0) return;
  const int nr = it.nrows;
  const int64_t n0 = (int64_t)(cbk - a.col_blk[slice]) * ECB;
  const int32_t *perm = reinterpret_cast<const int32_t *>(a.ws + a.L.perm);
  const float *tpart = reinterpret_cast<const float *>(a.ws + a.L.tpart);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kp = (r + 31) & ~31;  // ranks padded to the MFMA k step

  // 1. loads that do not depend on t, issued first: B fragments and the y
  //    chunks this thread will update (row = chunk / CPR, 8 columns each)
  const AdapterRef &ar = sl.ar;
  const int stride = ar.pooled ? r : ar.max_rank;  // B row stride (elements)
  const bool bvec = (stride % 8) == 0;
  bf16x8_t fb[RMX / 32][CB];
  // pooled B rows are r elements long: the vector loads need r % 8 == 0
  // (the pool base is 16-byte aligned and a page at least 256 bytes, so a
  // vector never straddles pages); other ranks take the generic loads
  const bool fast_b = FAST && (!POOL || (r & 7) == 0);
  if (fast_b) {
#pragma unroll
    for (int ks = 0; ks < RMX / 32; ++ks) {
      // uniform: no rank chunk left (the MFMA loop stops at the same step,
      // so the fragments past it are never read)
      if (ks > 0 && ks * 32 >= kp) break;
      const int jl = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t n = n0 + (wave * CB + cb) * 16 + (lane & 15);
        // a rank chunk past the rank loads chunk 0's vector (same lines);
        // the clamped (na, ja) is always inside the adapter's B
        const bool ok = ks * 32 < kp && n < sl.d && jl < r;
        const bool ok0 = n < sl.d && jl - ks * 32 < r;
        const int64_t na = ok || ok0 ? n : n0;
        const int ja = ok ? jl : (ok0 ? jl - ks * 32 : 0);
        const uint8_t *bp;
        if constexpr (POOL) {
          // every page-table entry is loaded unconditionally, so the
          // compiler issues them as one batch ahead of the B vectors
          const int64_t off = ((int64_t)r * ar.k + na * r + ja) * 2;
          const int64_t page =
              ar.page_table[(int64_t)it.adapter * ar.max_pages + (off >> ar.page_shift)];
          bp = ar.pool + (page << ar.page_shift) + (off & (ar.page_bytes - 1));
        } else {
          bp = ar.B + (((int64_t)it.adapter * ar.d + na) * ar.max_rank + ja) * 2;
        }
        fb[ks][cb] = keep_first(ld16(bp), ok ? r - jl : 0);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < RMX / 32; ++ks) {
      const int jl = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t n = n0 + (wave * CB + cb) * 16 + (lane & 15);
        bf16x8_t v = zero8();
        if (ks * 32 < kp && n < sl.d && jl < r) {
          if (bvec && jl + 8 <= r) {
            v = ld16(adapter_b_ptr(ar, it.adapter, r, n, jl));
          } else if (bvec && !ar.pooled) {
            // a slot row is padded to max_rank (a multiple of 8): load the
            // whole 8-rank vector and zero the ranks past r (padding may
            // hold anything)
            uint16_t e8[8];
            *reinterpret_cast<bf16x8_t *>(e8) = ld16(adapter_b_ptr(ar, it.adapter, r, n, jl));
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (jl + q >= r) e8[q] = 0;
            v = __builtin_bit_cast(bf16x8_t, e8);
          } else {
            uint16_t e8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
              e8[q] = (jl + q < r) ? *reinterpret_cast<const uint16_t *>(
                                         adapter_b_ptr(ar, it.adapter, r, n, jl + q))
                                   : (uint16_t)0;
            v = __builtin_bit_cast(bf16x8_t, e8);
          }
        }
        fb[ks][cb] = v;
      }
    }
  }
  const bool yvec = a.y_vec && (sl.col0 % 8) == 0;
  uint16_t *yb = reinterpret_cast<uint16_t *>(a.y) + sl.col0;
  uint16_t *yp[YCH];
  uint4 yv[YCH];
  if constexpr (FAST) {
    // row numbers first (one batch of loads), then the y runs
    int rows[YCH];
#pragma unroll
    for (int c = 0; c < YCH; ++c) {
      const int ch = (c / CPT) * 16 * CPR + tid + (c % CPT) * 256;
      const int row = ch / CPR;
      rows[c] = item_row<RB == 16>(ix, perm, it, row < nr ? row : 0);
    }
#pragma unroll
    for (int c = 0; c < YCH; ++c) {
      const int ch = (c / CPT) * 16 * CPR + tid + (c % CPT) * 256;
      const int row = ch / CPR;
      const int64_t n = n0 + (ch % CPR) * 8;
      const bool ok = row < nr && n < sl.d;
      uint16_t *p = yb + (int64_t)rows[c] * a.ldy + (ok ? n : n0);
      if constexpr (RB == 64) {
        // prefill runs: read once, then overwritten by a streaming store
        // (nontemporal: 37.6 -> 35.8 us at 8192 x 4096)
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        yv[c] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
      } else {
        yv[c] = *reinterpret_cast<const uint4 *>(p);
      }
      yp[c] = ok ? p : nullptr;
    }
  }
#pragma unroll
  for (int c = 0; c < (FAST ? 0 : YCH); ++c) {
    const int ch = (c / CPT) * 16 * CPR + tid + (c % CPT) * 256;  // pass c / CPT
    const int row = ch / CPR;
    const int64_t n = n0 + (ch % CPR) * 8;
    yp[c] = nullptr;
    yv[c] = make_uint4(0, 0, 0, 0);
    if (row < nr && n < sl.d) {
      yp[c] = yb + (int64_t)item_row<RB == 16>(ix, perm, it, row) * a.ldy + n;
      if (yvec && n + 8 <= sl.d) {
        yv[c] = *reinterpret_cast<const uint4 *>(yp[c]);
      } else {
        uint16_t e8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e8[q] = (n + q < sl.d) ? yp[c][q] : (uint16_t)0;
        yv[c] = __builtin_bit_cast(uint4, e8);
      }
    }
  }

  // 2. t = sum of the k-split partials, as bf16 hi + lo (4 ranks per thread);
  //    where the base GEMM computed t (one split, indexed by the row itself)
  //    it is read from there
  const bool t_by_row = a.fused_cap > 0;
  const int nsplit = t_by_row ? 1 : a.ksplit;
  const int kp4 = kp >> 2;
  for (int e = tid; e < RB * kp4; e += 256) {
    const int row = e / kp4;
    const int j = (e - row * kp4) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (FAST) {
      const bool ok = row < nr && j < r;
      const int rc = ok ? row : 0;
      const int64_t tp = t_by_row ? (int64_t)item_row<RB == 16>(ix, perm, it, rc) : it.pos + rc;
      v = tpart_sum4(tpart, tp, slice, ok ? j : 0, nsplit, a.L.rows, a.n_slices, a.L.R);
      // entries past the rank are never written by the shrink
      v.x = ok ? v.x : 0.f;
      v.y = ok && j + 1 < r ? v.y : 0.f;
      v.z = ok && j + 2 < r ? v.z : 0.f;
      v.w = ok && j + 3 < r ? v.w : 0.f;
    } else if (row < nr && j < r) {
      const int64_t tp = t_by_row ? (int64_t)item_row<RB == 16>(ix, perm, it, row) : it.pos + row;
      v = tpart_sum4(tpart, tp, slice, j, nsplit, a.L.rows, a.n_slices, a.L.R);
      // entries past the rank are never written by the shrink
      if (j + 1 >= r) v.y = 0.f;
      if (j + 2 >= r) v.z = 0.f;
      if (j + 3 >= r) v.w = 0.f;
    }
    const float f[4] = {v.x, v.y, v.z, v.w};
    uint16_t h[4], l[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h[c] = f32_to_bf16_bits(f[c]);
      l[c] = f32_to_bf16_bits(f[c] - bf16_bits_to_f32(h[c]));
    }
    *reinterpret_cast<uint2 *>(&th[row * KP + j]) =
        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
    *reinterpret_cast<uint2 *>(&tl[row * KP + j]) =
        make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
  }
  __syncthreads();

  // 3. acc[rb][cb] = t (rows) x B_s^T (16 columns), on the matrix cores
  f32x4_t acc[RBK][CB];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < RMX / 32; ++ks) {
    if (ks * 32 >= kp) break;
    const int jl = ks * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      const bf16x8_t fh = ld16(&th[(rb * 16 + (lane & 15)) * KP + jl]);
      const bf16x8_t fl = ld16(&tl[(rb * 16 + (lane & 15)) * KP + jl]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh, fb[ks][cb], acc[rb][cb], 0, 0, 0);
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl, fb[ks][cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }

  // 4. y += scale * acc, 16 rows at a time through LDS so that every thread
  //    updates whole 16-byte runs of one y row (rounded once)
  const float scale = sl.scales[it.adapter];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    if (rb * 16 >= nr) break;  // uniform
    if (rb > 0) __syncthreads();  // previous pass's reads of ys are done
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ys[(((lane >> 4) << 2) + i) * YLD + (wave * CB + cb) * 16 + (lane & 15)] = acc[rb][cb][i];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
      const int c = rb * CPT + h;
      if (yp[c] == nullptr) continue;
      const int ch = tid + h * 256;
      const int lr = ch / CPR;  // row within the pass
      const int col = (ch % CPR) * 8;
      const float4 s0 = *reinterpret_cast<const float4 *>(&ys[lr * YLD + col]);
      const float4 s1 = *reinterpret_cast<const float4 *>(&ys[lr * YLD + col + 4]);
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      uint16_t e8[8];
      const uint16_t *old = reinterpret_cast<const uint16_t *>(&yv[c]);
#pragma unroll
      for (int q = 0; q < 8; ++q) e8[q] = f32_to_bf16_bits(bf16_bits_to_f32(old[q]) + scale * sv[q]);
      const int64_t n = n0 + col;
      if (FAST || (yvec && n + 8 <= sl.d)) {
        if constexpr (RB == 64) {
          // prefill runs: y is far larger than L2 and each run is written
          // once, so the stores stream past it (nontemporal: 42.1 -> 37.9 us
          // at 8192 x 4096)
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, e8),
                                      reinterpret_cast<u32x4_t *>(yp[c]));
        } else {
          *reinterpret_cast<uint4 *>(yp[c]) = __builtin_bit_cast(uint4, e8);
        }
      } else {
        for (int q = 0; q < 8; ++q)
          if (n + q < sl.d) yp[c][q] = e8[q];
      }
    }
  }
}

// Decode expand on independent waves (16-row items).  Each wave updates one
// item's 16 rows over NU units of 64 columns of one slice with no LDS and no
// barrier: it computes the transposed product D' = B_s t^T on the matrix
// cores -- B_s rows (ranks contiguous) as the A operand, t rows as the B
// operand -- with the B_s rows permuted so that D' lands in the registers
// as whole y runs: A-operand row m of column block cb is column 16 (m / 4)
// + 4 cb + m % 4 of the unit's 64, so lane l ends up with y row l % 16,
// columns 16 (l / 16) .. + 15, after the four blocks (MFMA 16x16x32 D
// layout: lane l holds rows 4 (l / 16) + i of column l % 16).  It then
// reads those 32 bytes of y, adds scale * D' and writes them back.  t is
// split into bf16 hi + lo parts (two MFMAs per block), as in expand_body,
// and serves all NU units; every load of the wave is issued before its
// first MFMA (a wave's life is a few dependent memory round trips: kernel
// arguments and item header ~1.2 us, then its data, measured at the 70B
// q+v shape with per-wave s_memrealtime stamps).
// Needs: 16-byte aligned y with every slice's columns a multiple of 16 wide
// at a multiple of 8, the partials' row width a multiple of 8, and slots
// whose max_rank is a multiple of 8 or (POOL) every slice in a pool.
// 64-column units per wave.  One: the waves are co-resident and wait on
// memory, so more of them in flight beats more loads per wave (4 units at
// the 70B q+v shape: 14.3 -> 22.7 us); 80 VGPRs give six waves per SIMD.
// A workgroup's ITEMS waves take as many consecutive items over the same
// columns: items of one adapter are consecutive, so they read the same B_s
// rows and all but the first find them in the CU's cache (B loads were the
// largest part of this kernel's time: 14.3 -> 9.8 us without them).  Eight
// items per workgroup where the slots' padded B lines are shared and the
// grid still fills the CUs twice over (measured: 70B q+v 13.0 -> 12.3 us;
// with fewer workgroups, decode-4096 5.5 -> 5.9 us, and with a pool's
// single-item adapters, paged pool 26.0 -> 27.3 us), else four.
constexpr int kW16Units = 1;
constexpr int kW16Cols = 64 * kW16Units;        // columns per workgroup
template <int RMX, bool POOL, int ITEMS>
__global__ __launch_bounds__(64 * ITEMS) __attribute__((amdgpu_waves_per_eu(6))) void k_expand_w16(LoraArgs a) {
  constexpr int kW16Items = ITEMS;  // items per workgroup (one per wave)
  constexpr int NU = kW16Units;
  const int ncb = a.col_blk[a.n_slices];  // kW16Cols-column blocks over all slices
  const int per_xcd = (ncb + 7) >> 3;
  const int b = blockIdx.x;
  const int q = b >> 3;
  const int igrp = q / per_xcd;
  const int xcd = b & 7;
  const int cbk = ((xcd * ncb) >> 3) + (q - igrp * per_xcd);
  if (cbk >= (((xcd + 1) * ncb) >> 3)) return;
  const int item = igrp * kW16Items + (threadIdx.x >> 6);
  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  // the item's record is read beside the count, at an index clamped to the
  // list's capacity (the last group may reach past it)
  const int itc = min(item, (int)a.L.items_g_cap - 1);
  const Item it = reinterpret_cast<const Item *>(a.ws + a.L.items_g)[itc];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + itc;
  if (item >= hdr[kHdrItemsGather]) return;
  int slice = 0;
  while (slice + 1 < a.n_slices && cbk >= a.col_blk[slice + 1]) ++slice;
  const SliceRef &sl = a.sl[slice];
  const int r = ix->r[slice];
  if (r == 0) return;
  const int lane = threadIdx.x & 63;
  // the wave's columns: NU units of 64 starting at nw
  const int64_t nw = (int64_t)(cbk - a.col_blk[slice]) * kW16Cols;
  if (nw >= sl.d) return;  // uniform: no barrier follows
  const int rl = lane & 15;  // y row of the item this lane updates
  const int g = lane >> 4;   // its rank group (operands) and column group (result)
  const bool rowok = rl < it.nrows;
  const int row = ix->rows[rowok ? rl : 0];
  uint16_t *yrow = reinterpret_cast<uint16_t *>(a.y) + sl.col0 + (int64_t)row * a.ldy;
  // y first (it depends on nothing else): the lane's 16 columns of each unit
  uint4 yv[NU][2];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int64_t nc = nw + u * 64 + 16 * g;
    const uint16_t *yp = yrow + (nc < sl.d ? nc : nw);
    yv[u][0] = *reinterpret_cast<const uint4 *>(yp);
    yv[u][1] = *reinterpret_cast<const uint4 *>(yp + 8);
  }
  const int kp = (r + 31) & ~31;  // ranks padded to the MFMA k step

  // A operand: B_s rows of the permuted columns, ranks ks*32 + 8g .. + 7
  const AdapterRef &ar = sl.ar;
  const int cm = (rl >> 2) * 16 + (rl & 3);
  bf16x8_t fa[RMX / 32][NU][4];
#pragma unroll
  for (int ks = 0; ks < RMX / 32; ++ks) {
    if (ks > 0 && ks * 32 >= kp) break;  // uniform
    const int j = ks * 32 + 8 * g;
    const bool jok = j < r;
    const int ja = jok ? j : 0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int64_t n = nw + u * 64 + cm + 4 * cb;
        const bool nok = n < sl.d;
        const int64_t na = nok ? n : nw;
        bf16x8_t v;
        if constexpr (POOL) {
          if ((r & 7) == 0) {
            // r % 8 == 0: the 16-byte vector never straddles a page
            const int64_t off = ((int64_t)r * ar.k + na * r + ja) * 2;
            const int64_t page =
                ar.page_table[(int64_t)it.adapter * ar.max_pages + (off >> ar.page_shift)];
            v = ld16(ar.pool + (page << ar.page_shift) + (off & (ar.page_bytes - 1)));
          } else if ((r & 3) == 0) {
            // r % 4 == 0: two 8-byte halves, each 8-byte aligned (so inside
            // one page); a half past the rank reads the first one again
            uint2 hv[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int jh = (jok && j + 4 * hh < r) ? j + 4 * hh : ja;
              const int64_t off = ((int64_t)r * ar.k + na * r + jh) * 2;
              const int64_t page =
                  ar.page_table[(int64_t)it.adapter * ar.max_pages + (off >> ar.page_shift)];
              hv[hh] = *reinterpret_cast<const uint2 *>(ar.pool + (page << ar.page_shift) +
                                                        (off & (ar.page_bytes - 1)));
            }
            v = __builtin_bit_cast(bf16x8_t, make_uint4(hv[0].x, hv[0].y, hv[1].x, hv[1].y));
          } else {
            uint16_t e8[8];
#pragma unroll
            for (int w = 0; w < 8; ++w)
              e8[w] = (jok && nok && j + w < r)
                          ? *reinterpret_cast<const uint16_t *>(adapter_b_ptr(ar, it.adapter, r, na, j + w))
                          : (uint16_t)0;
            v = __builtin_bit_cast(bf16x8_t, e8);
          }
        } else {
          v = ld16(ar.B + (((int64_t)it.adapter * ar.d + na) * ar.max_rank + ja) * 2);
        }
        fa[ks][u][cb] = keep_first(v, (jok && nok) ? r - j : 0);
      }
  }

  // B operand: t[row][ks*32 + 8g .. + 7] as bf16 hi + lo (zero past the
  // rank and for rows past the item)
  const bool t_by_row = a.fused_cap > 0;
  const float *tpart = reinterpret_cast<const float *>(a.ws + a.L.tpart);
  bf16x8_t th[RMX / 32], tl[RMX / 32];
#pragma unroll
  for (int ks = 0; ks < RMX / 32; ++ks) {
    if (ks > 0 && ks * 32 >= kp) break;  // uniform
    const int j = ks * 32 + 8 * g;
    const int ja = j < r ? j : 0;
    float4 v0, v1;
    if (t_by_row) {
      const float *tp = tpart + ((int64_t)row * a.n_slices + slice) * a.L.R + ja;
      v0 = *reinterpret_cast<const float4 *>(tp);
      v1 = *reinterpret_cast<const float4 *>(tp + 4);
    } else {
      // the k-split partials, summed in split order (a rolled loop: the
      // splits of 8 ranks are two float4 loads each)
      const int64_t p = it.pos + (rowok ? rl : 0);
      const float *tp = tpart + tpart_index(0, p, slice, ja, a.L.rows, a.n_slices, a.L.R);
      const int64_t split_stride = (int64_t)a.L.rows * a.n_slices * a.L.R;
      v0 = *reinterpret_cast<const float4 *>(tp);
      v1 = *reinterpret_cast<const float4 *>(tp + 4);
#pragma unroll 2
      for (int qq = 1; qq < a.ksplit; ++qq) {
        const float4 u0 = *reinterpret_cast<const float4 *>(tp + qq * split_stride);
        const float4 u1 = *reinterpret_cast<const float4 *>(tp + qq * split_stride + 4);
        v0.x += u0.x; v0.y += u0.y; v0.z += u0.z; v0.w += u0.w;
        v1.x += u1.x; v1.y += u1.y; v1.z += u1.z; v1.w += u1.w;
      }
    }
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint16_t h[8], l[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float x = (rowok && j + w < r) ? f[w] : 0.f;
      h[w] = f32_to_bf16_bits(x);
      l[w] = f32_to_bf16_bits(x - bf16_bits_to_f32(h[w]));
    }
    th[ks] = __builtin_bit_cast(bf16x8_t, h);
    tl[ks] = __builtin_bit_cast(bf16x8_t, l);
  }

  const float scale = sl.scales[it.adapter];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    f32x4_t acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RMX / 32; ++ks) {
      if (ks > 0 && ks * 32 >= kp) break;  // uniform
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][u][cb], th[ks], acc[cb], 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][u][cb], tl[ks], acc[cb], 0, 0, 0);
      }
    }
    // y += scale * D' (lane: columns nc + 4 cb + i = acc[cb][i]), rounded once
    const int64_t nc = nw + u * 64 + 16 * g;
    if (!(rowok && nc < sl.d)) continue;
    const uint16_t *o0 = reinterpret_cast<const uint16_t *>(&yv[u][0]);
    const uint16_t *o1 = reinterpret_cast<const uint16_t *>(&yv[u][1]);
    uint16_t e[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint16_t old = c < 8 ? o0[c] : o1[c - 8];
      e[c] = f32_to_bf16_bits(bf16_bits_to_f32(old) + scale * acc[c >> 2][c & 3]);
    }
    uint4 w0, w1;
    __builtin_memcpy(&w0, e, 16);
    __builtin_memcpy(&w1, e + 8, 16);
    *reinterpret_cast<uint4 *>(yrow + nc) = w0;
    *reinterpret_cast<uint4 *>(yrow + nc + 8) = w1;
  }
}

// 16-row items (decode batches).  (Capping its registers so that 4-6
// workgroups fit per CU instead of 3 measured no faster at 4 and twice as
// slow at 5-6, where it spills.)
template <bool FAST, int RMX, bool POOL>
__global__ __launch_bounds__(256) void k_expand_mfma16(LoraArgs a) {
  expand_body<16, kExpandCols16, FAST, RMX, POOL>(a);
}
// 64-row items (prefill runs): three waves per SIMD (168 VGPRs) instead of
// two (228): prefill expand 47.1 -> 44.9 us, though the fast variant spills
// a few registers
template <bool FAST, int RMX, bool POOL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_expand_mfma64(
    LoraArgs a) {
  expand_body<64, 256, FAST, RMX, POOL>(a);
}

template <int RB, bool FAST, int RMX, bool POOL>
void expand_launch(const LoraArgs &a, dim3 grid, hipStream_t st) {
  if constexpr (RB == 16)
    hipLaunchKernelGGL((k_expand_mfma16<FAST, RMX, POOL>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_expand_mfma64<FAST, RMX, POOL>), grid, dim3(256), 0, st, a);
}

template <int RB, int RMX>
void expand_mode(const LoraArgs &a, int mode, dim3 grid, hipStream_t st) {
  if (mode == 1) expand_launch<RB, true, RMX, false>(a, grid, st);
  else if (mode == 2) expand_launch<RB, true, RMX, true>(a, grid, st);
  else expand_launch<RB, false, RMX, false>(a, grid, st);
}

template <int RB>
void expand_pick(const LoraArgs &a, int mode, bool r32, dim3 grid, hipStream_t st) {
  if (r32) expand_mode<RB, 32>(a, mode, grid, st);
  else expand_mode<RB, RMAX_MFMA>(a, mode, grid, st);
}

// ---------------------------------------------------------------------------
// Shrink over LDS-staged operand tiles (one slice per workgroup, at most 4
// rank blocks).  A load instruction that gives each of 16 rows 64 bytes
// (the MFMA operand layout read straight from memory) streams gathered rows
// at ~3.3 TB/s; whole 128-byte row segments stream at twice that.  So the
// item's x rows and the adapter's A rows go to a ring of LDS stages as
// 8 rows x 128 bytes per instruction (buffer_load / global_load ... lds:
// lane l's 16 bytes land at the instruction's LDS base + 16 l; chunk c of a
// row is stored at c ^ (row & 7), so the 16 lanes that read one fragment
// column hit distinct banks), STAGES - 1 k-tiles of 64 in flight, and the
// fragments are read back with ds_read_b128.  All four waves issue loads
// (each the same count per stage, padded with loads that write zeros to a
// scratch block, so one vmcnt bound covers every wave); one barrier per
// k-tile.  64-row items: wave w owns row block w and every rank block; 16-row
// items: wave w owns rank block w.  The outputs are disjoint, so no
// cross-wave sum.  Same fp32 partials as k_shrink_mfma.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void shrink_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// wait until at most n (uniform, 0 <= n <= N) vector memory ops are in flight
template <int N>
__device__ __forceinline__ void shrink_wait_le(int n) {
  if constexpr (N == 0) {
    shrink_wait_vmcnt<0>();
  } else {
    if (n >= N) shrink_wait_vmcnt<N>();
    else shrink_wait_le<N - 1>(n);
  }
}

// 16 bytes per lane from base + off into LDS (lane l at lds + 16 l); an
// offset at or past nbytes writes zeros and reads nothing (the range check
// is per dword against nbytes, so nbytes must stay below the pad offset
// 0xFFFFFFF0 for those loads to read nothing).  (Not a template: the
// buffer-resource type exists only in device compilation.)
__device__ __forceinline__ void x_load_lds(const void *base, uint32_t nbytes, void *lds, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off,
                                           0, 0, 0);
}

// 16 bytes per lane from the lane's own address into LDS (lane l at lds + 16 l)
__device__ __forceinline__ void a_load_lds(const uint8_t *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

template <int RB, int AROWS, int STAGES>
__global__ __launch_bounds__(256) void k_shrink_dma(LoraArgs a) {
  // AROWS: A rows a stage holds (16 to 128: the launch's rank blocks per
  // workgroup, 16 rows each), so small ranks leave LDS for more stages in
  // flight.  grid.y == n_slices: slice blockIdx.y's rank blocks; grid.y ==
  // 1: every slice's (the x rows are read once for all projections).
  constexpr int STAGE = (RB + AROWS) * 128;       // bytes per k-tile of 64
  constexpr int XI = RB / 8;                      // x load instructions per stage
  constexpr int SLOTS = (XI + AROWS / 8 + 3) / 4; // most loads per wave per stage
  // output blocks per wave: 64-row items -- row block `wave` x every rank
  // block; 16-row items -- rank blocks wave, wave + 4, ...
  constexpr int NACC = RB == 64 ? AROWS / 16 : (AROWS + 63) / 64;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + 1024];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  const Item it =
      reinterpret_cast<const Item *>(a.ws + (RB == 16 ? a.L.items_g : a.L.items_s))[item];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + item;
  if (item >= hdr[RB == 16 ? kHdrItemsGather : kHdrItemsSgmv]) return;
  int rk[kMaxSlices];
  item_ranks<RB == 16>(a, ix, it.adapter, rk);
  int vlo = 0, vhi = vblock_count(a, rk);
  if (gridDim.y > 1) {
    int nbq = 0;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) {
      if (q < (int)blockIdx.y) vlo += (rk[q] + 15) >> 4;
      if (q == (int)blockIdx.y) nbq = (rk[q] + 15) >> 4;
    }
    vhi = vlo + nbq;
  }
  // <= AROWS / 16: the plan keeps ranks within max_rank, and the launch
  // sizes AROWS for the largest ranks
  const int nb = vhi - vlo;
  if (nb <= 0) return;
  const int64_t kbeg = (int64_t)blockIdx.z * a.kchunk;
  if (kbeg >= a.k) return;
  const int64_t kend = min(a.k, kbeg + a.kchunk);
  const int nkt = (int)((kend - kbeg + 63) / 64);
  const int32_t *perm = reinterpret_cast<const int32_t *>(a.ws + a.L.perm);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NI = XI + 2 * nb;            // load instructions per stage
  const int LMAX = (NI + 3) >> 2;        // per wave, every wave the same

  // Per load slot of this wave: instruction i = 4 s + wave: x rows (i < XI),
  // A rows (i < NI) or the zero-writing pad.  Each lane's source: x as a
  // byte offset from the chunk's x (k-tile 0), A as a row (ARow).
  // x's extent for the loads' range check (the host keeps it below 4 GiB - 4 KiB)
  const uint32_t xbytes = (uint32_t)(a.L.rows * a.ldx * 2);
  uint32_t xoff[SLOTS];
  ARow arow[SLOTS];
  int achunk[SLOTS];
#pragma unroll
  for (int sl = 0; sl < SLOTS; ++sl) {
    const int i = 4 * sl + wave;
    xoff[sl] = 0xFFFFFFF0u;
    arow[sl] = ARow{nullptr, nullptr, 0, 0, 0};
    achunk[sl] = 0;
    if (i < XI) {
      const int P = i * 64 + lane;
      const int row = P >> 3;
      const int c = (P & 7) ^ (row & 7);
      const int rr = min(row, it.nrows - 1);  // rows past the item: any valid row, dropped
      const int m = RB == 16 ? ix->rows[rr] : perm[it.pos + rr];
      xoff[sl] = (uint32_t)((int64_t)m * a.ldx * 2 + kbeg * 2 + c * 16);
    } else if (i < NI) {
      const int P = (i - XI) * 64 + lane;
      const int j = P >> 3;  // row of the stage's A region: block vlo + j / 16
      const int c = (P & 7) ^ (j & 7);
      int slice, jb, r;
      vblock_find(a, rk, vlo + (j >> 4), slice, jb, r);
      // ranks past r: a valid row of the adapter, results dropped
      arow[sl] = make_arow(a.sl[slice].ar, it.adapter, min(jb * 16 + (j & 15), r - 1));
      arow_resolve(arow[sl], kbeg, kend);
      achunk[sl] = c;
    }
  }

  auto issue = [&](int kt) {
    uint8_t *st = smem + (kt % STAGES) * STAGE;
    const int64_t kt0 = kbeg + (int64_t)kt * 64;
#pragma unroll
    for (int sl = 0; sl < SLOTS; ++sl) {
      if (sl >= LMAX) break;
      const int i = 4 * sl + wave;
      if (i < XI) {
        // chunks past kend read as zeros (out of the buffer)
        const int c = ((((i * 64 + lane) & 7)) ^ (((i * 64 + lane) >> 3) & 7));
        const uint32_t off = kt0 + c * 8 < kend ? xoff[sl] + (uint32_t)kt * 128u : 0xFFFFFFF0u;
        x_load_lds(a.x, xbytes, st + i * 1024, off);
      } else if (i < NI) {
        // past kend: the split's first chunk of the row (finite; its x is zero)
        int64_t kc = kt0 + achunk[sl] * 8;
        if (kc >= kend) kc = kbeg;
        a_load_lds(arow_ptr(arow[sl], kc), st + RB * 128 + (i - XI) * 1024);
      } else {
        x_load_lds(a.x, xbytes, smem + STAGES * STAGE, 0xFFFFFFF0u);
      }
    }
  };

  f32x4_t acc[NACC];
#pragma unroll
  for (int v = 0; v < NACC; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool computes = RB == 64 || wave < nb;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  const int xrow = (RB == 64 ? wave * 16 : 0) + (lane & 15);
  const int arow0 = RB + (RB == 64 ? 0 : wave * 16) + (lane & 15);
  constexpr int ASTEP = RB == 64 ? 16 : 64;  // A rows between a wave's blocks

  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkt) issue(s);
  for (int kt = 0; kt < nkt; ++kt) {
    shrink_wait_le<SLOTS * (STAGES - 2)>(LMAX * min(STAGES - 2, nkt - 1 - kt));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + STAGES - 1 < nkt) issue(kt + STAGES - 1);
    if (computes) {
      const uint32_t sb = lds0 + (kt % STAGES) * STAGE;
      typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
      u32x4v xf[2], af[2][NACC];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t pc = (uint32_t)(((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16);
        const uint32_t xa = sb + xrow * 128 + pc;
        const uint32_t aa = sb + arow0 * 128 + pc;
        asm volatile("ds_read_b128 %0, %1" : "=v"(xf[ks]) : "v"(xa));
#pragma unroll
        for (int v = 0; v < NACC; ++v)
          asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(af[ks][v]) : "v"(aa), "i"(v * ASTEP * 128));
      }
      // the fragments pass through the wait, so no MFMA reads them before
      // their LDS reads have landed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        asm volatile("" : "+v"(xf[ks]));
#pragma unroll
        for (int v = 0; v < NACC; ++v) asm volatile("" : "+v"(af[ks][v]));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int v = 0; v < NACC; ++v)
          acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xf[ks]),
                                                           __builtin_bit_cast(bf16x8_t, af[ks][v]),
                                                           acc[v], 0, 0, 0);
    }
  }

  if (!computes) return;
  float *tpart = reinterpret_cast<float *>(a.ws + a.L.tpart);
#pragma unroll
  for (int v = 0; v < NACC; ++v) {
    const int b = RB == 64 ? v : wave + 4 * v;  // block of the workgroup's list
    if (b >= nb) continue;
    int slice, jb, r;
    vblock_find(a, rk, vlo + b, slice, jb, r);
    const int j = jb * 16 + (lane & 15);
    if (j >= r) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = (RB == 64 ? wave * 16 : 0) + ((lane >> 4) << 2) + e;
      if (row < it.nrows)
        tpart[tpart_index(blockIdx.z, it.pos + row, slice, j, a.L.rows, a.n_slices, a.L.R)] = acc[v][e];
    }
  }
}

}  // namespace

int shrink_dma_rows(const LoraArgs &a, bool per_slice) {
  if (a.dtype != 1 || (uint64_t)a.L.rows * a.ldx * 2 + 4096 >= (1ull << 32)) return 0;
  int need = 0;
  for (int q = 0; q < a.n_slices; ++q) {
    const int r16 = (a.sl[q].ar.max_rank + 15) / 16 * 16;
    need = per_slice ? std::max(need, r16) : need + r16;
  }
  return need <= 16 ? 16 : need <= 32 ? 32 : need <= 64 ? 64 : need <= 128 ? 128 : 0;
}

hipError_t launch_shrink_sgmv(const LoraArgs &a, int rows_per_item, bool per_slice,
                              hipStream_t st) {
  const unsigned gy = per_slice ? (unsigned)a.n_slices : 1u;
  // the LDS-staged kernel (x addressed with 32-bit offsets from the chunk)
  if (const int arows = shrink_dma_rows(a, per_slice)) {
    const unsigned nitems = (unsigned)(rows_per_item == 16 ? a.L.items_g_cap : a.L.items_s_cap);
    dim3 grid(nitems, gy, (unsigned)a.ksplit);
    // stages: ~16-72 KiB of LDS per workgroup (fewer stages, more
    // workgroups per CU measured faster where a workgroup streams little)
    if (rows_per_item == 16) {
      if (arows == 16) hipLaunchKernelGGL((k_shrink_dma<16, 16, kShrinkStages<16, 16>>), grid, dim3(256), 0, st, a);
      else if (arows == 32) hipLaunchKernelGGL((k_shrink_dma<16, 32, kShrinkStages<16, 32>>), grid, dim3(256), 0, st, a);
      else if (arows == 64) hipLaunchKernelGGL((k_shrink_dma<16, 64, kShrinkStages<16, 64>>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_shrink_dma<16, 128, kShrinkStages<16, 128>>), grid, dim3(256), 0, st, a);
    } else {
      if (arows == 16) hipLaunchKernelGGL((k_shrink_dma<64, 16, kShrinkStages<64, 16>>), grid, dim3(256), 0, st, a);
      else if (arows == 32) hipLaunchKernelGGL((k_shrink_dma<64, 32, kShrinkStages<64, 32>>), grid, dim3(256), 0, st, a);
      else if (arows == 64) hipLaunchKernelGGL((k_shrink_dma<64, 64, kShrinkStages<64, 64>>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_shrink_dma<64, 128, kShrinkStages<64, 128>>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  // per slice: at most 4 rank blocks per workgroup (ranks <= 64)
  if (rows_per_item == 16) {
    dim3 grid((unsigned)a.L.items_g_cap, gy, (unsigned)a.ksplit);
    if (per_slice) hipLaunchKernelGGL((k_shrink_mfma<16, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_shrink_mfma<16, false>), grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)a.L.items_s_cap, gy, (unsigned)a.ksplit);
    if (per_slice) hipLaunchKernelGGL((k_shrink_mfma<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_shrink_mfma<64, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_expand_sgmv(const LoraArgs &a0, int rows_per_item, hipStream_t st) {
  const int ecb = rows_per_item == 16 ? kExpandCols16 : 256;
  LoraArgs a = a0;
  a.col_blk[0] = 0;
  for (int q = 0; q < a.n_slices; ++q)
    a.col_blk[q + 1] = a.col_blk[q] + (int32_t)((a.sl[q].d + ecb - 1) / ecb);
  // one dimension: item-major, column blocks padded to a multiple of 8
  const int64_t cb8 = ((int64_t)a.col_blk[a.n_slices] + 7) / 8 * 8;
  // mode 1: fast loads, slots; 2: fast loads, every slice in a pool; 0: generic
  bool yfast = a.y_vec != 0, slots8 = true, pooled = true;
  for (int q = 0; q < a.n_slices; ++q) {
    yfast = yfast && a.sl[q].d % 8 == 0 && a.sl[q].col0 % 8 == 0;
    slots8 = slots8 && !a.sl[q].ar.pooled && a.sl[q].ar.max_rank % 8 == 0;
    pooled = pooled && a.sl[q].ar.pooled;
  }
  const int mode = !yfast ? 0 : slots8 ? 1 : pooled ? 2 : 0;
  bool r32 = true;
  for (int q = 0; q < a.n_slices; ++q) r32 = r32 && a.sl[q].ar.max_rank <= 32;
  // decode items on independent waves where the y runs, partial rows and B
  // rows allow 16-byte accesses, and t is one split (folded into the base
  // GEMM) or a sum of few: its rolled split sum is slower than expand_body's
  // batched one past that (measured: 16 splits at the decode-4096 shape
  // 5.9 -> 7.7 us, 7 at the 70B q+v shape 16.3 -> 22.8 us; folded t at that
  // shape 16.2 -> 14.3 us, 4 splits at the paged-pool shape 28.7 -> 27.4 us)
  bool w16 = rows_per_item == 16 && yfast && (slots8 || pooled) && (a.L.R % 8) == 0 &&
             (a.fused_cap > 0 || a.ksplit <= 4);
  for (int q = 0; q < a.n_slices; ++q) w16 = w16 && a.sl[q].d % 16 == 0;
  if (w16) {
    // kW16Cols-column blocks instead of ecb
    a.col_blk[0] = 0;
    for (int q = 0; q < a.n_slices; ++q)
      a.col_blk[q + 1] = a.col_blk[q] + (int32_t)((a.sl[q].d + kW16Cols - 1) / kW16Cols);
    const int64_t wb8 = ((int64_t)a.col_blk[a.n_slices] + 7) / 8 * 8;
    auto grid_of = [&](int items) {
      return dim3((unsigned)((a.L.items_g_cap + items - 1) / items * wb8));
    };
    if (pooled) {
      if (r32) hipLaunchKernelGGL((k_expand_w16<32, true, 4>), grid_of(4), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_expand_w16<RMAX_MFMA, true, 4>), grid_of(4), dim3(256), 0, st, a);
    } else if (grid_of(8).x >= 512) {
      if (r32) hipLaunchKernelGGL((k_expand_w16<32, false, 8>), grid_of(8), dim3(512), 0, st, a);
      else hipLaunchKernelGGL((k_expand_w16<RMAX_MFMA, false, 8>), grid_of(8), dim3(512), 0, st, a);
    } else {
      if (r32) hipLaunchKernelGGL((k_expand_w16<32, false, 4>), grid_of(4), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_expand_w16<RMAX_MFMA, false, 4>), grid_of(4), dim3(256), 0, st, a);
    }
  } else if (rows_per_item == 16)
    expand_pick<16>(a, mode, r32, dim3((unsigned)(a.L.items_g_cap * cb8)), st);
  else
    expand_pick<64>(a, mode, r32, dim3((unsigned)(a.L.items_s_cap * cb8)), st);
  return hipGetLastError();
}

}  // namespace lora
