// merge.hip -- the merged weight of one adapter: W' = W + c * s_a * B_a A_a.
//
// "Your LoRA Adapters Are Thrashing Your GPUs", section 02 (weight merging
// vs keeping adapters separate): merging precomputes W + (alpha/r) B A so
// inference runs the plain layer, at the price of rewriting the whole weight
// (and of serving one adapter at a time).  "Adapter Residency When One
// Replica Serves Many Fine-Tunes", "What the forward pass has to do
// differently", and "LoRA Adapters: Many Models in One", "What an adapter
// is", give the same identity.  c = +1 merges, c = -1 takes a merged
// adapter back out.
//
// The work is a rank-r update of a d x k matrix: 4 bytes of HBM traffic per
// bf16 element (read W, write W') against 2r flops, so the kernel is
// HBM-bound for every rank and is built around streaming W once:
//
//   bf16: 64 x 256 tiles; W in and W' out as whole 512-byte row segments
//     with nontemporal accesses, the rank-r product on MFMA from a transposed
//     A tile in LDS, the sum formed in LDS in the MFMA output layout (see
//     k_merge_bf16).
//   fp32: 64 x 64 tiles on the VALU (fp32 products, fp32 accumulation).
//
// Device-side errors (rank outside [0, max_rank], pool pages missing or
// outside the pool) make the kernel copy W unchanged.
#include "kernels.hpp"

namespace lora {

namespace {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t ldv16(const void *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

// Rank of adapter a if its data is usable, else 0 (W copied unchanged).
// Called by all 256 threads of the workgroup (it synchronises them).
__device__ inline int merge_rank(const MergeArgs &m) {
  const int r = m.ranks[m.adapter];
  int bad = r < 0 || r > m.ar.max_rank;
  if (!bad && m.ar.pooled && r > 0) {
    const int64_t bytes = (int64_t)r * (m.ar.k + m.ar.d) * m.ar.elem_bytes;
    const int64_t pages = (bytes + m.ar.page_bytes - 1) >> m.ar.page_shift;
    if (pages > m.ar.max_pages) {
      bad = 1;
    } else {
      const int32_t *pt = m.ar.page_table + (int64_t)m.adapter * m.ar.max_pages;
      for (int64_t j = threadIdx.x; j < pages; j += 256)
        if (pt[j] < 0 || pt[j] >= m.n_pages) bad = 1;
    }
  }
  bad = __syncthreads_or(bad);
  return bad ? 0 : r;
}

// Address of A_a[j][c] / B_a[n][j] with the storage kind fixed at compile
// time (a runtime slot/pool branch around every load would separate the
// loads into basic blocks and serialise them).  Elements of elem_bytes.
template <bool POOL>
__device__ __forceinline__ const uint8_t *a_addr(const MergeArgs &m, int r, int64_t j, int64_t c) {
  if (!POOL)
    return m.ar.A + (((int64_t)m.adapter * m.ar.max_rank + j) * m.ar.k + c) * m.ar.elem_bytes;
  (void)r;
  const int64_t off = (j * m.ar.k + c) * m.ar.elem_bytes;
  const int64_t page = m.ar.page_table[(int64_t)m.adapter * m.ar.max_pages + (off >> m.ar.page_shift)];
  return m.ar.pool + (page << m.ar.page_shift) + (off & (m.ar.page_bytes - 1));
}
template <bool POOL>
__device__ __forceinline__ const uint8_t *b_addr(const MergeArgs &m, int r, int64_t n, int64_t j) {
  if (!POOL)
    return m.ar.B + (((int64_t)m.adapter * m.ar.d + n) * m.ar.max_rank + j) * m.ar.elem_bytes;
  const int64_t off = ((int64_t)r * m.ar.k + n * r + j) * m.ar.elem_bytes;
  const int64_t page = m.ar.page_table[(int64_t)m.adapter * m.ar.max_pages + (off >> m.ar.page_shift)];
  return m.ar.pool + (page << m.ar.page_shift) + (off & (m.ar.page_bytes - 1));
}

}  // namespace

// Workgroup tile: 64 rows x 256 columns (4 waves x 16 rows).
//   1. the W tile is read with nontemporal 16-byte loads, 8 rows x 512 bytes
//      per instruction (whole row segments: measured 6.3 TB/s for a plain
//      copy in this pattern, against 2.3-4 TB/s for MFMA-layout pieces);
//   2. per 32-rank chunk, A_a[chunk, c0:c0+256] is staged in LDS transposed
//      to [column][rank] and each wave accumulates D[c][n] = sum_j At[c][j]
//      B[n][j] on v_mfma_f32_16x16x32_bf16 (16 column subtiles of 16 x 16);
//   3. the W tile goes to LDS (row pitch padded by 16 bytes so the MFMA-layout
//      accesses of 16 rows fall in different banks), each lane adds c s D to
//      its four consecutive columns of one row and rounds once;
//   4. W' leaves with nontemporal 16-byte stores in the load pattern.
constexpr int kTC = 256;             // tile columns
constexpr int kTR = 64;              // tile rows
constexpr int kAtP = 40;             // At row pitch (elements): 32 ranks + 8
constexpr int kWsP = kTC * 2 + 16;   // W tile row pitch in bytes

// Keep the first `keep` bf16 elements of a 16-byte fragment, zero the rest
// (ranks at or past r: slot padding may hold anything).  Branch-free.
__device__ __forceinline__ uint4 keep_first(uint4 u, int keep) {
  const uint32_t q[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t msk = 2 * i + 1 < keep ? 0xffffffffu : (2 * i < keep ? 0xffffu : 0u);
    o[i] = q[i] & msk;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// B fragment of row n for ranks j0 .. j0 + 7 (zero at or past r, or past d).
// Slots with 16-byte rows (max_rank % 8 == 0): one unconditional vector load
// at a clamped address, masked after; otherwise element loads.
template <bool POOL, bool BVEC>
__device__ __forceinline__ uint4 merge_bfrag(const MergeArgs &m, int r, int64_t n, int j0) {
  const bool ok = n < m.d && j0 < r;
  if (!POOL && BVEC) {
    const uint4 u = __builtin_bit_cast(
        uint4, ldv16(b_addr<POOL>(m, r, ok ? n : 0, ok ? j0 : 0)));
    return keep_first(u, ok ? r - j0 : 0);
  }
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    e[i] = ok && j0 + i < r ? *reinterpret_cast<const uint16_t *>(b_addr<POOL>(m, r, n, j0 + i)) : 0;
  return make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                    e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
}

// A vectors a thread stages for one 32-rank chunk: task v = tid + 256 q
// (q < 2) is the rank pair ch + 2 (v % 16) + {0, 1} and columns 8 (v / 16) ..
// +7 of the tile (two 16-byte loads).  Slots: loads at clamped addresses,
// zeroed after; pool: only valid vectors are translated.
template <bool POOL>
__device__ __forceinline__ void merge_aload(const MergeArgs &m, int r, int ch, int64_t c0, int ncols,
                                            uint4 (&a)[4]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int v = threadIdx.x + 256 * q;
    const int cc = (v >> 4) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = ch + 2 * (v & 15) + h;
      const bool ok = j < r && cc < ncols;
      if (!POOL) {
        const uint4 u = __builtin_bit_cast(uint4, ldv16(a_addr<POOL>(m, r, ok ? j : 0, c0 + (ok ? cc : 0))));
        a[2 * q + h] = ok ? u : make_uint4(0, 0, 0, 0);
      } else {
        a[2 * q + h] = ok ? __builtin_bit_cast(uint4, ldv16(a_addr<POOL>(m, r, j, c0 + cc)))
                          : make_uint4(0, 0, 0, 0);
      }
    }
  }
}

// At[c][jj]: each lane writes, for its 8 columns, one 32-bit word holding
// its two ranks (16 lanes of a column group hit 16 consecutive banks; odd
// column groups take the columns in a rotated order so the two half-waves
// land on different banks).
__device__ __forceinline__ void merge_astage(uint16_t *At, const uint4 (&a)[4]) {
  uint32_t *At32 = reinterpret_cast<uint32_t *>(At);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int v = threadIdx.x + 256 * q;
    const int p = v & 15, cg = v >> 4;
    const uint32_t lo[4] = {a[2 * q].x, a[2 * q].y, a[2 * q].z, a[2 * q].w};
    const uint32_t hi[4] = {a[2 * q + 1].x, a[2 * q + 1].y, a[2 * q + 1].z, a[2 * q + 1].w};
#pragma unroll
    for (int i0 = 0; i0 < 8; ++i0) {
      const int i = (i0 + 4 * (cg & 1)) & 7;
      const uint32_t e0 = (lo[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const uint32_t e1 = (hi[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      At32[((8 * cg + i) * kAtP) / 2 + p] = e0 | (e1 << 16);
    }
  }
}

template <bool POOL, bool BVEC>
__global__ __launch_bounds__(256) void k_merge_bf16(MergeArgs m) {
  __shared__ __attribute__((aligned(16))) uint16_t At[kTC * kAtP];
  __shared__ __attribute__((aligned(16))) uint8_t Ws[kTR * kWsP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NT = kTC / 16;  // 16-column subtiles per wave

  const int64_t c0 = (int64_t)blockIdx.x * kTC;
  const int64_t n0 = (int64_t)blockIdx.y * kTR;
  const int ncols = m.k - c0 < kTC ? (int)(m.k - c0) : kTC;
  const int r = merge_rank(m);
  const int rp = (r + 31) & ~31;
  const float sc = r > 0 ? m.coef * m.scales[m.adapter] : 0.f;
  const int64_t n = n0 + wave * 16 + (lane & 15);  // this lane's output row
  const int g = lane >> 4;

  // Loads complete in issue order, so what is needed first is issued first:
  // A and B of the first two rank chunks, then the W tile (8 rows x 512
  // bytes per instruction, nontemporal, at clamped addresses past the edges).
  uint4 a0[4], a1[4];
  merge_aload<POOL>(m, r, 0, c0, ncols, a0);
  merge_aload<POOL>(m, r, 32, c0, ncols, a1);
  const uint4 b0 = merge_bfrag<POOL, BVEC>(m, r, n, 8 * g);
  const uint4 b1 = merge_bfrag<POOL, BVEC>(m, r, n, 32 + 8 * g);
  const int lrow = tid >> 5, lcol = (tid & 31) * 8;
  const int lcol_c = lcol < ncols ? lcol : 0;
  u32x4_t w[kTR / 8];
#pragma unroll
  for (int i = 0; i < kTR / 8; ++i) {
    const int64_t nn = n0 + 8 * i + lrow;
    w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
        m.W + ((nn < m.d ? nn : m.d - 1) * m.ldw + c0 + lcol_c) * 2));
  }

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ch = 0; ch < rp; ch += 32) {
    uint4 bu;
    if (ch > 0) __syncthreads();  // the previous chunk's At reads are done
    if (ch == 0) {
      merge_astage(At, a0);
      bu = b0;
    } else if (ch == 32) {
      merge_astage(At, a1);
      bu = b1;
    } else {  // ranks above 64: loaded here (after the W tile)
      uint4 a2[4];
      merge_aload<POOL>(m, r, ch, c0, ncols, a2);
      merge_astage(At, a2);
      bu = merge_bfrag<POOL, BVEC>(m, r, n, ch + 8 * g);
    }
    __syncthreads();
    const bf16x8_t bfrag = __builtin_bit_cast(bf16x8_t, bu);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8_t afrag = ldv16(At + (t * 16 + (lane & 15)) * kAtP + 8 * g);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc[t], 0, 0, 0);
    }
  }

  // W tile to LDS, then each lane adds c s D to columns 16t + 4g .. +3 of row n
#pragma unroll
  for (int i = 0; i < kTR / 8; ++i)
    *reinterpret_cast<u32x4_t *>(Ws + (8 * i + lrow) * kWsP + lcol * 2) = w[i];
  __syncthreads();
  if (rp > 0) {
    uint8_t *row = Ws + (wave * 16 + (lane & 15)) * kWsP;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x2_t *p = reinterpret_cast<u32x2_t *>(row + (16 * t + 4 * g) * 2);
      const u32x2_t v = *p;
      const float x0 = __uint_as_float(v.x << 16) + sc * acc[t][0];
      const float x1 = __uint_as_float(v.x & 0xffff0000u) + sc * acc[t][1];
      const float x2 = __uint_as_float(v.y << 16) + sc * acc[t][2];
      const float x3 = __uint_as_float(v.y & 0xffff0000u) + sc * acc[t][3];
      *p = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    }
  }
  __syncthreads();
  // W' out in the load pattern
#pragma unroll
  for (int i = 0; i < kTR / 8; ++i) {
    const int64_t nn = n0 + 8 * i + lrow;
    if (nn < m.d && lcol < ncols)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(Ws + (8 * i + lrow) * kWsP + lcol * 2),
                                  reinterpret_cast<u32x4_t *>(m.Wo + (nn * m.ldo + c0 + lcol) * 2));
  }
}

// fp32: 64 columns x 64 rows per workgroup; A tile [r][64] and the B rows of
// the tile in LDS (ranks in chunks of 64); thread (ty, tx) owns rows
// ty + 16 i (i < 4) and columns 4 tx .. 4 tx + 3.
__global__ __launch_bounds__(256) void k_merge_f32(MergeArgs m) {
  __shared__ float As[64][64 + 4];   // [rank][column]
  __shared__ float Bs[64][64 + 1];   // [row][rank]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t n0 = (int64_t)blockIdx.y * 64;
  const int r = merge_rank(m);
  const float sc = r > 0 ? m.coef * m.scales[m.adapter] : 0.f;
  float acc[4][4] = {};
  for (int j0 = 0; j0 < r; j0 += 64) {
    __syncthreads();
    for (int v = tid; v < 64 * 64; v += 256) {
      const int j = v >> 6, c = v & 63;
      As[j][c] = (j0 + j < r && c0 + c < m.k)
                     ? *reinterpret_cast<const float *>(m.ar.pooled ? a_addr<true>(m, r, j0 + j, c0 + c)
                                                                 : a_addr<false>(m, r, j0 + j, c0 + c))
                     : 0.f;
      const int rr = v >> 6, jj = v & 63;
      Bs[rr][jj] = (j0 + jj < r && n0 + rr < m.d)
                       ? *reinterpret_cast<const float *>(m.ar.pooled ? b_addr<true>(m, r, n0 + rr, j0 + jj)
                                                                 : b_addr<false>(m, r, n0 + rr, j0 + jj))
                       : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < 64; ++j) {
      float b[4], a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = Bs[ty + 16 * i][j];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = As[j][4 * tx + q];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(b[i], a[q], acc[i][q]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + ty + 16 * i;
    if (n >= m.d) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t c = c0 + 4 * tx + q;
      if (c >= m.k) continue;
      const float w = *reinterpret_cast<const float *>(m.W + (n * m.ldw + c) * 4);
      *reinterpret_cast<float *>(m.Wo + (n * m.ldo + c) * 4) = r > 0 ? w + sc * acc[i][q] : w;
    }
  }
}

hipError_t launch_merge(const MergeArgs &m, hipStream_t st) {
  if (m.dtype == 1) {
    const dim3 grid((unsigned)((m.k + kTC - 1) / kTC), (unsigned)((m.d + kTR - 1) / kTR));
    if (m.ar.pooled)
      hipLaunchKernelGGL((k_merge_bf16<true, false>), grid, dim3(256), 0, st, m);
    else if ((m.ar.max_rank & 7) == 0)
      hipLaunchKernelGGL((k_merge_bf16<false, true>), grid, dim3(256), 0, st, m);
    else
      hipLaunchKernelGGL((k_merge_bf16<false, false>), grid, dim3(256), 0, st, m);
  } else {
    const dim3 grid((unsigned)((m.k + 63) / 64), (unsigned)((m.d + 63) / 64));
    hipLaunchKernelGGL(k_merge_f32, grid, dim3(256), 0, st, m);
  }
  return hipGetLastError();
}

}  // namespace lora
