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
//   grid (item, slice, k split).  16 x 16 output blocks (rows x ranks) on
//   v_mfma_f32_16x16x32_bf16; x rows are gathered through perm straight into
//   the A operand (16 bytes per lane), A_s rows into the B operand.  The 4
//   waves take alternate 32-wide k steps of the split; their partial blocks
//   are summed in wave order through LDS.  Output: fp32 partials, one per k
//   split (summed in split order by the expand).
// expand: y[perm[p], n] += scale_s * sum_j B_s[n, j] t[p, j]
//   grid (item, 256-column block of any slice).  t (the sum of the k-split
//   partials, in split order) is split into bf16 hi + lo parts (t = hi + lo to ~16 mantissa
//   bits), so two MFMAs per block keep t's precision; B_s rows feed the B
//   operand (ranks are contiguous in both slot and pool layouts).  Then
//   y = y + scale * acc, rounded once.  Rows without an adapter are never
//   touched.
#include "kernels.hpp"

namespace lora {

namespace {

constexpr int ECB = 256;      // columns per expand workgroup
constexpr int RMAX_MFMA = 64; // largest max_rank these kernels take

__device__ __forceinline__ bf16x8_t ld16(const void *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

__device__ __forceinline__ bf16x8_t zero8() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
}

template <int RB>
__global__ __launch_bounds__(256) void k_shrink_mfma(LoraArgs a) {
  constexpr int RBK = RB / 16;
  __shared__ f32x4_t red[4][RBK * 4][64];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  if (item >= hdr[RB == 16 ? kHdrItemsGather : kHdrItemsSgmv]) return;
  const Item it =
      reinterpret_cast<const Item *>(a.ws + (RB == 16 ? a.L.items_g : a.L.items_s))[item];
  const int slice = blockIdx.y;
  const SliceRef &sl = a.sl[slice];
  const int r = sl.ranks[it.adapter];
  if (r == 0) return;
  const int64_t kbeg = (int64_t)blockIdx.z * a.kchunk;
  if (kbeg >= a.k) return;
  const int64_t kend = min(a.k, kbeg + a.kchunk);
  const int32_t *perm = reinterpret_cast<const int32_t *>(a.ws + a.L.perm);
  float *tpart = reinterpret_cast<float *>(a.ws + a.L.tpart);
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(a.x);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kl = (lane >> 4) * 8;

  int64_t xoff[RBK];
  bool xv[RBK];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const int row = rb * 16 + (lane & 15);
    xv[rb] = row < it.nrows;
    xoff[rb] = xv[rb] ? (int64_t)perm[it.pos + row] * a.ldx : 0;
  }

  const int JB = (r + 15) / 16;
  for (int jg = 0; jg < JB; jg += 4) {
    f32x4_t acc[RBK][4];
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) acc[rb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int jrow[4];
    bool jv[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      jrow[jb] = (jg + jb) * 16 + (lane & 15);
      jv[jb] = jrow[jb] < r;
    }
    // U k-steps per round: all their loads are issued before their MFMAs
    constexpr int U = 4;
    for (int64_t kb0 = kbeg + wave * 32; kb0 < kend; kb0 += 128 * U) {
      bf16x8_t xf[U][RBK], af[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t kc = kb0 + 128 * u + kl;
        const bool kin = kc < kend;
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
          xf[u][rb] = (xv[rb] && kin) ? ld16(xb + xoff[rb] + kc) : zero8();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          af[u][jb] = (jv[jb] && kin) ? ld16(adapter_a_ptr(sl.ar, it.adapter, r, jrow[jb], kc))
                                      : zero8();
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
          for (int jb = 0; jb < 4; ++jb)
            if (jg + jb < JB)
              acc[rb][jb] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u][rb], af[u][jb], acc[rb][jb], 0, 0, 0);
    }
    __syncthreads();  // the previous group's reads of red are done
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) red[wave][rb * 4 + jb][lane] = acc[rb][jb];
    __syncthreads();
    for (int e = tid; e < RBK * 4 * 64; e += 256) {
      const int blk = e >> 6;
      const int ln = e & 63;
      const int rb = blk >> 2;
      const int jb = blk & 3;
      if (jg + jb >= JB) continue;
      const f32x4_t s = ((red[0][blk][ln] + red[1][blk][ln]) + red[2][blk][ln]) + red[3][blk][ln];
      const int j = (jg + jb) * 16 + (ln & 15);
      if (j >= r) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb * 16 + ((ln >> 4) << 2) + i;
        if (row < it.nrows)
          tpart[tpart_index(it.pos + row, slice, j, blockIdx.z, a.n_slices, a.R)] = s[i];
      }
    }
  }
}

template <int RB>
__global__ __launch_bounds__(256) void k_expand_mfma(LoraArgs a) {
  constexpr int RBK = RB / 16;
  constexpr int KP = RMAX_MFMA + 8;  // padded LDS row (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t th[RB * KP];
  __shared__ __attribute__((aligned(16))) uint16_t tl[RB * KP];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  if (item >= hdr[RB == 16 ? kHdrItemsGather : kHdrItemsSgmv]) return;
  const Item it =
      reinterpret_cast<const Item *>(a.ws + (RB == 16 ? a.L.items_g : a.L.items_s))[item];
  int slice = 0;
  while (slice + 1 < a.n_slices && (int)blockIdx.y >= a.col_blk[slice + 1]) ++slice;
  const SliceRef &sl = a.sl[slice];
  const int r = sl.ranks[it.adapter];
  if (r == 0) return;
  const int nr = it.nrows;
  const int64_t n0 = (int64_t)(blockIdx.y - a.col_blk[slice]) * ECB;
  const int32_t *perm = reinterpret_cast<const int32_t *>(a.ws + a.L.perm);
  const float *tpart = reinterpret_cast<const float *>(a.ws + a.L.tpart);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kp = (r + 31) & ~31;  // ranks padded to the MFMA k step

  // t = sum of the k-split partials, as bf16 hi + lo
  for (int e = tid; e < RB * kp; e += 256) {
    const int row = e / kp;
    const int j = e - row * kp;
    float v = 0.f;
    if (row < nr && j < r) v = tpart_sum(tpart, it.pos + row, slice, j, a.ksplit, a.n_slices, a.R);
    const uint16_t hi = f32_to_bf16_bits(v);
    const uint16_t lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
    th[row * KP + j] = hi;
    tl[row * KP + j] = lo;
  }
  __syncthreads();

  const AdapterRef &ar = sl.ar;
  const int stride = ar.pooled ? r : ar.max_rank;  // B row stride (elements)
  const bool vec_ok = (stride % 8) == 0;
  f32x4_t acc[RBK][4];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int jk = 0; jk < kp; jk += 32) {
    const int jl = jk + (lane >> 4) * 8;
    bf16x8_t fh[RBK], fl[RBK], fb[4];
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      fh[rb] = ld16(&th[(rb * 16 + (lane & 15)) * KP + jl]);
      fl[rb] = ld16(&tl[(rb * 16 + (lane & 15)) * KP + jl]);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int64_t n = n0 + (wave * 4 + cb) * 16 + (lane & 15);
      bf16x8_t v = zero8();
      if (n < sl.d && jl < r) {
        if (vec_ok && jl + 8 <= r) {
          v = ld16(adapter_b_ptr(ar, it.adapter, r, n, jl));
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
      fb[cb] = v;
    }
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh[rb], fb[cb], acc[rb][cb], 0, 0, 0);
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl[rb], fb[cb], acc[rb][cb], 0, 0, 0);
      }
  }

  // y += scale * acc: every y value of this lane is loaded before any is
  // stored (a store could alias a later load, so the compiler would
  // otherwise serialise each read-modify-write on the load latency)
  const float scale = sl.scales[it.adapter];
  uint16_t *yb = reinterpret_cast<uint16_t *>(a.y) + sl.col0;
  uint16_t *yp[RBK][4];
  uint16_t yv[RBK][4][4];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rb * 16 + ((lane >> 4) << 2) + i;
      yp[rb][i] = row < nr ? yb + (int64_t)perm[it.pos + row] * a.ldy : nullptr;
    }
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int64_t n = n0 + (wave * 4 + cb) * 16 + (lane & 15);
        yv[rb][i][cb] = (yp[rb][i] != nullptr && n < sl.d) ? yp[rb][i][n] : (uint16_t)0;
      }
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int64_t n = n0 + (wave * 4 + cb) * 16 + (lane & 15);
        if (yp[rb][i] != nullptr && n < sl.d)
          yp[rb][i][n] = f32_to_bf16_bits(bf16_bits_to_f32(yv[rb][i][cb]) + scale * acc[rb][cb][i]);
      }
}

}  // namespace

hipError_t launch_shrink_sgmv(const LoraArgs &a, int rows_per_item, hipStream_t st) {
  if (rows_per_item == 16) {
    dim3 grid((unsigned)a.L.items_g_cap, (unsigned)a.n_slices, (unsigned)a.ksplit);
    hipLaunchKernelGGL(k_shrink_mfma<16>, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)a.L.items_s_cap, (unsigned)a.n_slices, (unsigned)a.ksplit);
    hipLaunchKernelGGL(k_shrink_mfma<64>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_expand_sgmv(const LoraArgs &a0, int rows_per_item, hipStream_t st) {
  LoraArgs a = a0;
  a.col_blk[0] = 0;
  for (int q = 0; q < a.n_slices; ++q)
    a.col_blk[q + 1] = a.col_blk[q] + (int32_t)((a.sl[q].d + ECB - 1) / ECB);
  if (rows_per_item == 16) {
    dim3 grid((unsigned)a.L.items_g_cap, (unsigned)a.col_blk[a.n_slices]);
    hipLaunchKernelGGL(k_expand_mfma<16>, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)a.L.items_s_cap, (unsigned)a.col_blk[a.n_slices]);
    hipLaunchKernelGGL(k_expand_mfma<64>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lora
