// lora_gather.hip -- LoRA correction for decode-sized batches (gather path).
//
// "Adapter Residency When One Replica Serves Many Fine-Tunes", section "What
// the forward pass has to do differently": the base projection covers the
// whole batch; each adapter is then applied to its own rows only, as two
// small products through a rank-r bottleneck, scaled and added.  "S-LoRA:
// ...", section "Batched LoRA computation": one launch handles every adapter
// over adapter-sorted rows, with a wavefront-level reduction.
//
// Work items come from the plan: up to 16 consecutive rows of the sorted
// permutation that share one adapter.
//
// shrink: t[p, j] = sum_k A_s[j, k] x[perm[p], k]   (j < r_s, k -> r)
//   grid (item, slice x 16-rank block, k split).  A_s[j0:j0+16, kc:kc+256] is staged
//   in LDS once per 256-wide k step and reused by the 16 rows of the item
//   (4 rows per wave).  Each lane owns 4 consecutive k and keeps 4 x 16
//   partial sums (bf16 pairs through v_dot2_f32_bf16, fp32 through FMA); the
//   64 lanes are then combined by a butterfly reduce-scatter that leaves
//   output (row = lane / 16, rank = lane % 16) in lane `lane`.  Each k split
//   writes its own fp32 partial; no atomics.
// expand: y[perm[p], n] += scale_s * sum_j B_s[n, j] t[p, j]   (r -> d)
//   grid (item, 512-column block of any slice).  The k-split partials of the
//   item's rows are summed in split order into LDS, then each thread owns
//   two columns and
//   all rows of the item: acc = sum_j B t in fp32, then y = y + scale * acc
//   rounded once.  Rows without an adapter are never touched.
#include "kernels.hpp"

namespace lora {

namespace {

constexpr int KSTEP = 256;   // k per LDS stage
constexpr int JB = 16;       // ranks per shrink workgroup
constexpr int RPW = 4;       // rows per wave in the shrink
constexpr int ECOLS = 512;   // columns per expand workgroup

template <int DT>
struct Elem;
template <>
struct Elem<0> {
  using T = float;
  static constexpr int bytes = 4;
};
template <>
struct Elem<1> {
  using T = uint16_t;
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float load_f32(const float *p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t *p) { return bf16_bits_to_f32(*p); }

// One halving step of the butterfly reduce-scatter: lanes whose bit HALF is
// set keep the upper half of their values, the others the lower half, and
// each adds its partner's copy of the half it keeps.
template <int HALF>
__device__ __forceinline__ void butterfly_step(float (&v)[64], int lane) {
  const bool hi = (lane & HALF) != 0;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float send = hi ? v[i] : v[i + HALF];
    const float keep = hi ? v[i + HALF] : v[i];
    v[i] = keep + __shfl_xor(send, HALF, 64);
  }
  if constexpr (HALF > 1) butterfly_step<HALF / 2>(v, lane);
}

// 64 values per lane -> lane l returns the 64-lane sum of value l.
__device__ __forceinline__ float butterfly_reduce_scatter64(float (&v)[64], int lane) {
  butterfly_step<32>(v, lane);
  return v[0];
}

template <int DT>
__global__ __launch_bounds__(256) void k_shrink_gather(LoraArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int ROWB = KSTEP * EB + 16;  // padded LDS row (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t As[JB * ROWB];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  // item slots exist up to the list's capacity: read them beside the count
  const Item it = reinterpret_cast<const Item *>(a.ws + a.L.items_g)[item];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + item;
  if (item >= hdr[kHdrItemsGather]) return;
  const int jblocks = (a.R + JB - 1) / JB;
  const int slice = blockIdx.y / jblocks;
  const SliceRef &sl = a.sl[slice];
  const int r = ix->r[slice];
  const int j0 = (blockIdx.y - slice * jblocks) * JB;
  if (j0 >= r) return;
  const int nj = min(JB, r - j0);
  const int64_t kbeg = (int64_t)blockIdx.z * a.kchunk;
  if (kbeg >= a.k) return;
  const int64_t kend = min(a.k, kbeg + a.kchunk);
  float *tpart = reinterpret_cast<float *>(a.ws + a.L.tpart);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const T *xb = reinterpret_cast<const T *>(a.x);

  int64_t rowoff[RPW];
  bool rowv[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int p = wave * RPW + rr;
    rowv[rr] = p < it.nrows;
    rowoff[rr] = rowv[rr] ? (int64_t)ix->rows[p] * a.ldx : 0;
  }

  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;

  constexpr int VPR = KSTEP * EB / 16;      // 16-byte vectors per staged row
  constexpr int VPT = JB * VPR / 256;       // per thread
  for (int64_t kc = kbeg; kc < kend; kc += KSTEP) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * 256;
      const int jj = v / VPR;
      const int c = v % VPR;
      const int64_t kk = kc + (int64_t)c * (16 / EB);
      uint4 val = make_uint4(0, 0, 0, 0);
      if (jj < nj && kk < kend)
        val = *reinterpret_cast<const uint4 *>(adapter_a_ptr(sl.ar, it.adapter, r, j0 + jj, kk));
      *reinterpret_cast<uint4 *>(&As[jj * ROWB + c * 16]) = val;
    }
    __syncthreads();
    const int64_t kk = kc + lane * 4;
    const bool kin = kk < kend;
    if constexpr (DT == 1) {
      uint2 xv[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        xv[rr] = make_uint2(0, 0);
        if (rowv[rr] && kin) xv[rr] = *reinterpret_cast<const uint2 *>(xb + rowoff[rr] + kk);
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const uint2 av = *reinterpret_cast<const uint2 *>(&As[jj * ROWB + lane * 8]);
        const bf16x2_t a0 = __builtin_bit_cast(bf16x2_t, av.x);
        const bf16x2_t a1 = __builtin_bit_cast(bf16x2_t, av.y);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          float s = acc[rr * JB + jj];
          s = __builtin_amdgcn_fdot2_f32_bf16(a0, __builtin_bit_cast(bf16x2_t, xv[rr].x), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(a1, __builtin_bit_cast(bf16x2_t, xv[rr].y), s, false);
          acc[rr * JB + jj] = s;
        }
      }
    } else {
      float4 xv[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        xv[rr] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rowv[rr] && kin) xv[rr] = *reinterpret_cast<const float4 *>(xb + rowoff[rr] + kk);
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const float4 av = *reinterpret_cast<const float4 *>(&As[jj * ROWB + lane * 16]);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          float s = acc[rr * JB + jj];
          s = fmaf(av.x, xv[rr].x, s);
          s = fmaf(av.y, xv[rr].y, s);
          s = fmaf(av.z, xv[rr].z, s);
          s = fmaf(av.w, xv[rr].w, s);
          acc[rr * JB + jj] = s;
        }
      }
    }
  }

  const float sum = butterfly_reduce_scatter64(acc, lane);
  const int rr = lane >> 4;
  const int jj = lane & 15;
  if (rowv[rr] && jj < nj) {
    const int64_t p = it.pos + wave * RPW + rr;
    tpart[tpart_index(blockIdx.z, p, slice, j0 + jj, a.L.rows, a.n_slices, a.L.R)] = sum;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_expand_gather(LoraArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int VEC = 16 / EB;  // elements per 16-byte vector
  __shared__ __attribute__((aligned(16))) float ts[kRowsPerGatherItem * kMaxRank];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.L.hdr);
  const int item = blockIdx.x;
  const Item it = reinterpret_cast<const Item *>(a.ws + a.L.items_g)[item];
  const ItemRows *ix = reinterpret_cast<const ItemRows *>(a.ws + a.L.items_gx) + item;
  if (item >= hdr[kHdrItemsGather]) return;
  int slice = 0;
  while (slice + 1 < a.n_slices && (int)blockIdx.y >= a.col_blk[slice + 1]) ++slice;
  const SliceRef &sl = a.sl[slice];
  const int r = ix->r[slice];
  if (r == 0) return;
  const int nr = it.nrows;
  const float *tpart = reinterpret_cast<const float *>(a.ws + a.L.tpart);
  const int tid = threadIdx.x;

  const int r4 = (r + 3) >> 2;  // float4 runs per row
  for (int idx = tid; idx < nr * r4; idx += 256) {
    const int row = idx / r4;
    const int j = (idx - row * r4) * 4;
    float4 v = tpart_sum4(tpart, it.pos + row, slice, j, a.ksplit, a.L.rows, a.n_slices, a.L.R);
    // entries past the rank are never written by the shrink
    if (j + 1 >= r) v.y = 0.f;
    if (j + 2 >= r) v.z = 0.f;
    if (j + 3 >= r) v.w = 0.f;
    *reinterpret_cast<float4 *>(&ts[row * kMaxRank + j]) = v;
  }
  __syncthreads();

  const int64_t n = (int64_t)(blockIdx.y - a.col_blk[slice]) * ECOLS + 2 * tid;
  if (n >= sl.d) return;
  const bool c1 = n + 1 < sl.d;
  float acc[kRowsPerGatherItem][2];
#pragma unroll
  for (int i = 0; i < kRowsPerGatherItem; ++i) acc[i][0] = acc[i][1] = 0.f;

  // 16-byte vector loads of B rows where the row start is 16-byte aligned.
  const AdapterRef &ar = sl.ar;
  const bool vec_ok = ar.pooled ? ((r * EB) % 16 == 0) : ((ar.max_rank * EB) % 16 == 0);
  const int jv = vec_ok ? (r / VEC) * VEC : 0;
  const T *b0p = reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, n, 0));
  const T *b1p = c1 ? reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, n + 1, 0)) : b0p;
  for (int j = 0; j < jv; j += VEC) {
    // a pooled row may continue on another page: translate each vector
    const T *p0 = ar.pooled ? reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, n, j)) : b0p + j;
    const T *p1 = ar.pooled ? reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, c1 ? n + 1 : n, j))
                            : b1p + j;
    const uint4 u0 = *reinterpret_cast<const uint4 *>(p0);
    const uint4 u1 = c1 ? *reinterpret_cast<const uint4 *>(p1) : make_uint4(0, 0, 0, 0);
    float bv0[VEC], bv1[VEC];
    if constexpr (DT == 1) {
      const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w};
      const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bv0[2 * q] = __uint_as_float(w0[q] << 16);
        bv0[2 * q + 1] = __uint_as_float(w0[q] & 0xffff0000u);
        bv1[2 * q] = __uint_as_float(w1[q] << 16);
        bv1[2 * q + 1] = __uint_as_float(w1[q] & 0xffff0000u);
      }
    } else {
      bv0[0] = __uint_as_float(u0.x); bv0[1] = __uint_as_float(u0.y);
      bv0[2] = __uint_as_float(u0.z); bv0[3] = __uint_as_float(u0.w);
      bv1[0] = __uint_as_float(u1.x); bv1[1] = __uint_as_float(u1.y);
      bv1[2] = __uint_as_float(u1.z); bv1[3] = __uint_as_float(u1.w);
    }
#pragma unroll
    for (int row = 0; row < kRowsPerGatherItem; ++row) {
      if (row < nr) {
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
          const float tv = ts[row * kMaxRank + j + q];
          acc[row][0] = fmaf(bv0[q], tv, acc[row][0]);
          acc[row][1] = fmaf(bv1[q], tv, acc[row][1]);
        }
      }
    }
  }
  for (int j = jv; j < r; ++j) {
    const float bv0 = load_f32(reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, n, j)));
    const float bv1 = c1 ? load_f32(reinterpret_cast<const T *>(adapter_b_ptr(ar, it.adapter, r, n + 1, j))) : 0.f;
#pragma unroll
    for (int row = 0; row < kRowsPerGatherItem; ++row) {
      if (row < nr) {
        const float tv = ts[row * kMaxRank + j];
        acc[row][0] = fmaf(bv0, tv, acc[row][0]);
        acc[row][1] = fmaf(bv1, tv, acc[row][1]);
      }
    }
  }

  // y += scale * acc: all of this thread's y values are loaded before any
  // is stored (a store could alias a later load, which would otherwise
  // serialise every read-modify-write on the load latency)
  const float scale = sl.scales[it.adapter];
  T *yb = reinterpret_cast<T *>(a.y) + sl.col0;
  T *yr[kRowsPerGatherItem];
  T y0[kRowsPerGatherItem], y1[kRowsPerGatherItem];
#pragma unroll
  for (int row = 0; row < kRowsPerGatherItem; ++row) {
    yr[row] = row < nr ? yb + (int64_t)ix->rows[row] * a.ldy + n : nullptr;
    y0[row] = yr[row] ? yr[row][0] : T(0);
    y1[row] = (yr[row] && c1) ? yr[row][1] : T(0);
  }
#pragma unroll
  for (int row = 0; row < kRowsPerGatherItem; ++row) {
    if (yr[row] == nullptr) continue;
    if constexpr (DT == 1) {
      yr[row][0] = f32_to_bf16_bits(bf16_bits_to_f32(y0[row]) + scale * acc[row][0]);
      if (c1) yr[row][1] = f32_to_bf16_bits(bf16_bits_to_f32(y1[row]) + scale * acc[row][1]);
    } else {
      yr[row][0] = y0[row] + scale * acc[row][0];
      if (c1) yr[row][1] = y1[row] + scale * acc[row][1];
    }
  }
}

}  // namespace

hipError_t launch_shrink_gather(const LoraArgs &a, hipStream_t st) {
  dim3 grid((unsigned)a.L.items_g_cap, (unsigned)(a.n_slices * ((a.R + JB - 1) / JB)),
            (unsigned)a.ksplit);
  if (a.dtype == 1)
    hipLaunchKernelGGL(k_shrink_gather<1>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_shrink_gather<0>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_expand_gather(const LoraArgs &a0, hipStream_t st) {
  LoraArgs a = a0;
  a.col_blk[0] = 0;
  for (int q = 0; q < a.n_slices; ++q)
    a.col_blk[q + 1] = a.col_blk[q] + (int32_t)((a.sl[q].d + ECOLS - 1) / ECOLS);
  dim3 grid((unsigned)a.L.items_g_cap, (unsigned)a.col_blk[a.n_slices]);
  if (a.dtype == 1)
    hipLaunchKernelGGL(k_expand_gather<1>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_expand_gather<0>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
