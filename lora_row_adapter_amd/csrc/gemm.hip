// gemm.hip -- base projection y = x W^T ("S-LoRA: what the paper actually
// says ...", section "Batched LoRA computation": the base term is one
// ordinary GEMM over the whole batch; "Adapter Residency ...", section "What
// the forward pass has to do differently": the base projection is the large
// shared matrix multiplication).
//
// x [M, k] and W [d, k] are both k-contiguous ("NT"), so each MFMA operand
// fragment is one 16-byte load per lane along k.
//
// bf16: CDNA4 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation.  A 256-thread
// workgroup (4 wave64s in 2 x 2) owns a 128 x 128 output tile; each wave owns
// 64 x 64 = 4 x 4 MFMA blocks.  k advances in 64-wide steps staged through LDS
// (rows padded by 16 bytes so the 16 lanes reading one fragment column hit
// distinct banks); the next step's global loads are issued before the current
// step's MFMAs.  Tiles are numbered so that the 8 XCDs each get whole column
// strips of W: consecutive workgroup ids land on different XCDs, and the
// workgroups that share one W strip share that XCD's L2.
//
// fp32: plain VALU FMA tiles (64 x 64, 4 x 4 per thread); true fp32 products.
#include "kernels.hpp"

namespace lora {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

// MFMA 16x16x32 bf16 fragment layout (CDNA3/CDNA4):
//   A (16 x 32): lane l holds row l % 16, k = 8 * (l / 16) .. +7
//   B (32 x 16): lane l holds column l % 16, k = 8 * (l / 16) .. +7
//   D (16 x 16): lane l holds column l % 16, rows 4 * (l / 16) + i, i = 0..3
__global__ __launch_bounds__(256) void k_gemm_bf16(int M, int N, int K, const uint16_t *__restrict__ x,
                                                   int64_t ldx, const uint16_t *__restrict__ W,
                                                   int64_t ldw, uint16_t *__restrict__ y,
                                                   int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

  // XCD-aware tile order: workgroup b runs on XCD b % 8.  Give each XCD a
  // contiguous run of tile columns (W strips), rows fastest inside it.
  const int nblk = tiles_m * tiles_n;
  int b = blockIdx.x;
  int t;
  if ((nblk & 7) == 0) {
    const int per_xcd = nblk >> 3;
    t = (b & 7) * per_xcd + (b >> 3);
  } else {
    t = b;
  }
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: 128 rows x 64 k = 1024 16-byte vectors per
  // operand, 4 per thread.
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + i * 256;
      const int row = v >> 3;
      const int kk = k0 + ((v & 7) << 3);
      const int gm = m0 + row;
      const int gn = n0 + row;
      uint4 za = make_uint4(0, 0, 0, 0), zb = make_uint4(0, 0, 0, 0);
      if (gm < M && kk < K) za = *reinterpret_cast<const uint4 *>(x + (int64_t)gm * ldx + kk);
      if (gn < N && kk < K) zb = *reinterpret_cast<const uint4 *>(W + (int64_t)gn * ldw + kk);
      ra[i] = za;
      rb[i] = zb;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + i * 256;
      const int row = v >> 3;
      const int c = (v & 7) << 3;
      *reinterpret_cast<uint4 *>(&As[row * LDK + c]) = ra[i];
      *reinterpret_cast<uint4 *>(&Bs[row * LDK + c]) = rb[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8_t af[4], bf[4];
      const int kc = ks + ((lane >> 4) << 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ar = wm * 64 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8_t *>(&As[ar * LDK + kc]);
        const int br = wn * 64 + i * 16 + (lane & 15);
        bf[i] = *reinterpret_cast<const bf16x8_t *>(&Bs[br * LDK + kc]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: round to bf16 (RNE) and store
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + (lane & 15);
      const int rbase = m0 + wm * 64 + i * 16 + ((lane >> 4) << 2);
      if (col < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + e;
          if (row < M) y[(int64_t)row * ldy + col] = f32_to_bf16_bits(acc[i][j][e]);
        }
      }
    }
  }
}

constexpr int FBM = 64, FBN = 64, FBK = 16;

__global__ __launch_bounds__(256) void k_gemm_f32(int M, int N, int K, const float *__restrict__ x,
                                                  int64_t ldx, const float *__restrict__ W,
                                                  int64_t ldw, float *__restrict__ y, int64_t ldy) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const int tiles_m = (M + FBM - 1) / FBM;
  const int tm = blockIdx.x % tiles_m;
  const int tn = blockIdx.x / tiles_m;
  const int m0 = tm * FBM, n0 = tn * FBN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    {
      const int row = tid >> 2;
      const int kk = k0 + ((tid & 3) << 2);
      float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
      if (m0 + row < M && kk < K) va = *reinterpret_cast<const float4 *>(x + (int64_t)(m0 + row) * ldx + kk);
      if (n0 + row < N && kk < K) vb = *reinterpret_cast<const float4 *>(W + (int64_t)(n0 + row) * ldw + kk);
      const int c = (tid & 3) << 2;
      As[c + 0][row] = va.x; As[c + 1][row] = va.y; As[c + 2][row] = va.z; As[c + 3][row] = va.w;
      Bs[c + 0][row] = vb.x; Bs[c + 1][row] = vb.y; Bs[c + 2][row] = vb.z; Bs[c + 3][row] = vb.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty + 16 * i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx + 16 * j;
      if (col < N) y[(int64_t)row * ldy + col] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm(int32_t dtype, int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                       const void *W, int64_t ldw, void *y, int64_t ldy, hipStream_t st) {
  if (M <= 0 || d <= 0) return hipSuccess;
  if (dtype == 1) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((d + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_bf16, dim3(tiles_m * tiles_n), dim3(256), 0, st, (int)M, (int)d,
                       (int)k, (const uint16_t *)x, ldx, (const uint16_t *)W, ldw, (uint16_t *)y,
                       ldy, tiles_m, tiles_n);
  } else {
    const int tiles_m = (int)((M + FBM - 1) / FBM);
    const int tiles_n = (int)((d + FBN - 1) / FBN);
    hipLaunchKernelGGL(k_gemm_f32, dim3(tiles_m * tiles_n), dim3(256), 0, st, (int)M, (int)d,
                       (int)k, (const float *)x, ldx, (const float *)W, ldw, (float *)y, ldy);
  }
  return hipGetLastError();
}

}  // namespace lora
