// gemm_q.hip -- base projection with a quantized base weight:
//   y = x W^T,  W = dequant(q)       x bf16 [M, k], y bf16 [M, d]
//
// "Your LoRA Adapters Are Thrashing Your GPUs", section 02 (INT4 / INT8 base
// weights with adapters kept in 16 bits): production deployments quantize
// the base model and keep the LoRA matrices in 16-bit floats.  Formats
// (the pages name only the bit widths; these are the plain symmetric
// readings):
//   INT8: q int8 [d, k], one fp32 scale per output row: W[n, k] = s[n] q[n, k]
//   INT4: q two's-complement nibbles, two per byte (element 2i in the low
//         nibble), one fp32 scale per output row and k-group of `group`
//         elements: W[n, k] = s[n, k / group] q[n, k]
//
// Kernel: the bf16 pipeline GEMM's structure (4-stage ring of k-tiles of 64,
// operands streamed HBM -> LDS by buffer_load ... lds, XCD-aware tile order,
// MFMA 16x16x32 bf16, fp32 accumulation), except that the W stage holds the
// packed integers (half or a quarter of the bf16 bytes: the decode-sized GEMM
// is bound by the bytes each CU streams, so this is where the gain is).
// Once per k-tile all 256 threads convert the packed tile into a bf16 tile
// (two LDS buffers, so a single barrier per k-tile still orders everything):
//   INT8: exact integers (|q| <= 128 is exact in bf16); the row scale is
//         applied to the fp32 accumulator in the epilogue (exact W).
//   INT4: q * s rounded once to bf16 (the group scale cannot be factored out
//         of the whole k sum).
#include "kernels.hpp"

namespace lora {

namespace {

template <int N>
__device__ __forceinline__ void q_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void q_load_lds(const void *base, uint32_t nbytes, void *lds,
                                           uint32_t voff, int size) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                             voff, 0, 0, 0);
}

// LDS reads of the packed stage.  The compiler cannot tell that these
// addresses were filled by a DMA that the explicit vmcnt waits and the
// barrier have already completed, and would put a wait for every load in
// flight (the prefetched stages too) before each one.  So a thread's reads
// of one tile (up to three 16-byte chunks) and their lgkmcnt wait are one
// asm statement: nothing can read the results before the wait.
template <int NCH>
__device__ __forceinline__ void lds_read_chunks(const uint8_t *const (&p)[3], uint4 (&v)[3]) {
  uint32_t a[3];
#pragma unroll
  for (int i = 0; i < 3; ++i)
    a[i] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p[i];
  if constexpr (NCH == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a[0]));
  } else if constexpr (NCH == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(a[0]), "v"(a[1]));
  } else {
    asm volatile(
        "ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]));
  }
}
// ... and the stores of the bf16 tile, for the same reason (the compiler
// would wait for every DMA in flight before each one).  Their completion is
// waited for explicitly before the barrier that publishes the tile.
typedef uint32_t q_u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_write16(void *p, uint4 v) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)p;
  const q_u32x4_t w = {v.x, v.y, v.z, v.w};
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(w) : "memory");
}
__device__ __forceinline__ void lds_writes_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

#ifndef LORA_Q_PRODUCER_WAVES
#define LORA_Q_PRODUCER_WAVES 8
#endif
constexpr int kQProducerWaves = LORA_Q_PRODUCER_WAVES;  // 4 or 8

// FMT 1: INT8 (64 bytes per row per k-tile), 2: INT4 (32 bytes).
//
// 512 threads in two roles (one wave of each on every SIMD):
//   producers (waves 4-7): issue the DMA loads of the stages, wait for them,
//     and convert the packed tile kt + 1 into bf16 while ...
//   consumers (waves 0-3): run the MFMAs of tile kt and hold the accumulators.
// One barrier per k-tile: before it the producers have tile kt + 1 resident
// and the bf16 tile kt written; after it the consumers are done with tile
// kt - 1, so its stage and bf16 buffer may be refilled.
template <int BM, int BN, int WM, int WN, int STAGES, int FMT, int NPW>
__global__ __launch_bounds__(256 + 64 * NPW) void k_gemm_q_pipe(QGemmArgs p) {
  constexpr int NPT = 64 * NPW;                       // producer threads (the first 256 issue the DMA)
  constexpr int QB = FMT == 1 ? 64 : 32;              // packed bytes per row per k-tile
  constexpr int QCPR = QB / 16;                       // 16-byte chunks per packed row
  constexpr int QROWS = ((BN * QCPR + 255) / 256) * 256 / QCPR;  // rows loaded (whole instrs)
  constexpr int Q_INSTR = QROWS * QCPR / 256;         // packed loads per producer thread per k-tile
  constexpr int A_INSTR = BM * 8 / 256;               // x loads per producer thread per k-tile
  constexpr int S_INSTR = FMT == 2 ? (BN + 255) / 256 : 0;  // scale loads (INT4)
  constexpr int LOADS = A_INSTR + Q_INSTR + S_INSTR;
  constexpr int BKB = 128;                            // bf16 bytes per row per k-tile
  constexpr int A_BYTES = BM * BKB;
  constexpr int Q_BYTES = QROWS * QB;
  constexpr int S_BYTES = S_INSTR * 4 * 256;         // 4 waves x S_INSTR x 64 lanes x 4 bytes
  constexpr int STAGE_BYTES = A_BYTES + Q_BYTES + S_BYTES;
  constexpr int BT_BYTES = BN * BKB;                  // one dequantized W tile
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int CLD = BN + 8;
  static_assert(WM * WN == 4, "4 consumer waves");
  static_assert(FM * WM * 16 == BM && FN * WN * 16 == BN, "tile split");
  static_assert(STAGES >= 3, "the dequant pass reads one stage ahead");
  constexpr int SMEM = STAGES * STAGE_BYTES + 2 * BT_BYTES;
  static_assert(SMEM >= BM * CLD * 2, "epilogue fits");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  uint8_t *bt_base = smem + STAGES * STAGE_BYTES;

  const int b = blockIdx.x;
  const int nblk = p.tiles_m * p.tiles_n;
  const int t = ((nblk & 7) == 0) ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int tm = t % p.tiles_m;
  const int tn = t / p.tiles_m;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int nrows = min(BN, p.N - n0);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool producer = wave >= 4;
  const int pw = wave - 4;                // producer wave 0 .. NPW - 1
  const int ptid = threadIdx.x - 256;     // producer thread 0 .. NPT - 1
  const bool loader = producer && pw < 4; // producer waves that issue and wait for the DMA

  const uint32_t a_bytes = (uint32_t)(min(BM, p.M - m0) * p.ldx * 2);
  const uint32_t q_bytes = (uint32_t)(nrows * p.ldq);
  const uint16_t *xa = p.x + (int64_t)m0 * p.ldx;
  const uint8_t *qb = p.q + (int64_t)n0 * p.ldq;
  const float *sb = p.scales + (int64_t)n0 * p.ngroups;  // INT4 group scales of the tile rows
  const uint32_t s_bytes = (uint32_t)(nrows * p.ngroups * 4);
  const int nk = p.K / 64;

  // ----- producer state: source offsets (x swizzled as in the bf16
  // pipeline; packed chunk P = row * QCPR + c lands at P * 16) -----
  uint32_t va[A_INSTR], vq[Q_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int P = (pw * A_INSTR + i) * 64 + lane;
    const int row = P >> 3;
    const int c = (P & 7) ^ (row & 7);
    va[i] = (uint32_t)(row * p.ldx * 2 + c * 16);
  }
#pragma unroll
  for (int i = 0; i < Q_INSTR; ++i) {
    const int P = (pw * Q_INSTR + i) * 64 + lane;
    const int row = P / QCPR;
    const int c = P % QCPR;
    vq[i] = row < BN ? (uint32_t)(row * p.ldq + c * 16) : 0xFFFFFFF0u;
  }
  auto issue = [&](int kt, int stage) {
    uint8_t *sa = smem + stage * STAGE_BYTES;
    uint8_t *sq = sa + A_BYTES;
    const uint32_t kb = (uint32_t)kt * BKB;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      q_load_lds(xa, a_bytes, sa + (pw * A_INSTR + i) * 1024, va[i] + kb, 16);
    const uint32_t kq = (uint32_t)kt * QB;
#pragma unroll
    for (int i = 0; i < Q_INSTR; ++i)
      q_load_lds(qb, q_bytes, sq + (pw * Q_INSTR + i) * 1024,
                 vq[i] == 0xFFFFFFF0u ? vq[i] : vq[i] + kq, 16);
    if constexpr (FMT == 2) {
      // scale of row (lane + 64 * i) for this k-tile's group: 4 bytes per lane
      float *ss = reinterpret_cast<float *>(sq + Q_BYTES);
      const int g = (kt * 64) / p.group;
#pragma unroll
      for (int i = 0; i < S_INSTR; ++i) {
        const int row = (pw * S_INSTR + i) * 64 + lane;
        const uint32_t off = row < BN ? (uint32_t)((row * p.ngroups + g) * 4) : 0xFFFFFFF0u;
        q_load_lds(sb, s_bytes, ss + (pw * S_INSTR + i) * 64, off, 4);
      }
    }
  };
  // Packed tile of stage `stage` -> bf16 tile `buf` (row r, chunk c of 8
  // values at c ^ (r & 7), as the MFMA loop reads it).
  auto dequant = [&](int stage, int buf) {
    const uint8_t *sq = smem + stage * STAGE_BYTES + A_BYTES;
    uint8_t *bt = bt_base + buf * BT_BYTES;
    if constexpr (FMT == 1) {
      // one 16-byte packed chunk = 16 k values = two bf16 chunks; chunk
      // P = ptid + 256 i (slots past the tile read chunk 0 and are dropped)
      constexpr int NCH = (BN * 4 + NPT - 1) / NPT;
      static_assert(NCH <= 3, "chunks per producer thread");
      const uint8_t *src[3];
      uint4 uu[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int P = ptid + NPT * i;
        src[i] = sq + (P < BN * 4 ? P : 0) * 16;
      }
      lds_read_chunks<NCH>(src, uu);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int P = ptid + NPT * i;
        if (P >= BN * 4) continue;
        const int row = P >> 2, c = P & 3;
        const uint32_t w[4] = {uu[i].x, uu[i].y, uu[i].z, uu[i].w};
        uint32_t o[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          o[2 * h] = pack_bf16x2((float)(int8_t)(w[h] & 0xff), (float)(int8_t)((w[h] >> 8) & 0xff));
          o[2 * h + 1] = pack_bf16x2((float)(int8_t)((w[h] >> 16) & 0xff), (float)(int8_t)(w[h] >> 24));
        }
        uint8_t *dst = bt + row * BKB;
        lds_write16(dst + (((2 * c) ^ (row & 7)) * 16), make_uint4(o[0], o[1], o[2], o[3]));
        lds_write16(dst + (((2 * c + 1) ^ (row & 7)) * 16), make_uint4(o[4], o[5], o[6], o[7]));
      }
    } else {
      // one 16-byte packed chunk = 32 k values = four bf16 chunks
      const float *ss = reinterpret_cast<const float *>(sq + Q_BYTES);
      constexpr int NCH = (BN * 2 + NPT - 1) / NPT;
      static_assert(NCH <= 3, "chunks per producer thread");
      const uint8_t *src[3];
      uint4 uu[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int P = ptid + NPT * i;
        src[i] = sq + (P < BN * 2 ? P : 0) * 16;
      }
      lds_read_chunks<NCH>(src, uu);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int P = ptid + NPT * i;
        if (P >= BN * 2) continue;
        const int row = P >> 1, c = P & 1;
        const float s = ss[row];
        const uint32_t w[4] = {uu[i].x, uu[i].y, uu[i].z, uu[i].w};
        uint8_t *dst = bt + row * BKB;
#pragma unroll
        for (int h = 0; h < 4; ++h) {  // 8 nibbles -> one bf16 chunk
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t lo = ((int32_t)(w[h] << (28 - 8 * e))) >> 28;
            const int32_t hi = ((int32_t)(w[h] << (24 - 8 * e))) >> 28;
            o[e] = pack_bf16x2(s * (float)lo, s * (float)hi);
          }
          lds_write16(dst + (((4 * c + h) ^ (row & 7)) * 16), make_uint4(o[0], o[1], o[2], o[3]));
        }
      }
    }
  };

  // ----- consumer state -----
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wm0 = (wave / WN) * (FM * 16);   // consumer waves 0..3
  const int wn0 = (wave % WN) * (FN * 16);

  // prologue: stages 0 .. STAGES - 2 in flight, tile 0 converted
  if (loader) {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nk) issue(st, st);
    const int rem = min(STAGES - 2, nk - 1);
    if (rem >= 2) q_wait_vmcnt<2 * LOADS>();
    else if (rem == 1) q_wait_vmcnt<LOADS>();
    else q_wait_vmcnt<0>();
  }
  // every producer's loads of tile 0 are in before anyone converts it
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (producer) {
    dequant(0, 0);
    lds_writes_done();
  }

  for (int kt = 0; kt < nk; ++kt) {
    if (loader) {
      // tile kt + 1 must be resident for its dequant pass (loads complete
      // in issue order, so tile kt is too)
      const int rem = min(STAGES - 3, nk - 2 - kt);
      if (rem >= 1) q_wait_vmcnt<LOADS>();
      else q_wait_vmcnt<0>();
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (producer) {
      if (loader && kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
      if (kt + 1 < nk) dequant((kt + 1) % STAGES, (kt + 1) & 1);
      lds_writes_done();
    } else {
      const uint8_t *sa = smem + (kt % STAGES) * STAGE_BYTES;
      const uint8_t *bt = bt_base + (kt & 1) * BT_BYTES;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int pc = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16;
        bf16x8_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t *>(sa + (wm0 + i * 16 + (lane & 15)) * BKB + pc);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t *>(bt + (wn0 + j * 16 + (lane & 15)) * BKB + pc);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: (INT8: times the row scale) round to bf16, through LDS, 16-byte row stores
  constexpr int CPR = BN / 8;
  uint16_t *ct = reinterpret_cast<uint16_t *>(smem);
  __syncthreads();
  if (!producer) {
    float csc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn0 + j * 16 + (lane & 15);
      csc[j] = (FMT == 1 && col < p.N) ? p.scales[col] : 1.f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ct[(wm0 + i * 16 + ((lane >> 4) << 2) + e) * CLD + wn0 + j * 16 + (lane & 15)] =
              f32_to_bf16_bits(FMT == 1 ? acc[i][j][e] * csc[j] : acc[i][j][e]);
  }
  __syncthreads();
  for (int ch = threadIdx.x; ch < BM * CPR; ch += 256 + NPT) {
    const int row = ch / CPR;
    const int c = ch - row * CPR;
    const int gm = m0 + row;
    const int gn = n0 + c * 8;
    if (gm >= p.M || gn >= p.N) continue;
    const uint16_t *src = ct + row * CLD + c * 8;
    uint16_t *dst = p.y + (int64_t)gm * p.ldy + gn;
    if (p.vec_store && gn + 8 <= p.N) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
      for (int e = 0; e < 8 && gn + e < p.N; ++e) dst[e] = src[e];
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int FMT>
void launch_q(const QGemmArgs &a0, hipStream_t st) {
  QGemmArgs a = a0;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  constexpr int NPW = kQProducerWaves;
  hipLaunchKernelGGL((k_gemm_q_pipe<BM, BN, WM, WN, STAGES, FMT, NPW>), dim3(a.tiles_m * a.tiles_n),
                     dim3(256 + 64 * NPW), 0, st, a);
}

template <int FMT>
void launch_q_fmt(const QGemmArgs &a, hipStream_t st) {
  // the bf16 pipeline's tile rule, restricted to the shapes built here
  const int64_t t144 = (a.N % 144 == 0) ? ((a.M + 127) / 128) * (a.N / 144) : INT64_MAX;
  const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
  const int64_t t64 = ((a.M + 63) / 64) * ((a.N + 63) / 64);
  const double c144 = t144 == INT64_MAX ? 1e30 : (double)((t144 + 255) / 256) * 128 * 144 * 0.97;
  const double c128 = (double)((t128 + 255) / 256) * 128 * 128 * 1.0;
  const double c64 = (double)((t64 + 255) / 256) * 64 * 64 * 2.2;
  if (c144 <= c128 && c144 <= c64) launch_q<128, 144, 4, 1, 4, FMT>(a, st);
  else if (c128 <= c64) launch_q<128, 128, 2, 2, 4, FMT>(a, st);
  else launch_q<64, 64, 2, 2, 4, FMT>(a, st);
}

}  // namespace

hipError_t launch_gemm_q(const QGemmArgs &a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.fmt == 1) launch_q_fmt<1>(a, st);
  else launch_q_fmt<2>(a, st);
  return hipGetLastError();
}

}  // namespace lora
