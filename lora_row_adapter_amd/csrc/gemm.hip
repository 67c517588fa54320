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
#include <atomic>
#include <type_traits>

#include "kernels.hpp"
#include "plan_body.hpp"

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

// ---------------------------------------------------------------------------
// Pipelined bf16 GEMM (K a multiple of 64, 16-byte aligned rows).
//
// Operand tiles go straight from HBM/L2 into LDS with buffer_load ... lds
// (each lane's 16 bytes land at LDS base + 16 * lane; lanes past the end of
// the buffer write zeros, which pads the M / N tails).  STAGES k-tiles are in
// flight at once in a ring of LDS buffers, so load latency is hidden behind
// the MFMAs of the tiles already resident.  Rows of a tile are 64 bf16 =
// 8 chunks of 16 bytes, stored with chunk c of row r at position c ^ (r & 7)
// so the 16 lanes that read one fragment column hit distinct banks.
//
// Tile BM x BN per 512-thread workgroup: 4 consumer waves (WM x WN, each
// owning (BM / WM) x (BN / WN) outputs as 16 x 16 MFMA blocks) and 4
// producer waves that only issue the tile loads and wait for them.  One
// barrier per k-tile hands a landed tile to the consumers and a drained
// stage back to the producers; the consumers never wait on the memory
// counter, so their MFMAs are not held up behind loads still streaming in
// (measured at the 70B q+v shape: 91.5 -> 84.7 us against the same loop
// with every wave loading and multiplying).
// ---------------------------------------------------------------------------
struct PipeArgs {
  int M, N, K;
  const uint16_t *x;
  int64_t ldx;
  const uint16_t *W;
  int64_t ldw;
  uint16_t *y;
  int64_t ldy;
  int tiles_m, tiles_n;
  int vec_store;  // y rows 16-byte aligned (ldy % 8 == 0, aligned base)
  FusedT ft;      // TX kernels only
  // split-K pairs (SK == 2): fp32 partial tiles, per pair an arrival word
  // and a ready flag, this launch's epoch (never 0), the bound of the
  // second workgroup's wait (polls) and the counter of expired waits
  float *part;
  uint64_t *sync;
  uint64_t epoch;
  int32_t spin_limit;
  int32_t *expired;
  // The plan of the layer's batch: split-K pairs (has_plan != 0) run it in
  // the first-arriving workgroup of pair 0 once its partial is out; unsplit
  // tiles (plan_wg != 0) in one workgroup past the tiles, launched where it
  // fits on a CU beside a tile's workgroup, so it runs alongside the tiles
  // from the start.
  int32_t has_plan;
  int32_t plan_wg;
  PlanArgs plan;
};

// buffer resource over one split-K pair's partial slot
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(uint8_t *slot) {
  return __builtin_amdgcn_make_buffer_rsrc(slot, 0, 8 * 2 * 10 * 64 * 16, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most min(rem, R) tiles of LOADS loads each are in flight.
template <int LOADS, int R>
__device__ __forceinline__ void wait_rem(int rem) {
  if constexpr (R <= 0) {
    wait_vmcnt<0>();
  } else {
    if (rem >= R) wait_vmcnt<R * LOADS>();
    else wait_rem<LOADS, R - 1>(rem);
  }
}

// One 16-byte-per-lane load from global memory straight into LDS:
// lane l's bytes at [base + voff, +16) land at lds + 16 * l; lanes with
// voff + 16 > nbytes write zeros.  (Kept out of the kernel templates: the
// buffer-resource type exists only in device compilation.)
__device__ __forceinline__ void load16_to_lds(const void *base, uint32_t nbytes, void *lds,
                                              uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, 0, 0, 0);
}

// TX: the shrink rides along (FusedT).  The 16 padding rows of the W stage
// (BN = 144 is not a multiple of the 32-row load pattern) carry this column
// tile's 16 stacked A rows, loaded by the producer that owns them from
// per-lane addresses; the consumers run one more 16-column MFMA block and
// scatter its fp32 results into t after the k loop.  Where the ranks sum
// past the launch's capacity, the consumers then compute this tile's second
// set of 16 columns with operands straight from global memory (a fallback:
// x is read again).
// The same from a per-lane global address (no bounds: the caller keeps
// every lane's 16 bytes inside a live buffer).
__device__ __forceinline__ void load16_to_lds_at(const uint8_t *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Start of row j of adapter a's A in slice q for the folded shrink (v =
// slice << 16 | adapter << 8 | rank), or nullptr when a pool entry cannot
// be used (outside the pool, or a page past the table).
// A kernel-argument value taken into a scalar register: a per-lane select
// among such values stays a select (of loaded arguments the compiler makes
// a load from a per-lane argument address, whose wait would also wait for
// every tile load in flight)
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T *uni(T *p) {
  return reinterpret_cast<T *>((uintptr_t)uni((int64_t)(uintptr_t)p));
}

// The slice's fields are picked by a select over the argument's entries.
__device__ __forceinline__ const uint8_t *fused_arow(const FusedT &ft, int v, int K) {
  const int q = v >> 16, a = (v >> 8) & 255, j = v & 255;
  const uint8_t *A = uni(ft.A[0]);
  const int32_t *pt = uni(ft.page_table[0]);
  int R = uni(ft.R[0]), sh = uni(ft.page_shift[0]);
  int64_t mp = uni((int64_t)ft.max_pages[0]);
  int64_t np = uni(ft.n_pages[0]);
#pragma unroll
  for (int s = 1; s < kMaxSlices; ++s)
    if (q == s) {
      A = uni(ft.A[s]);
      pt = uni(ft.page_table[s]);
      R = uni(ft.R[s]);
      sh = uni(ft.page_shift[s]);
      mp = uni((int64_t)ft.max_pages[s]);
      np = uni(ft.n_pages[s]);
    }
  if (pt == nullptr) return A + (((int64_t)a * R + j) * K) * 2;
  const int64_t off = (int64_t)j * K * 2;
  const int64_t idx = off >> sh;
  if (idx >= mp) return nullptr;
  const int64_t page = pt[(int64_t)a * mp + idx];
  if (page < 0 || page >= np) return nullptr;
  return A + (page << sh) + (off & ((int64_t(1) << sh) - 1));
}

template <int BM, int BN, int WM, int WN, int STAGES, bool PC, bool TX, int SK>
__device__ __forceinline__ void pipe_body(const PipeArgs &p) {
  constexpr int NC = WM * WN;                            // MFMA (consumer) waves
  constexpr int NT = PC ? 64 * NC + 256 : 256;           // threads
  static_assert(NC == 4 || (NC == 8 && PC), "4 waves, or 8 beside separate producers");
  static_assert(SK == 1 || (SK == 2 && PC), "split-K pairs use the producer layout");
  constexpr int BKB = 128;                               // bytes per tile row (64 bf16)
  constexpr int BROWS = ((BN + 31) / 32) * 32;           // B rows loaded (multiple of 32)
  constexpr int A_INSTR = BM * 8 / 256;                  // 16-byte loads per thread per k-tile
  constexpr int B_INSTR = BROWS * 8 / 256;
  constexpr int LOADS = A_INSTR + B_INSTR;
  constexpr int A_BYTES = BM * BKB;
  // TX where the W tile has no padding rows (BN a multiple of 32): the 16 t
  // rows follow it in the stage, loaded by the last two producers
  constexpr bool TXW = TX && BN % 32 == 0;
  constexpr int STAGE_BYTES = (BM + BROWS + (TXW ? 16 : 0)) * BKB;
  constexpr int FM = BM / WM / 16;
  // TX: the t block is the last 16-column block of the last wave column
  // (TXW: every wave column has one more block slot, used by the last only)
  constexpr int FN = TXW ? BN / WN / 16 + 1 : (BN + (TX ? 16 : 0)) / WN / 16;
  constexpr int CLD = BN + 8;                            // epilogue LDS row (bf16)
  static_assert(FM * WM * 16 == BM && (FN - (TXW ? 1 : 0)) * WN * 16 == BN + (TX && !TXW ? 16 : 0),
                "tile split");
  static_assert(!TX || (PC && (TXW || BROWS - BN == 16)), "t rows fill the W stage's padding");
  constexpr int ECH = (STAGES * STAGE_BYTES >= BM * CLD * 2) ? BM : BM / 2;  // epilogue rows per pass
  static_assert(STAGES * STAGE_BYTES >= ECH * CLD * 2, "epilogue fits");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];
  static_assert(STAGES * STAGE_BYTES >= plan_detail::plan_sort_lds(plan_detail::kPlanRowBitsMax),
                "the plan of the largest batch fits the tile's LDS");
  // TX: t column c of this tile's pass p -> (slice << 16 | adapter << 8 |
  // rank) or -1 at [16 p + c]; [32]: the clamped rank sum
  __shared__ int32_t tmap[TX ? 33 : 1];

  // XCD-aware order: workgroup b runs on XCD b % 8; each XCD gets whole
  // column strips (every row tile and k half of them), so the workgroups
  // that read one W strip share that XCD's L2
  const int b = blockIdx.x;
  const int ngrid = p.tiles_m * p.tiles_n * SK;
  if constexpr (SK == 1) {
    // the extra workgroup, launched only where two of this kernel's
    // workgroups fit on a CU (its LDS at most half of it): the plan alone
    constexpr bool kPlanWg = 2 * STAGES * STAGE_BYTES <= 160 * 1024;
    if (b >= ngrid) {
      if constexpr (kPlanWg) plan_detail::plan_body<NT>(p.plan, smem, sizeof(smem));
      return;
    }
  }
  const int t = ((ngrid & 7) == 0) ? (b & 7) * (ngrid >> 3) + (b >> 3) : b;
  const int tm = t % p.tiles_m;
  const int ksp = (t / p.tiles_m) % SK;  // k half of a split-K pair
  const int tn = t / p.tiles_m / SK;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const bool producer = PC && wave >= NC;
  const int pw = producer ? wave - NC : wave;  // index among the producers / among the consumers
  // Split-K pairs take the two halves of k (an uneven split, meant to let
  // one half's partial be written while the other still multiplies,
  // measured 4 us slower: the longer half sets the end)
  const int nk_all = p.K / 64;
  const int nk0 = SK == 2 ? nk_all / 2 : nk_all;
  const int kt0 = ksp == 0 ? 0 : nk0;                     // first k-tile of this half
  const uint32_t kbase = (uint32_t)kt0 * 128u;             // its byte offset in a row

  const uint32_t a_bytes = (uint32_t)(min(BM, p.M - m0) * p.ldx * 2);
  const uint32_t b_bytes = (uint32_t)(min(BN, p.N - n0) * p.ldw * 2);
  const uint16_t *xa = p.x + (int64_t)m0 * p.ldx;
  const uint16_t *wb = p.W + (int64_t)n0 * p.ldw;

  // Per-thread source offsets (k-tile 0).  Load i of loading wave w fills LDS
  // chunks (w * INSTR + i) * 64 + lane of its operand region.
  uint32_t va[A_INSTR], vb[B_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int P = (pw * A_INSTR + i) * 64 + lane;
    const int row = P >> 3;
    const int c = (P & 7) ^ (row & 7);
    va[i] = (uint32_t)(row * p.ldx * 2 + c * 16) + kbase;
  }
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    const int P = (pw * B_INSTR + i) * 64 + lane;
    const int row = P >> 3;
    const int c = (P & 7) ^ (row & 7);
    // rows past BN (padding of the load pattern) read past the buffer: zeros
    vb[i] = row < BN ? (uint32_t)(row * p.ldw * 2 + c * 16) + kbase : 0xFFFFFFF0u;
  }

  // TX: the producer whose load pattern covers the padding rows builds the
  // column map (a wave-wide scan of the clamped ranks in (slice, adapter)
  // order) and the per-lane source rows of its padding-row loads; unused
  // columns read this tile's first x row instead (their results are dropped).
  // It issues the rest of its prologue loads first, so the ranks' latency
  // does not hold up the first tiles.  Column j of pass p of column tile tn
  // holds triple p * cap + 16 tn + j of the ordered list.
  // TXW: producers 2 and 3 each load 8 of the t rows (one more load per
  // tile, lanes of rows past the list masked off), column j of pass p of
  // column tile tn again holding entry p * cap + 16 tn + j of the list
  // (below); the column tiles past the list skip the t block.  (Spreading
  // a short list over every column tile, entry tn + j * tiles_n, measured
  // 0.45 us slower at 256 x 4096 x 4096: every tile then pays the block.)
  constexpr int TP = (BN / 8) / B_INSTR;                // that producer
  constexpr int TE = TX && !TXW ? (TP + 1) * B_INSTR - BN / 8 : 0;  // its padding-row loads per tile
  static_assert(!TX || TXW || (TP + 1) * B_INSTR * 8 == BROWS, "padding rows within one producer");
  static_assert(!TXW || NC == 4, "two of the four producers load the t rows");
  const bool t_loader = TX && producer && (TXW ? pw >= 2 : pw == TP);
  const uint8_t *tsrc[B_INSTR];
  const uint8_t *tw_src = nullptr;  // TXW: this lane's t-row source (k-tile 0), or none
  bool tw_act = false;              // TXW: this producer's t load runs (uniform)
  // the ranks of this lane's four (slice, adapter) entries and their
  // slices' max ranks, loaded before the prologue's tile loads so that the
  // wait for them does not also wait for those
  int rraw[4], rmax[4];
  auto load_ranks = [&] {
    if constexpr (TX && !TXW) {
      const FusedT &ft = p.ft;
      const int nent = ft.n_slices * ft.S;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // unconditional loads at a clamped entry, masked afterwards
        const int fc = min(lane * 4 + u, nent - 1);
        const int qc = fc / max(ft.S, 1);
        // the slice's pointer and max rank picked by a select over the
        // argument's entries (a per-lane index into them is a memory load)
        const int32_t *rk = uni(ft.ranks[0]);
        int rm = uni(ft.R[0]);
#pragma unroll
        for (int q = 1; q < kMaxSlices; ++q)
          if (qc == q) {
            rk = uni(ft.ranks[q]);
            rm = uni(ft.R[q]);
          }
        rraw[u] = rk[fc - qc * ft.S];
        rmax[u] = rm;
      }
    }
  };
  // TXW: the ordered list runs over every slot row (slice q, adapter a,
  // rank j < the slice's max_rank), so it is known from the arguments alone:
  // no load stands before the t loads and no map goes through LDS; columns
  // past an adapter's rank are computed and never read.  txw_decode(e): list
  // entry e as slice << 16 | adapter << 8 | rank, or -1 past the end --
  // branch-free (selects over the slices; a = floor(r / R) as
  // (r + 1/2) * rcp(R) in fp32, exact while r < 2^16 and R <= 128: the
  // fraction (j + 1/2) / R stays at least 1/(2R) >= 2^-8 from an integer,
  // far above the few-ulp error of the approximate reciprocal and product)
  int txw_total = 0;
  if constexpr (TXW) {
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)
      if (q < p.ft.n_slices) txw_total += p.ft.S * p.ft.R[q];
  }
  auto txw_decode = [&](int e) -> int {
    int v = -1, base = 0;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q) {
      const int R = q < p.ft.n_slices ? p.ft.R[q] : 0;  // uniform
      const int span = p.ft.S * R;
      const int r = e - base;
      const int a = (int)(((float)r + 0.5f) * __builtin_amdgcn_rcpf((float)max(R, 1)));
      const int vq = (q << 16) | (a << 8) | (r - a * R);
      v = (r >= 0 && r < span) ? vq : v;
      base += span;
    }
    return v;
  };
  auto build_map = [&] {
    if constexpr (TXW) {
      // this producer's 8 rows (lane l: row l / 8, chunk l % 8 of the
      // swizzled row)
      const FusedT &ft = p.ft;
      const int row = 8 * (pw - 2) + (lane >> 3);
      const int c = (lane & 7) ^ (row & 7);
      const int v = txw_decode(16 * tn + row);
      const uint8_t *arow = v >= 0 ? fused_arow(ft, v, p.K) : nullptr;
      tw_src = arow ? arow + c * 16 + kbase : nullptr;
      tw_act = __ballot(tw_src != nullptr) != 0;
    } else if constexpr (TX) {
      const FusedT &ft = p.ft;
      const int nent = ft.n_slices * ft.S;
      int rl[4], q4[4], a4[4], loc = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = lane * 4 + u;
        const int q = f / max(ft.S, 1);
        q4[u] = q;
        a4[u] = f - q * ft.S;
        rl[u] = f < nent ? min(max(rraw[u], 0), rmax[u]) : 0;
        loc += rl[u];
      }
      int inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      const int total = __shfl(inc, 63, 64);
      if (lane < 32) tmap[lane] = -1;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int e0 = pass * ft.cap + 16 * tn;
        int start = inc - loc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          for (int e = max(start, e0); e < min(start + rl[u], e0 + 16); ++e)
            tmap[16 * pass + e - e0] = (q4[u] << 16) | (a4[u] << 8) | (e - start);
          start += rl[u];
        }
      }
      if (lane == 0) tmap[32] = total;
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) {
        const int P = (pw * B_INSTR + i) * 64 + lane;
        const int row = P >> 3;
        const int c = (P & 7) ^ (row & 7);
        const int v = row >= BN ? tmap[row - BN] : -1;
        const uint8_t *arow = v >= 0 ? fused_arow(ft, v, p.K) : nullptr;
        tsrc[i] = (arow ? arow : reinterpret_cast<const uint8_t *>(xa)) + c * 16 + kbase;
      }
    }
  };

  const int nk = ksp == 0 ? nk0 : nk_all - nk0;
  // part: 0 every load of the tile, 1 all but the padding rows, 2 those only
  auto issue = [&](int kt, int stage, int part = 0) {
    uint8_t *sa = smem + stage * STAGE_BYTES;
    uint8_t *sb = sa + A_BYTES;
    const uint32_t kb = (uint32_t)kt * BKB;
    if (part != 2) {
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i)
        load16_to_lds(xa, a_bytes, sa + (pw * A_INSTR + i) * 1024, va[i] + kb);
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      if (TX && !TXW && t_loader && (pw * B_INSTR + i) * 8 >= BN) {
        if (part != 1) load16_to_lds_at(tsrc[i] + kb, sb + (pw * B_INSTR + i) * 1024);
      } else if (part != 2) {
        load16_to_lds(wb, b_bytes, sb + (pw * B_INSTR + i) * 1024,
                      vb[i] == 0xFFFFFFF0u ? vb[i] : vb[i] + kb);
      }
    }
    // TXW: one load of 8 t rows, issued where any of its lanes has a row
    if (TXW && t_loader && tw_act && part != 1) {
      if (tw_src != nullptr) load16_to_lds_at(tw_src + kb, sb + BROWS * BKB + (pw - 2) * 1024);
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};


  const int wm0 = (pw / WN) * (FM * 16);
  const int wn0 = (pw % WN) * (TXW ? BN / WN : FN * 16);
  // TX: whether this wave's last column block is the t block (uniform)
  const bool t_wave = TX && (pw % WN) == WN - 1;

  // TX: the ids of the t wave's rows: one batch of loads at clamped rows,
  // then two per register (ids outside [0, 256) -- none or invalid, never an
  // adapter of the map -- as 0xFFFF)
  uint32_t idr[TX ? FM : 1][4], id2[TX ? FM : 1][2];
  auto load_ids = [&] {
    if constexpr (TX) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          idr[i][e] = (uint32_t)p.ft.ids[min(m0 + wm0 + i * 16 + ((lane >> 4) << 2) + e, p.M - 1)];
    }
  };
  auto pack_ids = [&] {
    if constexpr (TX) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; e += 2)
          id2[i][e >> 1] = (idr[i][e] < 256u ? idr[i][e] : 0xFFFFu) |
                           ((idr[i][e + 1] < 256u ? idr[i][e + 1] : 0xFFFFu) << 16);
    }
  };

  // one k32 step: fragments of this wave's rows and of every column block
  // (one base offset per operand, the blocks at immediate offsets), then
  // the FM x FN MFMAs (TXW: FN - 1 without this tile's t block)
  auto kstep = [&](int soff, int ks, auto ton) {
    constexpr int NJ = (TXW && !decltype(ton)::value) ? FN - 1 : FN;
    const int pc = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16;
    int ao = soff + (wm0 + (lane & 15)) * BKB + pc;
    int bo = soff + A_BYTES + (wn0 + (lane & 15)) * BKB + pc;
    // opaque to the compiler, which would otherwise hoist one address
    // register per fragment out of the k loop instead of using the
    // instructions' immediate offsets
    asm volatile("" : "+v"(ao), "+v"(bo));
    bf16x8_t af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t *>(smem + ao + i * 16 * BKB);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t *>(smem + bo + j * 16 * BKB);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  auto compute = [&](int kt, auto ton) {
    const int soff = (kt % STAGES) * STAGE_BYTES;
    kstep(soff, 0, ton);
    // with two MFMA waves per SIMD the other wave covers the fragment
    // latency; keeping this wave's k32 steps apart holds its registers to
    // one fragment set
    if constexpr (NC == 8) __builtin_amdgcn_sched_barrier(0);
    kstep(soff, 1, ton);
  };
  // LT loads per tile, the last TL of them (the t rows) issued in the
  // prologue after the others
  auto wait_tile_t = [&](int kt, auto lt_c, auto tl_c) {
    constexpr int LT = decltype(lt_c)::value, TL = decltype(tl_c)::value;
    if (TL > 0 && kt < STAGES - 2) {
      // its prologue issued the t rows of tiles 0..STAGES-2 after the
      // rest: what may still be in flight once tile kt has landed
      static_assert(!TX || STAGES == 3 || STAGES == 4, "prologue orders for 2 or 3 tiles ahead");
      if (STAGES == 3) {
        if (nk >= 2) wait_vmcnt<TL>();
        else wait_vmcnt<0>();
      } else if (kt == 0) {
        if (nk >= 3) wait_vmcnt<2 * TL>();
        else wait_vmcnt<0>();
      } else {
        if (nk >= 4) wait_vmcnt<TL + LT>();
        else wait_vmcnt<0>();
      }
      return;
    }
    // the tiles after kt that may stay in flight: up to STAGES - 2
    wait_rem<LT, (STAGES - 2 < 63 / LT ? STAGES - 2 : 63 / LT)>(min(STAGES - 2, nk - 1 - kt));
  };
  auto wait_tile = [&](int kt) {
    using I0 = std::integral_constant<int, 0>;
    if (TXW && t_loader && tw_act)
      wait_tile_t(kt, std::integral_constant<int, LOADS + 1>{}, I0{});
    else if (TX && !TXW && t_loader)
      wait_tile_t(kt, std::integral_constant<int, LOADS>{}, std::integral_constant<int, TE>{});
    else
      wait_tile_t(kt, std::integral_constant<int, LOADS>{}, I0{});
  };
  // Raw barriers below: a wave's loads of tile kt are complete (vmcnt);
  // after the barrier every loading wave's are, and every multiplying wave
  // has finished reading the stage that the next issue overwrites.  (A
  // fenced barrier would wait for all loads in flight, including the tiles
  // still streaming in.)
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (TXW && t_loader) {
    // the t rows' sources first, while no load is in flight (arithmetic on
    // the arguments), then the tiles with their t rows in order
    build_map();
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s, s);
  } else if (t_loader) {
    load_ranks();
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s, s, 1);
    build_map();
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s, s, 2);
  } else if (!PC || producer) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s, s);
  }
  // Explicit LDS fragment reads, for the waves whose fragment latency
  // nothing else covers (one MFMA wave per SIMD): ds_read_b128 with explicit
  // lgkmcnt waits.  As ordinary loads the compiler cannot tell them from the
  // stages the DMA is still filling and waits for every load in flight
  // before each read.  NJ: the column blocks read and multiplied.
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  auto lfrag = [&](int soff, int ks, u32x4v (&af)[FM], u32x4v (&bfr)[FN], auto njc) {
    constexpr int NJ = decltype(njc)::value;
    const int pc = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16;
    const uint32_t ao = lds0 + soff + (wm0 + (lane & 15)) * BKB + pc;
    const uint32_t bo = lds0 + soff + A_BYTES + (wn0 + (lane & 15)) * BKB + pc;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(af[i]) : "v"(ao), "i"(i * 16 * BKB));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(bfr[j]) : "v"(bo), "i"(j * 16 * BKB));
  };
  // at most N LDS reads outstanding; the fragments pass through the
  // statements, so nothing reads them before the wait
  auto fwait = [&](auto nconst, u32x4v (&af)[FM], u32x4v (&bfr)[FN], auto njc) {
    constexpr int N = decltype(nconst)::value, NJ = decltype(njc)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(af[i]));
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(bfr[j]));
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(af[i]));
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(bfr[j]));
  };
  auto mma = [&](const u32x4v (&af)[FM], const u32x4v (&bfr)[FN], auto njc) {
    constexpr int NJ = decltype(njc)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                            __builtin_bit_cast(bf16x8_t, bfr[j]),
                                                            acc[i][j], 0, 0, 0);
  };
  // the four MFMA waves of the folded 64 x 64 tiles double-buffer their
  // fragments (measured at 256 x 4096 x 4096: 19.3 -> 18.5 us folded; the
  // plain tiles gain nothing)
  constexpr bool DB = PC && NC == 4 && TXW;
  static_assert(!TXW || (BM == 64 && BN == 64), "the t rows past the W tile: 64 x 64 tiles");
  using FNc = std::integral_constant<int, FN>;

  if constexpr (!PC) {
    // One MFMA wave per SIMD that also issues its share of the tile loads
    // (256 x 256 tiles: the accumulators take a SIMD's registers).  Nothing
    // else hides the fragment reads, so they are double-buffered: k-step
    // 1's fragments load during k-step 0's MFMAs, the next tile's k-step 0
    // fragments during k-step 1's (its barrier comes between the two, once
    // this tile's reads have landed).  (As ordinary loads each read's
    // latency was exposed: 43% MFMA busy at the 8192 x 4096 x 4096 prefill
    // shape.)
    u32x4v fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    // the waits count LDS reads in order: once at most FM + FN of the
    // later set are outstanding (15 at most, the counter's range), the
    // earlier set has landed
    constexpr int NFR = FM + FN < 15 ? FM + FN : 15;
    wait_tile(0);
    barrier();
    if (STAGES - 1 < nk) issue(STAGES - 1, (STAGES - 1) % STAGES);
    lfrag(0, 0, fa0, fb0, FNc{});
    // the last tile is peeled off so that the loop body has no branch
    // around the next tile's reads (the compiler would merge the wait counts
    // of both paths and wait for those reads too)
    for (int kt = 0; kt < nk - 1; ++kt) {
      lfrag((kt % STAGES) * STAGE_BYTES, 1, fa1, fb1, FNc{});
      fwait(std::integral_constant<int, NFR>{}, fa0, fb0, FNc{});
      mma(fa0, fb0, FNc{});
      // the k-step-0 MFMAs stay ahead of the wait for the next tile's loads
      // (the scheduler would otherwise sink them past the barrier and the
      // wait would no longer overlap them)
      __builtin_amdgcn_sched_barrier(0);
      wait_tile(kt + 1);
      // this wave's reads of tile kt are in registers before the barrier
      // that lets tile kt + STAGES overwrite its stage
      fwait(std::integral_constant<int, 0>{}, fa1, fb1, FNc{});
      barrier();
      if (kt + STAGES < nk) issue(kt + STAGES, (kt + STAGES) % STAGES);
      lfrag(((kt + 1) % STAGES) * STAGE_BYTES, 0, fa0, fb0, FNc{});
      mma(fa1, fb1, FNc{});
      __builtin_amdgcn_sched_barrier(0);
    }
    lfrag(((nk - 1) % STAGES) * STAGE_BYTES, 1, fa1, fb1, FNc{});
    fwait(std::integral_constant<int, NFR>{}, fa0, fb0, FNc{});
    mma(fa0, fb0, FNc{});
    fwait(std::integral_constant<int, 0>{}, fa1, fb1, FNc{});
    mma(fa1, fb1, FNc{});
  } else if (producer) {
    for (int kt = 0; kt < nk; ++kt) {
      wait_tile(kt);
      barrier();
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    }
  } else if constexpr (DB) {
    // Four MFMA waves, one per SIMD (the folded 64 x 64 tiles): as for the
    // single-role waves above, k-step 1's fragments load during k-step 0's
    // MFMAs and the next tile's k-step 0 fragments during k-step 1's, right
    // after the barrier that releases that tile; this tile's reads have
    // landed before the barrier after which its stage is refilled.
    // TXW: the t block only in the last wave column, and only where this
    // tile has a list entry.
    barrier();
    const bool ton = !TXW || (t_wave && txw_total > 16 * tn);
    auto loop = [&](auto njc) {
      constexpr int NJ = decltype(njc)::value;
      constexpr int NFR = FM + NJ < 15 ? FM + NJ : 15;
      using NFc = std::integral_constant<int, NFR>;
      using Z = std::integral_constant<int, 0>;
      u32x4v fa0[FM], fb0[FN], fa1[FM], fb1[FN];
      lfrag(0, 0, fa0, fb0, njc);
      for (int kt = 0; kt < nk - 1; ++kt) {
        const int soff = (kt % STAGES) * STAGE_BYTES;
        lfrag(soff, 1, fa1, fb1, njc);
        fwait(NFc{}, fa0, fb0, njc);
        mma(fa0, fb0, njc);
        __builtin_amdgcn_sched_barrier(0);
        fwait(Z{}, fa1, fb1, njc);
        barrier();
        lfrag(((kt + 1) % STAGES) * STAGE_BYTES, 0, fa0, fb0, njc);
        mma(fa1, fb1, njc);
        __builtin_amdgcn_sched_barrier(0);
      }
      lfrag(((nk - 1) % STAGES) * STAGE_BYTES, 1, fa1, fb1, njc);
      fwait(NFc{}, fa0, fb0, njc);
      mma(fa0, fb0, njc);
      fwait(Z{}, fa1, fb1, njc);
      mma(fa1, fb1, njc);
    };
    if (!TXW || ton) loop(FNc{});
    else loop(std::integral_constant<int, TXW ? FN - 1 : FN>{});
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      barrier();
      compute(kt, std::true_type{});
    }
  }

  // The finished tile: the accumulators plus, for a split-K pair, the other
  // half's partial (added where each block is consumed, so no second
  // accumulator set is held in registers)
  uint8_t *part_in = nullptr;
  if constexpr (SK == 2) {
    // The two k halves of a tile meet here.  The workgroup that arrives
    // second adds the first one's fp32 partial and runs the epilogue; the
    // first writes its partial, raises the pair's ready flag and leaves.
    // Arrival order comes from swapping this launch's epoch into the pair's
    // arrival word (any other value there means "first"); only the second
    // waits, and only for a workgroup that has already arrived.  The second
    // puts both words back to 0 once it has seen them (no other workgroup
    // touches them again in this launch), so a later launch that carries the
    // same epoch -- a replayed graph -- finds the pair as if new.  Its wait
    // is bounded; an expired wait (the tile then holds a stale partial) is
    // counted in *expired, which lora_check reports.  a + b == b + a in
    // fp32, so the result does not depend on which half arrives first.
    // Every access to the partial, the flag and the arrival word is
    // device-scope (sc1: coherent across the XCDs' L2s by itself, as the
    // compiler emits relaxed agent-scope atomics), and the writer waits for
    // its partial stores to complete before it raises the flag, so no
    // cache-wide write-back or invalidate is needed (those cost 4.6 us per
    // launch at the 70B q+v shape).
    const int pair = tm + p.tiles_m * tn;
    uint64_t *arrive = p.sync + 2 * pair;
    uint64_t *ready = arrive + 1;
    static_assert(NC * FM * FN * 64 * 16 <= 8 * 2 * 10 * 64 * 16, "partial fits its slot");
    uint8_t *part_base = reinterpret_cast<uint8_t *>(p.part) + (size_t)pair * (8 * 2 * 10 * 64 * 16);
    const __amdgpu_buffer_rsrc_t part = part_rsrc(part_base);
    __shared__ int s_second;
    __syncthreads();  // every wave is past its k loop
    if (tid == 0) {  // relaxed: the partial is published through the ready flag
      const bool second =
          __hip_atomic_exchange(arrive, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.epoch;
      if (second) __hip_atomic_store(arrive, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_second = second;
    }
    __syncthreads();
    if (!s_second) {
      if (!producer) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[i][j]), part,
                                                   (((pw * FM + i) * FN + j) * 64 + lane) * 16, 0,
                                                   kCpolSc1);
        wait_vmcnt<0>();  // this wave's partial stores are performed
      }
      __syncthreads();
      if (tid == 0) __hip_atomic_store(ready, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The layer's plan needs only the row ids: this workgroup, its half
      // of the tile handed over, runs it in its freed LDS while the other
      // half finishes the tile -- so the plan needs no kernel, stream or
      // event of its own, and the kernels after the GEMM see it in stream
      // order
      if (p.has_plan && pair == 0) plan_detail::plan_body_lean<NT>(p.plan, smem, sizeof(smem));
      return;
    }
    if (tid == 0) {
      // bounded: the first half has arrived, so its flag follows its
      // partial within microseconds
      bool seen = false;
      for (int n = 0; n < p.spin_limit; ++n) {
        if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.epoch) {
          seen = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (seen)
        __hip_atomic_store(ready, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_fetch_add(p.expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    part_in = part_base;
  }
  const bool owner = !producer;  // the MFMA waves hold the finished tile
  auto tile_val = [&](int i, int j) -> f32x4_t {
    if constexpr (SK == 2)
      return acc[i][j] + __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         part_rsrc(part_in), (((pw * FM + i) * FN + j) * 64 + lane) * 16,
                                                         0, kCpolSc1));
    return acc[i][j];
  };

  if constexpr (TX) {
    // t: this tile's rows x its 16 t columns, kept where the row's adapter
    // owns the column (tmap was written before the k loop's barriers;
    // TXW: the list decoded from the arguments)
    if (owner && t_wave) {
      const FusedT &ft = p.ft;
      load_ids();
      pack_ids();
      auto scatter = [&](int v, const f32x4_t (&t)[FM]) {
        if (v < 0) return;
        const int q = v >> 16, a = (v >> 8) & 255, j = v & 255;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = m0 + wm0 + i * 16 + ((lane >> 4) << 2) + e;
            if (m < p.M && ((id2[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu) == (uint32_t)a)
              ft.tpart[((int64_t)m * ft.n_slices + q) * ft.Rw + j] = t[i][e];
          }
      };
      f32x4_t t0[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) t0[i] = tile_val(i, FN - 1);
      scatter(TXW ? txw_decode(16 * tn + (lane & 15)) : tmap[lane & 15], t0);
      if ((TXW ? txw_total : tmap[32]) > ft.cap) {  // uniform
        // second pass: MFMA operands straight from global memory (x rows in
        // the A-operand layout, the column's A row in the B-operand layout),
        // loads at clamped rows / a valid dummy row, all issued before use
        const int v1 = TXW ? txw_decode(ft.cap + 16 * tn + (lane & 15)) : tmap[16 + (lane & 15)];
        const int kl = (lane >> 4) * 8;
        const uint8_t *arow = v1 >= 0 ? fused_arow(ft, v1, p.K) : nullptr;
        const uint16_t *asrc = arow ? reinterpret_cast<const uint16_t *>(arow) + kl
                                    : p.x + (int64_t)m0 * p.ldx + kl;
        const uint16_t *xr[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          xr[i] = p.x + (int64_t)min(m0 + wm0 + i * 16 + (lane & 15), p.M - 1) * p.ldx + kl;
        f32x4_t t1[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) t1[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < p.K; k0 += 32) {  // K % 64 == 0
          bf16x8_t xf[FM];
#pragma unroll
          for (int i = 0; i < FM; ++i) xf[i] = *reinterpret_cast<const bf16x8_t *>(xr[i] + k0);
          const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(asrc + k0);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            t1[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[i], af, t1[i], 0, 0, 0);
        }
        scatter(v1, t1);
      }
    }
  }

  // epilogue: bf16 tile through LDS (ECH rows per pass), then 16-byte row stores
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  uint16_t *ct = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
  for (int r0 = 0; r0 < BM; r0 += ECH) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm0 + i * 16;
      if (!owner || rb < r0 || rb >= r0 + ECH) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (TX && j == FN - 1 && (TXW || t_wave)) continue;
        const f32x4_t v = tile_val(i, j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ct[(rb - r0 + ((lane >> 4) << 2) + e) * CLD + wn0 + j * 16 + (lane & 15)] =
              f32_to_bf16_bits(v[e]);
      }
    }
    __syncthreads();
    for (int ch = tid; ch < ECH * CPR; ch += NT) {
      const int row = ch / CPR;
      const int c = ch - row * CPR;
      const int gm = m0 + r0 + row;
      const int gn = n0 + c * 8;
      if (gm >= p.M || gn >= p.N) continue;
      const uint16_t *src = ct + row * CLD + c * 8;
      uint16_t *dst = p.y + (int64_t)gm * p.ldy + gn;
      if (p.vec_store && gn + 8 <= p.N) {
        if constexpr (BM == 256 && BN == 256) {
          // the largest tiles run at prefill sizes, where y is far larger
          // than L2: the stores stream past it
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(src),
                                      reinterpret_cast<u32x4_t *>(dst));
        } else {
          *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
        }
      } else {
        for (int e = 0; e < 8 && gn + e < p.N; ++e) dst[e] = src[e];
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, bool PC, bool TX>
__global__ __launch_bounds__(PC ? 64 * WM * WN + 256 : 256) void k_gemm_bf16_pipe(PipeArgs p) {
  pipe_body<BM, BN, WM, WN, STAGES, PC, TX, 1>(p);
}

// 256-row tiles with eight MFMA waves beside the four producers: split-K
// pairs (SK = 2) over 256 x 144 tiles, and unsplit 256 x 160 tiles.  Where
// the W stage's rows (with the folded shrink's 16) split into two 16-column
// multiples, the waves take 64 x (rows / 2) each (4 x 2), else 32 x 144
// (8 x 1): per k step a wave reads (M_w + N_w) fragment rows for M_w x N_w
// outputs, so the 4 x 2 split reads 25% fewer LDS bytes per flop (measured
// at the 70B q+v shape with the shrink folded in: 85.4 -> 82.7 us).
template <int BN, bool TX, int SK>
__global__ __launch_bounds__(768) void k_gemm_bf16_split(PipeArgs p) {
  constexpr int WN = ((BN + (TX ? 16 : 0)) % 32 == 0) ? 2 : 1;
  pipe_body<256, BN, 8 / WN, WN, 3, true, TX, SK>(p);
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

// Values a launch writes to the split-K pairs' exchange words, one per
// launch, never 0 (the words' resting value)
std::atomic<uint64_t> g_epoch{0x9E3779B97F4A7C15ull};
uint64_t next_epoch() {
  uint64_t e;
  do e = g_epoch.fetch_add(1, std::memory_order_relaxed);
  while (e == 0);
  return e;
}
constexpr int32_t kSpinDefault = 1 << 22;  // polls of ~2 x 64 clocks: ~0.3 s
std::atomic<int32_t> g_spin_limit{kSpinDefault};

// Whether two workgroups of kernel `fn` (`threads` each) fit on one CU
// (registers and LDS): then one more workgroup can run the plan beside the
// tiles.
bool plan_fits_beside(const void *fn, int threads) {
  hipFuncAttributes at{};
  if (!kernel_attributes(fn, &at)) return false;
  KernelFootprint f;
  f.threads = threads;
  f.vgprs = at.numRegs;
  f.lds = at.sharedSizeBytes;
  return fits_beside(f, f);
}

// Returns false when asked to carry a plan it cannot (no launch then).
template <int BM, int BN, int WM, int WN, int STAGES, bool TX = false>
bool launch_pipe(const PipeArgs &pa0, hipStream_t st, const PlanArgs *plan = nullptr) {
  PipeArgs pa = pa0;
  pa.tiles_m = (pa.M + BM - 1) / BM;
  pa.tiles_n = (pa.N + BN - 1) / BN;
  // separate producer waves where the consumers' accumulators leave room
  // for a second wave per SIMD (at most 128 fp32 per lane)
  constexpr bool PC = (BM / WM) * (BN / WN) / 64 <= 128;
  constexpr int threads = PC ? 64 * WM * WN + 256 : 256;
  const auto fn = k_gemm_bf16_pipe<BM, BN, WM, WN, STAGES, PC, TX>;
  const int ngrid = pa.tiles_m * pa.tiles_n;
  int extra = 0;
  if (plan != nullptr && plan->M > 0) {
    if (!plan_fits_beside((const void *)fn, threads)) return false;
    pa.plan = *plan;
    pa.plan_wg = 1;
    extra = 1;
  }
  hipLaunchKernelGGL(fn, dim3(ngrid + extra), dim3(threads), 0, st, pa);
  return true;
}

bool pipe_ok(int64_t k, int64_t ldx, int64_t ldw) {
  return (k % 64) == 0 && (uint64_t)256 * ldx * 2 < (1ull << 32) &&
         (uint64_t)256 * ldw * 2 < (1ull << 32);
}

// LDS stages of the 64 x 64 tiles (measured at 256 x 4096 x 4096: 3
// stages 18.3 us, 4 15.4, 6 21.7, 8 19.6)
constexpr int kStages64 = 4;

// Tile choice: fill the 256 CUs with as few, as large tiles as possible.
// Relative per-FLOP costs of the shapes were measured on MI355X (bigger
// tiles move fewer bytes per FLOP into LDS).  Returns the index into the
// launch switch below.
int choose_tile(int64_t M, int64_t d) {
  struct Cand { int bm, bn; double cost; };
  const Cand cands[] = {{256, 256, 0.87}, {256, 128, 0.90}, {128, 144, 0.97},
                        {128, 128, 1.00}, {64, 64, 2.2},   {256, 160, 0.92}};
  int best = 3;
  double best_t = 1e30;
  for (int c = 0; c < 6; ++c) {
    const Cand &cd = cands[c];
    if ((cd.bn == 144 && d % 144 != 0) || (cd.bn == 160 && d % 160 != 0)) continue;
    const int64_t tiles = ((M + cd.bm - 1) / cd.bm) * ((d + cd.bn - 1) / cd.bn);
    const int64_t rounds = (tiles + 255) / 256;
    const double t_est = (double)rounds * cd.bm * cd.bn * cd.cost;
    if (t_est < best_t * 0.999) {
      best_t = t_est;
      best = c;
    }
  }
  return best;
}

PipeArgs pipe_args(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx, const void *W,
                   int64_t ldw, void *y, int64_t ldy) {
  PipeArgs pa{};
  pa.M = (int)M;
  pa.N = (int)d;
  pa.K = (int)k;
  pa.x = (const uint16_t *)x;
  pa.ldx = ldx;
  pa.W = (const uint16_t *)W;
  pa.ldw = ldw;
  pa.y = (uint16_t *)y;
  pa.ldy = ldy;
  pa.vec_store = ((ldy % 8) == 0 && ((uintptr_t)y & 15) == 0) ? 1 : 0;
  return pa;
}

// Split-K pairs for the 128 x 144 shapes with more than one 128-row tile
// (e.g. the 70B q+v decode pair): 256 x 144 tiles, each computed by two
// workgroups over the two halves of k -- eight MFMA waves plus the four
// producers per workgroup, the same 256 workgroups as 128 x 144 tiles at
// 512 rows, but every workgroup streams (256 + 144) x k/2 operand bytes
// instead of (128 + 144) x k and each W line is shared by two workgroups
// instead of four (measured at the 70B q+v shape: main loop 81 -> 62 us;
// the load path, not the MFMAs, bounds it).
constexpr int kSplitBM = 256, kSplitBN = 144;
constexpr size_t kSplitPartBytes = (size_t)8 * 2 * 10 * 64 * 16;  // per pair (t block included)

int64_t split_pairs(int64_t M, int64_t d) {
  return ((M + kSplitBM - 1) / kSplitBM) * ((d + kSplitBN - 1) / kSplitBN);
}
// GEMM region: a 256-byte header (word kHdrSyncExpired counts expired pair
// waits when the region is a lora_gemm workspace), the pairs' partial
// slots, then their arrival / ready words
constexpr size_t kGemmHdrBytes = 256;
size_t split_bytes(int64_t M, int64_t d) {
  const int64_t P = split_pairs(M, d);
  return kGemmHdrBytes + ((size_t)P * kSplitPartBytes + 255) / 256 * 256 +
         ((size_t)P * 16 + 255) / 256 * 256;
}
bool split_ok(int64_t M, int64_t k, int64_t d, void *gws, size_t gws_bytes) {
  // k >= 256: each half holds at least two k-tiles
  return gws != nullptr && ((uintptr_t)gws & 255u) == 0 && M > 128 && (k % 128) == 0 && k >= 256 &&
         gws_bytes >= split_bytes(M, d);
}
template <bool TX>
void launch_split(PipeArgs pa, int64_t M, int64_t d, void *gws, int32_t *expired, hipStream_t st,
                  const PlanArgs *plan) {
  pa.has_plan = plan != nullptr;
  if (plan) pa.plan = *plan;
  const int64_t P = split_pairs(M, d);
  pa.tiles_m = (int)((M + kSplitBM - 1) / kSplitBM);
  pa.tiles_n = (int)((d + kSplitBN - 1) / kSplitBN);
  static_assert(kSplitBN == 144, "split-K pairs use 256 x 144 tiles");
  uint8_t *region = reinterpret_cast<uint8_t *>(gws);
  pa.part = reinterpret_cast<float *>(region + kGemmHdrBytes);
  pa.sync = reinterpret_cast<uint64_t *>(region + kGemmHdrBytes +
                                         ((size_t)P * kSplitPartBytes + 255) / 256 * 256);
  pa.expired = expired ? expired : reinterpret_cast<int32_t *>(region) + kHdrSyncExpired;
  pa.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  pa.epoch = next_epoch();
  hipLaunchKernelGGL((k_gemm_bf16_split<144, TX, 2>), dim3(pa.tiles_m * pa.tiles_n * 2), dim3(768),
                     0, st, pa);
}
// Unsplit 256 x 160 tiles (e.g. 2048 rows x 5120 columns: 256 tiles, where
// 256 x 256 tiles leave 96 CUs idle)
bool launch_wide(PipeArgs pa, int64_t M, int64_t d, hipStream_t st, const PlanArgs *plan) {
  if (plan != nullptr && plan->M > 0) return false;  // its LDS leaves no room beside it
  pa.tiles_m = (int)((M + 255) / 256);
  pa.tiles_n = (int)((d + 159) / 160);
  hipLaunchKernelGGL((k_gemm_bf16_split<160, false, 1>), dim3(pa.tiles_m * pa.tiles_n), dim3(768),
                     0, st, pa);
  return true;
}

}  // namespace

size_t gemm_ws_bytes(int64_t M, int64_t k, int64_t d) {
  if (M <= 128 || d <= 0 || (k % 128) != 0 || k < 256 || choose_tile(M, d) != 2) return 0;
  return split_bytes(M, d);
}

void set_sync_spin_limit(int32_t polls) {
  g_spin_limit.store(polls < 0 ? kSpinDefault : polls, std::memory_order_relaxed);
}


hipError_t launch_gemm(int32_t dtype, int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                       const void *W, int64_t ldw, void *y, int64_t ldy, void *gws,
                       size_t gws_bytes, hipStream_t st, int32_t *expired, const PlanArgs *plan) {
  if (M <= 0 || d <= 0) return hipSuccess;
  if (dtype == 1) {
    if (pipe_ok(k, ldx, ldw)) {
      PipeArgs pa = pipe_args(M, k, d, x, ldx, W, ldw, y, ldy);
      bool ok = true;  // false: asked to carry a plan the launch cannot
      switch (choose_tile(M, d)) {
        case 0: ok = launch_pipe<256, 256, 2, 2, 2>(pa, st, plan); break;
        case 1: ok = launch_pipe<256, 128, 4, 1, 3>(pa, st, plan); break;
        case 2:
          if (split_ok(M, k, d, gws, gws_bytes)) {
            launch_split<false>(pa, M, d, gws, expired, st, plan);
          } else {
            ok = launch_pipe<128, 144, 4, 1, 3>(pa, st, plan);
          }
          break;
        case 3: ok = launch_pipe<128, 128, 2, 2, 4>(pa, st, plan); break;
        case 5: ok = launch_wide(pa, M, d, st, plan); break;
        default: ok = launch_pipe<64, 64, 2, 2, kStages64>(pa, st, plan); break;
      }
      return ok ? hipGetLastError() : hipErrorInvalidValue;
    }
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

int32_t gemm_fused_cap(int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw) {
  if (M <= 0 || d <= 0 || !pipe_ok(k, ldx, ldw)) return 0;
  const int tile = choose_tile(M, d);
  if (tile == 2) return (int32_t)(16 * ((d + 143) / 144));
  if (tile == 4) return (int32_t)(16 * ((d + 63) / 64));
  return 0;
}

// The kernel and block size launch_gemm / launch_gemm_fused would run.
static void gemm_pick(int32_t dtype, int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw,
                      bool split, bool fused, const void **fn, int *threads) {
  *threads = 256;
  if (dtype != 1) {
    *fn = (const void *)k_gemm_f32;
    return;
  }
  if (!pipe_ok(k, ldx, ldw)) {
    *fn = (const void *)k_gemm_bf16;
    return;
  }
  const int tile = choose_tile(M, d);
  switch (fused && tile != 4 ? 2 : tile) {
    case 0: *fn = (const void *)k_gemm_bf16_pipe<256, 256, 2, 2, 2, false, false>; break;
    case 1: *fn = (const void *)k_gemm_bf16_pipe<256, 128, 4, 1, 3, true, false>; *threads = 512; break;
    case 2:
      if (split) {
        *fn = fused ? (const void *)k_gemm_bf16_split<144, true, 2>
                    : (const void *)k_gemm_bf16_split<144, false, 2>;
        *threads = 768;
      } else {
        *fn = fused ? (const void *)k_gemm_bf16_pipe<128, 144, 4, 1, 3, true, true>
                    : (const void *)k_gemm_bf16_pipe<128, 144, 4, 1, 3, true, false>;
        *threads = 512;
      }
      break;
    case 3: *fn = (const void *)k_gemm_bf16_pipe<128, 128, 2, 2, 4, true, false>; *threads = 512; break;
    case 5: *fn = (const void *)k_gemm_bf16_split<160, false, 1>; *threads = 768; break;
    default:
      *fn = fused ? (const void *)k_gemm_bf16_pipe<64, 64, 2, 2, kStages64, true, true>
                  : (const void *)k_gemm_bf16_pipe<64, 64, 2, 2, kStages64, true, false>;
      *threads = 512;
      break;
  }
}

bool gemm_footprint(int32_t dtype, int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw,
                    void *gws, size_t gws_bytes, bool fused, KernelFootprint *out) {
  const void *fn = nullptr;
  int threads = 256;
  gemm_pick(dtype, M, k, d, ldx, ldw, dtype == 1 && split_ok(M, k, d, gws, gws_bytes), fused, &fn,
            &threads);
  hipFuncAttributes at{};
  if (!kernel_attributes(fn, &at)) return false;
  out->threads = threads;
  out->vgprs = at.numRegs;
  out->lds = at.sharedSizeBytes;
  return true;
}

hipError_t launch_gemm_fused(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                             const void *W, int64_t ldw, void *y, int64_t ldy, const FusedT &ft,
                             void *gws, size_t gws_bytes, hipStream_t st, int32_t *expired,
                             const PlanArgs *plan) {
  if (ft.cap <= 0 || ft.cap != gemm_fused_cap(M, k, d, ldx, ldw) ||
      ft.n_slices * ft.S > kFusedMaxEntries || ft.S > 256 || ft.n_slices > kMaxSlices)
    return hipErrorInvalidValue;
  PipeArgs pa = pipe_args(M, k, d, x, ldx, W, ldw, y, ldy);
  pa.ft = ft;
  if (choose_tile(M, d) == 4) {
    // the 64 x 64 tiles decode the list with an fp32 reciprocal of each
    // slice's max_rank, exact up to 128 (the MFMA path takes at most 64)
    for (int q = 0; q < ft.n_slices; ++q)
      if (ft.R[q] < 0 || ft.R[q] > 128) return hipErrorInvalidValue;
    if (!launch_pipe<64, 64, 2, 2, kStages64, true>(pa, st, plan)) return hipErrorInvalidValue;
  } else if (split_ok(M, k, d, gws, gws_bytes)) {
    launch_split<true>(pa, M, d, gws, expired, st, plan);
  } else if (!launch_pipe<128, 144, 4, 1, 3, true>(pa, st, plan)) {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool gemm_runs_plan(int32_t dtype, int64_t M, int64_t k, int64_t d, int64_t ldx, int64_t ldw,
                    void *gws, size_t gws_bytes, bool fused) {
  if (dtype != 1 || M <= 0 || d <= 0 || !pipe_ok(k, ldx, ldw)) return false;
  if (split_ok(M, k, d, gws, gws_bytes) && choose_tile(M, d) == 2) return true;
  KernelFootprint f;
  return gemm_footprint(dtype, M, k, d, ldx, ldw, gws, gws_bytes, fused, &f) && f.lds > 0 &&
         fits_beside(f, f) && (fused || choose_tile(M, d) != 5);
}

}  // namespace lora
