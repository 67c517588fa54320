/*
 * lora_row.h -- C ABI of liblora_row.so: the multi-adapter LoRA linear layer
 * on AMD MI355X (gfx950, CDNA4).
 *
 * The layer (one shared base weight, a per-row adapter choice):
 *
 *   y[m, :] = x[m, :] W^T + scale[s] * (x[m, :] A_s^T) B_s^T     s = adapter_ids[m] >= 0
 *   y[m, :] = x[m, :] W^T                                         adapter_ids[m] == -1
 *
 *   x [M, k], W [d, k] (out x in), A_s [r_s, k], B_s [d, r_s], y [M, d];
 *   scale[s] = alpha_s / r_s (true rank), stored with the adapter.
 *
 * Sources (page title, section):
 *   - "S-LoRA: what the paper actually says about serving thousands of LoRA
 *     adapters", "Batched LoRA computation": per-request output is the shared
 *     base term plus (alpha/r) B_k A_k x_i for that request's adapter k; the
 *     base is one GEMM over the whole batch, the corrections one segmented
 *     operation over rows sorted by adapter.
 *   - "LoRA Adapters: Many Models in One", "The model runner's part": stacked
 *     A/B tensors with one slot per active adapter and a per-token slot index
 *     (or none); "Using it": every slot is allocated at the maximum rank and
 *     smaller adapters are padded.
 *   - "Adapter Residency When One Replica Serves Many Fine-Tunes", "What the
 *     forward pass has to do differently": base projection dense over the
 *     batch, each adapter applied to its rows only (a gather/scatter over row
 *     indices); the scale belongs with the adapter.
 *   - "S-LoRA: ...", "Unified paging": adapter weights held in fixed-size
 *     blocks of one pool, found through a per-adapter block list.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) unless a parameter says "host".  The caller owns every buffer;
 *     the library never allocates or frees device memory inside these calls.
 *   - Row-major layouts.  Leading dimensions are in elements.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Compute calls are asynchronous on it and never synchronise, except
 *     lora_check and lora_profile_read, which say so.
 *   - Errors are returned as lora_status_t; nothing throws across the ABI.
 *     Argument errors are detected on the host before anything is launched.
 *     Errors in DEVICE-resident arguments (ids, ranks, page-table entries)
 *     are detected on the device: the offending rows are treated as having
 *     no adapter, are counted, and lora_check reports the counts.
 *   - One workspace must not be used by two calls in flight at once (e.g. on
 *     two streams).
 */
#ifndef LORA_ROW_H
#define LORA_ROW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 3

typedef enum lora_status {
  LORA_OK = 0,
  LORA_ERR_ARG = 1,         /* null pointer, bad enum, negative size, bad flag combination */
  LORA_ERR_SHAPE = 2,       /* sizes / leading dims / alignment not supported */
  LORA_ERR_DTYPE = 3,       /* unsupported dtype */
  LORA_ERR_RANK = 4,        /* max_rank out of the supported range */
  LORA_ERR_WORKSPACE = 5,   /* workspace too small or misaligned */
  LORA_ERR_PAGE = 6,        /* pool geometry invalid (page size, counts) */
  LORA_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  LORA_ERR_UNSUPPORTED = 8  /* valid request that this library does not implement */
} lora_status_t;

/* The two range enumerators of the enums a caller passes in make every
 * int32 value a valid value of the type (a C caller may pass any int; the
 * library checks it and answers LORA_ERR_DTYPE / LORA_ERR_ARG). */
typedef enum lora_dtype {
  LORA_DTYPE_F32 = 0,   /* x, W, A, B, y in fp32; true fp32 products, fp32 accumulation */
  LORA_DTYPE_BF16 = 1,  /* x, W, A, B, y in bf16; fp32 accumulation, RNE on store */
  LORA_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  LORA_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} lora_dtype_t;

typedef enum lora_path {
  LORA_PATH_AUTO = 0,    /* MFMA (SGMV) kernels where supported, else gather */
  LORA_PATH_GATHER = 1,  /* VALU kernels: per-row gather, bf16 dot2 / fp32 FMA, wavefront
                            reduction over k, A staged in LDS (any dtype, rank <= 256) */
  LORA_PATH_SGMV = 2     /* MFMA tiles over the adapter-sorted segments (bf16, max_rank <= 64;
                            LORA_ERR_UNSUPPORTED otherwise) */
} lora_path_t;

/* Flags for lora_linear. */
#define LORA_FLAG_REUSE_PLAN 1u  /* skip the plan step and use the plan already in the
                                    workspace (made by lora_plan or an earlier lora_linear on
                                    the same adapter_ids, M and adapter set).  One plan serves
                                    every adapted layer of a step, since ids are per token. */
#define LORA_FLAG_SEPARATE_SHRINK 2u  /* run the shrink as its own kernel even where the base
                                         GEMM could carry it (see lora_linear_sliced) */

/* Where adapter weights live. */
typedef enum lora_adapter_kind {
  LORA_ADAPTERS_SLOTS = 0,  /* stacked, rank-padded slots */
  LORA_ADAPTERS_POOL = 1,   /* unified pool of fixed-size pages + per-adapter page table */
  LORA_ADAPTERS_RANGE_MIN_ = -0x7FFFFFFF - 1,
  LORA_ADAPTERS_RANGE_MAX_ = 0x7FFFFFFF
} lora_adapter_kind_t;

/*
 * Adapter set.  The struct itself is HOST memory (read during the call only);
 * the arrays it points to are device memory.
 *
 * SLOTS: A [n_adapters, max_rank, k] and B [n_adapters, d, max_rank], same
 *   dtype as x.  Slot s holds A_s in rows 0..r_s-1 of A[s] and B_s in columns
 *   0..r_s-1 of B[s]; padding may hold anything (NaN included) and never
 *   reaches the result (a kernel may load it, inside a 16-byte vector that
 *   it zeroes first, or as whole rows of A whose products it never reads).
 * POOL: `pool` is n_pages * page_bytes bytes.  Adapter a's logical byte space
 *   is A_a (r_a x k, row-major) followed by B_a (d x r_a, row-major, row
 *   stride r_a), both unpadded, in x's dtype; logical page j of it is physical
 *   page page_table[a * max_pages + j] of the pool.  page_bytes is a power of
 *   two >= 256.  Entries that an adapter does not need are ignored.
 * ranks: device int32 [n_adapters], true rank r_s of each slot / adapter,
 *   0 <= r_s <= max_rank (a rank outside that range is a device-side error).
 */
typedef struct lora_adapters {
  int32_t kind;               /* lora_adapter_kind_t */
  int32_t n_adapters;         /* S: number of slots (SLOTS) or adapters (POOL) */
  int32_t max_rank;           /* R: 1..256; slot padding width (SLOTS), rank cap (both) */
  int32_t max_pages;          /* POOL: columns of page_table */
  const int32_t *ranks;       /* device int32 [S] */
  const void *A;              /* SLOTS: device [S, R, k] */
  const void *B;              /* SLOTS: device [S, d, R] */
  const void *pool;           /* POOL: device bytes [n_pages * page_bytes] */
  const int32_t *page_table;  /* POOL: device int32 [S, max_pages] */
  int64_t page_bytes;         /* POOL */
  int64_t n_pages;            /* POOL */
} lora_adapters_t;

/* ABI version of the loaded library (LORA_ABI_VERSION it was built with). */
int32_t lora_abi_version(void);

/* Static description of a status code. */
const char *lora_status_str(lora_status_t status);

/*
 * Bytes of workspace lora_linear / lora_plan need for up to max_rows rows
 * with this adapter set (covers every path).  Host-only; no device access.
 * Returns 0 on invalid arguments.  The workspace is caller-owned device
 * memory, 256-byte aligned; its contents need no initialisation.
 */
size_t lora_workspace_bytes(int64_t max_rows, int64_t d, int64_t k, lora_dtype_t dtype,
                            const lora_adapters_t *adapters);

/*
 * Bytes of workspace lora_gemm uses for this shape: the fp32 partial tiles
 * and arrival/ready words of its split-K workgroup pairs.  0 when the shape
 * runs unsplit tiles (then lora_gemm needs no workspace).  Host-only.
 */
size_t lora_gemm_workspace_bytes(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype);

/*
 * Base projection only: y = x W^T ("S-LoRA: what the paper actually says
 * ...", section "Batched LoRA computation": the base term is one GEMM over
 * the whole batch).  Same kernels as the base step of lora_linear: with a
 * workspace of lora_gemm_workspace_bytes(M, k, d, dtype) bytes (or a
 * lora_linear workspace for the same rows, whose GEMM region it is), rows
 * with no adapter in lora_linear are bitwise equal to this.  Shapes that
 * split k across workgroup pairs fall back to unsplit tiles when workspace
 * is NULL or smaller (same values up to fp32 summation order).
 * x [M, k] (ldx >= k), W [d, k] (ldw >= k), y [M, d] (ldy >= d).
 * bf16: k, ldx, ldw multiples of 8 and ldy a multiple of 2; f32: k, ldx, ldw
 * multiples of 4.  workspace: device, 256-byte aligned (else
 * LORA_ERR_WORKSPACE), caller-owned, no initialisation needed; it must not
 * be in use by another call that is still running.  M == 0 is a no-op.
 */
lora_status_t lora_gemm(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                        int64_t ldx, const void *W, int64_t ldw, void *y, int64_t ldy,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * The LoRA linear layer (see the top of this file).
 *   adapter_ids: device int32 [M]; -1 = no adapter; other values outside
 *                [0, n_adapters) are device-side errors (row treated as none).
 *   scales:      device fp32 [n_adapters]; scale of slot / adapter s.
 *   workspace:   device, >= lora_workspace_bytes(M, d, k, dtype, adapters).
 *   path:        lora_path_t; flags: LORA_FLAG_* (0 for none).
 * Steps: plan (validate ids, stable sort of adapted rows by adapter,
 * segment and work-item tables), base GEMM y = x W^T, shrink t = x A_s^T
 * over k into fp32 partials (one per k split), expand y += scale_s t B_s^T
 * on adapted rows only (t = the partials summed in split order).  All run
 * on `stream`.  The plan rides inside the base GEMM's launch where that
 * launch can carry it without slowing its tiles (split-K workgroup pairs:
 * the first to arrive runs it; tiles whose kernel fits twice on a CU: one
 * extra workgroup runs it beside them); otherwise it is its own kernel,
 * beside the GEMM on the library's side stream (one per device, default
 * priority, joined by an event before the shrink) where one of its
 * workgroups fits on a CU next to one of the GEMM's, else on `stream` ahead
 * of the GEMM.  From the caller's view the call is ordered on `stream` as
 * usual.  Rows with no adapter are written once, by the GEMM.
 * Results are run-to-run deterministic (no floating-point atomics).
 */
lora_status_t lora_linear(lora_dtype_t dtype, int64_t M, int64_t k, int64_t d, const void *x,
                          int64_t ldx, const void *W, int64_t ldw,
                          const lora_adapters_t *adapters, const int32_t *adapter_ids,
                          const float *scales, void *y, int64_t ldy, void *workspace,
                          size_t workspace_bytes, int32_t path, uint32_t flags, void *stream);

/*
 * Several projections of the same input in one call -- e.g. the q and v
 * projections of an attention layer ("Your LoRA Adapters Are Thrashing Your
 * GPUs", section 02: Q and V are the usual adapted pair; section 01 shows
 * each adapted projection as W + B A applied to the same x).  Slice i is a
 * LoRA linear layer of width d_i with its own adapter set and scales; all
 * slices share x, the per-row adapter_ids and one plan.
 *   W: [sum_i d_i, k] -- the slices' base weights stacked by rows (slice 0
 *      first), ldw >= k.
 *   y: [M, sum_i d_i] -- slice i owns columns [sum_{j<i} d_j, + d_i).
 *   slices: HOST array of n_slices (1..LORA_MAX_SLICES) descriptors; every
 *      slice has the same n_adapters (an adapter that does not touch a
 *      slice has rank 0 there).
 * One GEMM over the stacked W, one shrink and one expand launch cover all
 * slices (x is read once by the shrink).  A row is adapted only if its
 * adapter is valid in every slice (else it is counted and gets the base).
 * lora_linear is this call with one slice.
 * Folded shrink: for bf16 with every slice's adapters in SLOTS (16-byte
 * aligned A) or in pools whose pages hold whole A rows, the MFMA path, a
 * shape whose base GEMM runs 128 x 144 tiles (sum_i d_i a multiple of 144,
 * e.g. the q + v pair of a 70B layer at 512 rows) or 64 x 64 tiles (decode
 * batches, e.g. 256 rows x 4096 columns), and n_slices * n_adapters *
 * max_rank <= 32 x the GEMM's column tiles, the base GEMM also computes
 * t = x A^T for every (slice, adapter, rank) and no shrink is launched:
 * each column tile takes 16 of those columns in its k loop, and where they
 * number more than 16 x the column tiles, 16 more in a slower second pass.
 * (128 x 144 tiles list the ranks below each adapter's rank, clamped to
 * [0, max_rank]; 64 x 64 tiles every rank below max_rank, the columns past
 * an adapter's rank computed and never read.)  LORA_FLAG_SEPARATE_SHRINK
 * turns the folding off.  Results agree with the separate shrink to fp32
 * rounding (t is summed in another order).
 */
#define LORA_MAX_SLICES 4
typedef struct lora_slice {
  int64_t d;                 /* output columns of this slice */
  const float *scales;       /* device fp32 [n_adapters] */
  lora_adapters_t adapters;  /* this slice's adapter set */
} lora_slice_t;

size_t lora_workspace_bytes_sliced(int64_t max_rows, int64_t k, lora_dtype_t dtype,
                                   int32_t n_slices, const lora_slice_t *slices);

lora_status_t lora_linear_sliced(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                 int64_t ldx, const void *W, int64_t ldw, int32_t n_slices,
                                 const lora_slice_t *slices, const int32_t *adapter_ids, void *y,
                                 int64_t ldy, void *workspace, size_t workspace_bytes,
                                 int32_t path, uint32_t flags, void *stream);

/*
 * lora_linear_sliced without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP-graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * lora_linear_sliced (bitwise: the same kernels run), except:
 *   - the plan regions, shrink partials and the base GEMM's split-K partials
 *     live in a static device array of LORA_NOALLOC_SCRATCH_BYTES that the
 *     library holds on every GPU it runs on until the process ends; a call
 *     whose workspace need (lora_workspace_bytes_sliced) exceeds it returns
 *     LORA_ERR_WORKSPACE and launches nothing;
 *   - the call allocates nothing (no hipMalloc / hipFree, no stream or event
 *     creation): the plan runs inside the base GEMM's launch where it can,
 *     else on `stream` ahead of the GEMM (never on the side stream), and
 *     launches are not timed by lora_profile_*;
 *   - every call on one GPU shares that GPU's array and its contents stay
 *     from the last call: calls that overlap on one GPU (two streams, two
 *     threads) race, so the caller serialises them; LORA_FLAG_REUSE_PLAN
 *     reuses the last plan made in the array;
 *   - the device error counters it keeps are not reported (use
 *     lora_linear_sliced with a workspace and lora_check to read them).
 * The first call on a device looks up the array's device address there
 * (make that call outside any graph capture).
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lora_status_t lora_linear_sliced_noalloc(lora_dtype_t dtype, int64_t M, int64_t k, const void *x,
                                         int64_t ldx, const void *W, int64_t ldw,
                                         int32_t n_slices, const lora_slice_t *slices,
                                         const int32_t *adapter_ids, void *y, int64_t ldy,
                                         int32_t path, uint32_t flags, void *stream);

/*
 * Quantized base weight (bf16 activations and adapters; the base GEMM
 * dequantizes on the fly).  "Your LoRA Adapters Are Thrashing Your GPUs",
 * section 02: production deployments quantize the base model to INT4 or INT8
 * and keep the LoRA weights in 16 bits.  Symmetric formats (no zero point):
 *   LORA_W_INT8: q int8 [d, ldq bytes], scales fp32 [d]:
 *       W[n, j] = scales[n] * q[n, j]; the scale multiplies the fp32 dot
 *       product (the dequantized weight is exact).
 *   LORA_W_INT4: q two's-complement 4-bit values, two per byte, element 2i of
 *       a row in the low nibble of byte i, element 2i + 1 in the high nibble;
 *       scales fp32 [d, k / group]:
 *       W[n, j] = scales[n * (k / group) + j / group] * q[n, j]; each
 *       q * scale is rounded once to bf16 before the MFMA.
 * group: INT4 k-group, a multiple of 64 that divides k (INT8: ignored).
 * ldq: row stride in bytes, a multiple of 16, >= k (INT8) or k / 2 (INT4).
 * q and scales are device memory; q 16-byte aligned.  k % 64 == 0.
 */
typedef enum lora_wformat {
  LORA_W_INT8 = 1,
  LORA_W_INT4 = 2
} lora_wformat_t;

typedef struct lora_qweight {
  int32_t format;       /* lora_wformat_t */
  int32_t group;        /* INT4 k-group size */
  const void *q;        /* device, packed weights [d, ldq] */
  int64_t ldq;          /* bytes */
  const float *scales;  /* device fp32: INT8 [d]; INT4 [d, k / group] */
} lora_qweight_t;

/* y = x dequant(W)^T, bf16 x [M, k] and y [M, d] (as lora_gemm). */
lora_status_t lora_gemm_q(int64_t M, int64_t k, int64_t d, const void *x, int64_t ldx,
                          const lora_qweight_t *W, void *y, int64_t ldy, void *stream);

/*
 * lora_linear_sliced with a quantized base weight: W stacks the slices'
 * quantized weights by rows ([sum_i d_i] rows, scales stacked alike); the
 * adapters, ids, workspace (lora_workspace_bytes_sliced with bf16) and every
 * other argument as in lora_linear_sliced.  bf16 only.
 */
lora_status_t lora_linear_sliced_q(int64_t M, int64_t k, const void *x, int64_t ldx,
                                   const lora_qweight_t *W, int32_t n_slices,
                                   const lora_slice_t *slices, const int32_t *adapter_ids, void *y,
                                   int64_t ldy, void *workspace, size_t workspace_bytes,
                                   int32_t path, uint32_t flags, void *stream);

/*
 * The plan step alone (what lora_linear runs first): classify rows, sort
 * the adapted rows by (adapter, row) -- stable -- and build the segment
 * table.  "Adapter Residency ...", "Batch composition under many adapters":
 * rows sorted by adapter before the forward pass, each adapter's rows
 * contiguous.  d and k are needed only to check page counts of a pool.
 * M <= LORA_PLAN_MAX_ROWS.
 */
#define LORA_PLAN_MAX_ROWS 8192
lora_status_t lora_plan(int64_t M, int64_t k, int64_t d, lora_dtype_t dtype,
                        const lora_adapters_t *adapters, const int32_t *adapter_ids,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Device pointers into a workspace holding a plan (no device access). */
typedef struct lora_plan_view {
  const int32_t *counters;     /* [0] bad ids [1] bad ranks [2] bad pages [3] n_adapted
                                  [4] n_segments [5] gather items [6] sgmv items [7] rows */
  const int32_t *perm;         /* [n_adapted]: adapted rows, sorted by (adapter, row) */
  const int32_t *seg_adapter;  /* [n_segments], ascending */
  const int32_t *seg_start;    /* [n_segments]: index into perm */
  const int32_t *seg_len;      /* [n_segments] */
  int64_t capacity_rows;       /* rows the view was laid out for */
} lora_plan_view_t;

lora_status_t lora_plan_view(const void *workspace, size_t workspace_bytes, int64_t M,
                             const lora_adapters_t *adapters, lora_plan_view_t *out);

/*
 * Merged weight of one adapter, for the single-adapter fast path:
 *   W_out = W + coef * scales[adapter] * B_a A_a        (W, W_out: [d, k])
 * "Your LoRA Adapters Are Thrashing Your GPUs", section 02 (weight merging vs
 * keeping adapters separate): with W' = W + (alpha/r) B A the layer is the
 * plain x W'^T, one adapter at a time; coef = 1 merges, coef = -1 takes a
 * merged adapter back out (up to the rounding of the two stores).  When
 * every row of a batch uses the same adapter, lora_gemm with the merged
 * weight replaces lora_linear.
 *   adapters: SLOTS or POOL set (the adapter's rank is read on the device);
 *   scales: device fp32 [n_adapters]; W, W_out: device, ldw / ldo >= k;
 *   W_out == W (same ldw) merges in place; other overlaps are LORA_ERR_ARG.
 * bf16: k, ldw, ldo multiples of 8, MFMA kernel, fp32 sum of the rank-r
 * product, one RNE rounding of W + coef*s*BA; fp32: multiples of 4, VALU.
 * A rank outside [0, max_rank] or missing pool pages (device-side errors)
 * leave W_out = W.  Asynchronous on `stream`.
 */
lora_status_t lora_merge(lora_dtype_t dtype, int64_t d, int64_t k, const void *W, int64_t ldw,
                         const lora_adapters_t *adapters, int32_t adapter, const float *scales,
                         float coef, void *W_out, int64_t ldo, void *stream);

/*
 * Page-table translation as the kernels do it ("S-LoRA: what the paper
 * actually says ...", "Unified paging": an adapter's weights sit in
 * fixed-size blocks of one pool, located through that adapter's block
 * list), exported for bit-exact checks:
 * phys_off[i] = page_table[adapter[i]][logical_off[i] / page_bytes] * page_bytes
 *               + logical_off[i] % page_bytes,
 * or -1 when adapter[i] is outside [0, n_adapters), the logical page is past
 * max_pages, or the entry is outside [0, n_pages).
 * adapter, logical_off, phys_off: device arrays of n entries.  POOL only.
 */
lora_status_t lora_translate(const lora_adapters_t *adapters, const int32_t *adapter,
                             const int64_t *logical_off, int64_t n, int64_t *phys_off,
                             void *stream);

/*
 * Device-side error report of a workspace.  The per-row counts follow the
 * readings of "LoRA Adapters: Many Models in One", "The model runner's part"
 * (a per-token slot index, or none) and "S-LoRA: ...", "Unified paging" (an
 * adapter's blocks found through its page list): a row whose id, rank or
 * pages cannot be used is served as a row without adapter and counted.
 *
 * Synchronises `stream`, then reads:
 *   n_bad_ids, n_bad_ranks, n_bad_pages -- counts of the last plan run in
 *     this workspace: rows with an id outside [-1, n_adapters), rows whose
 *     adapter rank is outside [0, max_rank], rows whose adapter pages are
 *     missing or outside the pool;
 *   n_sync_expired -- split-K workgroup pairs of the base GEMM whose second
 *     half stopped waiting for the first half's partial (a bounded wait of
 *     ~0.3 s; that output tile is wrong).  Cumulative since the workspace
 *     was zero-filled: lora_linear* count it at word 8 of the workspace,
 *     lora_gemm at word 8 of its own workspace.  Zero-fill a workspace once
 *     when allocating it for this count to mean anything; 0 in normal runs.
 * Output pointers are HOST and may be NULL.
 */
lora_status_t lora_check(const void *workspace, void *stream, int64_t *n_bad_ids,
                         int64_t *n_bad_ranks, int64_t *n_bad_pages, int64_t *n_sync_expired);

/*
 * Testing hook for the error path of the split-K pairs (no page defines
 * it).  Sets the bound, in polls, of the second workgroup's wait in later
 * launches; 0 makes every such wait expire at once (wrong tiles, counted as
 * n_sync_expired, every workgroup exits normally); a negative value restores
 * the default.  Process-wide; not for production use.
 */
lora_status_t lora_test_sync_spin_limit(int32_t polls);

/*
 * Per-kernel GPU timing.  While enabled, every kernel that lora_linear /
 * lora_gemm / lora_plan launches is bracketed by two hipEvents recorded on
 * the launch stream; lora_profile_read synchronises on those events and
 * accumulates elapsed time per kernel class.  Disabled by default.  The
 * library creates its events once (lazily) and keeps them until unload.
 */
typedef enum lora_kernel_class {
  LORA_K_PLAN = 0,
  LORA_K_GEMM = 1,
  LORA_K_SHRINK = 2,        /* gather-path shrink */
  LORA_K_EXPAND = 3,        /* gather-path expand */
  LORA_K_SGMV_SHRINK = 4,
  LORA_K_SGMV_EXPAND = 5,
  LORA_K_COUNT = 6
} lora_kernel_class_t;

typedef struct lora_profile {
  double ms[LORA_K_COUNT];      /* summed kernel time per class */
  int64_t launches[LORA_K_COUNT];
  int64_t dropped;              /* launches not timed because the event ring was full */
} lora_profile_t;

lora_status_t lora_profile_enable(int32_t on);
lora_status_t lora_profile_read(lora_profile_t *out, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* LORA_ROW_H */
