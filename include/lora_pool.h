/*
 * lora_pool.h -- adapter activation into a paged device pool (C ABI, part of
 * liblora_row.so).
 *
 * The step before the LoRA linear layer: making an adapter's weights
 * resident on the device so lora_linear can use them through the POOL form
 * of lora_adapters_t (include/lora_row.h).
 *
 *   - "S-LoRA: what the paper actually says about serving thousands of LoRA
 *     adapters", section "Unified paging": adapter weights live in
 *     fixed-size blocks of one device pool and each adapter keeps the list of
 *     its blocks.
 *   - "Multi-LoRA Adapter Caching in Production ...", sections "Core
 *     Principle: Treat LoRA as a Tiered Cache" (replace the least recently
 *     used adapter when the device slots are full, refresh recency on a hit,
 *     never evict an adapter that running work still uses) and "Cold-Load
 *     Latency Should Be Categorized into Tiers" (an adapter held in host
 *     memory costs one host-to-device upload); "Why Pure LRU Fails in
 *     Multi-Tenant Scenarios" (pin hot adapters).
 *   - "Your LoRA Adapters Are Thrashing Your GPUs", sections 03 "The True
 *     Cost of an Adapter Swap" (the PCIe transfer time of an adapter) and 05
 *     "Multi-Adapter Serving" (LRU eviction by default; pinned adapters are
 *     never evicted).
 *
 * Model.  A manager owns the bookkeeping of a caller-owned device pool of
 * n_pages pages of page_bytes bytes, the caller-owned device page table
 * (int32 [n_adapters, max_pages]) and the caller-owned device rank array
 * (int32 [n_adapters]).  Adapter a's logical byte space is A_a (r x k,
 * row-major) followed by B_a (d x r, row-major), both unpadded, elements of
 * elem_bytes bytes -- exactly the POOL layout lora_linear reads.  Loading an
 * adapter takes ceil(r (k + d) elem_bytes / page_bytes) pages, the
 * lowest-numbered free ones; when too few are free, resident adapters that
 * are not pinned are evicted, least recently used first.  Pinned adapters
 * (reference counted; e.g. those of a batch in flight) are never evicted.
 *
 * Device updates are asynchronous on the given stream, in this order: one
 * kernel writes the page-table rows and ranks of every adapter the call
 * loads or evicts, then one kernel copies the weights of all adapters of
 * the call into their pages, reading the caller's host memory directly
 * over the host link (one workgroup per chunk of up to 64 KiB).  This needs
 * host memory the device can address -- pinned memory from hipHostMalloc
 * (torch's pin_memory) -- which must stay valid until the stream reaches
 * the copy.  Any other host memory is copied with hipMemcpyAsync instead
 * (one copy per run of consecutive pages) and the call waits for those
 * copies before returning.  An adapter that is not resident (never loaded,
 * or evicted) has rank -1 and a page-table row of -1, so rows that name it
 * are counted as bad ranks by the plan (lora_check) and read nothing.  The
 * caller orders kernels that use the pool after the loads (same stream, or
 * an event).  Pages freed by an eviction are reused by later loads in
 * stream order: work on other streams that still reads an adapter must
 * keep it pinned.
 *
 * Accounting-only mode: with pool, page_table and ranks all NULL the
 * manager does every placement / LRU / pinning decision but touches no
 * device memory (for capacity planning and tests).
 *
 * Thread safety: one manager may be used from several host threads (calls
 * are serialised by a lock inside it).  Errors: LORA_ERR_ARG (NULL or
 * out-of-range argument, pin of a non-resident adapter, unpin below zero,
 * eviction of a pinned adapter), LORA_ERR_RANK (rank outside 0..max_rank),
 * LORA_ERR_PAGE (an adapter needs more than max_pages pages, or not enough
 * pages can be freed -- then nothing has changed), LORA_ERR_HIP (a kernel or
 * copy failed to enqueue; the host bookkeeping has then already changed).
 * Host weights must be aligned to elem_bytes (LORA_ERR_ARG otherwise).
 */
#ifndef LORA_POOL_H
#define LORA_POOL_H

#include <stdint.h>

#include "lora_row.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lora_pool lora_pool_t; /* opaque host object */

typedef struct lora_pool_desc {
  void *pool;          /* device bytes [n_pages * page_bytes], or NULL (accounting only) */
  int32_t *page_table; /* device int32 [n_adapters * max_pages], or NULL */
  int32_t *ranks;      /* device int32 [n_adapters], or NULL */
  int64_t n_pages;     /* 1 .. 2^31 - 1 */
  int64_t page_bytes;  /* power of two >= 256 */
  int32_t n_adapters;  /* adapter ids 0 .. n_adapters - 1 */
  int32_t max_pages;   /* columns of the page table */
  int32_t max_rank;    /* 1 .. 256 */
  int32_t elem_bytes;  /* 2 (bf16) or 4 (fp32) */
  int64_t k;           /* A is r x k */
  int64_t d;           /* B is d x r */
} lora_pool_desc_t;

typedef struct lora_pool_stats {
  int64_t loads;        /* successful lora_pool_load calls */
  int64_t evictions;    /* adapters evicted (LRU or explicit) */
  int64_t bytes_copied; /* host-to-device weight bytes of those loads */
  int64_t free_pages;
  int64_t resident;     /* adapters resident now */
} lora_pool_stats_t;

/*
 * Create a manager.  With device pointers, the page table and the ranks are
 * set to -1 (asynchronously on `stream`).  *out receives the manager.
 */
lora_status_t lora_pool_create(const lora_pool_desc_t *desc, void *stream, lora_pool_t **out);

/* Destroy a manager (host memory only; the device buffers stay the caller's). */
void lora_pool_destroy(lora_pool_t *pool);

/*
 * The POOL adapter set that lora_linear / lora_plan read (host struct filled
 * from the descriptor).
 */
lora_status_t lora_pool_adapters(const lora_pool_t *pool, lora_adapters_t *out);

/*
 * Make `adapter` resident with rank `rank`, copying A (host, rank x k) and
 * B (host, d x rank), both row-major in elem_bytes-sized elements, into its
 * pages.  An adapter that is already resident keeps its pages if the new
 * rank needs the same number, else it is re-placed (LORA_ERR_ARG if it is
 * pinned).  Rank 0 (an adapter that does not touch this projection) takes
 * no pages and copies nothing; host_A / host_B may then be NULL.  Counts as
 * a use (LRU).  Eviction candidates are the unpinned adapters holding pages.
 */
lora_status_t lora_pool_load(lora_pool_t *pool, int32_t adapter, int32_t rank, const void *host_A,
                             const void *host_B, void *stream);

/*
 * Several loads in one call: the same as lora_pool_load for adapters[i] in
 * order, except that (a) no adapter of the batch is evicted to make room
 * for a later one, (b) the batch is all or nothing: if one load fails (bad
 * argument, a pinned adapter that would have to move, too few pages) the
 * call returns its error and nothing has changed, and (c) the device work
 * is one rows kernel and one copy kernel for the whole batch (more only if
 * the batch is large).  adapters, ranks, host_A, host_B: host arrays of n
 * entries (an adapter at most once); host_A / host_B may be NULL in
 * accounting-only mode.
 */
lora_status_t lora_pool_load_batch(lora_pool_t *pool, int32_t n, const int32_t *adapters,
                                   const int32_t *ranks, const void *const *host_A,
                                   const void *const *host_B, void *stream);

/* Evict `adapter` now (LORA_ERR_ARG if it is pinned; OK if not resident). */
lora_status_t lora_pool_evict(lora_pool_t *pool, int32_t adapter, void *stream);

/* Mark resident adapters as used (LRU order); host array of n ids. */
lora_status_t lora_pool_touch(lora_pool_t *pool, const int32_t *adapters, int32_t n);

/*
 * Pin / unpin resident adapters (host array of n ids; reference counted).
 * Pinning also counts as a use.  All-or-nothing: on error nothing changes.
 */
lora_status_t lora_pool_pin(lora_pool_t *pool, const int32_t *adapters, int32_t n);
lora_status_t lora_pool_unpin(lora_pool_t *pool, const int32_t *adapters, int32_t n);

/*
 * State of one adapter: resident flag, rank, pin count, pages used, and (if
 * pages_out is not NULL) its physical pages in logical order, -1 after the
 * last (host int32 [max_pages]).  Output pointers may be NULL.
 */
lora_status_t lora_pool_query(const lora_pool_t *pool, int32_t adapter, int32_t *resident,
                              int32_t *rank, int32_t *pins, int32_t *n_pages, int32_t *pages_out);

lora_status_t lora_pool_get_stats(const lora_pool_t *pool, lora_pool_stats_t *out);

#ifdef __cplusplus
}
#endif

#endif /* LORA_POOL_H */
