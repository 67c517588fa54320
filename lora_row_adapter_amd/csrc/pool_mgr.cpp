// pool_mgr.cpp -- host side of include/lora_pool.h: making adapters resident
// in a paged device pool.
//
// "S-LoRA: ...", section "Unified paging": adapter weights occupy fixed-size
// pages of one pool and each adapter keeps the list of its pages.
// "Multi-LoRA Adapter Caching in Production ...", sections "Core Principle:
// Treat LoRA as a Tiered Cache" and "Why Pure LRU Fails in Multi-Tenant
// Scenarios", and "Your LoRA Adapters Are Thrashing Your GPUs", section 05
// "Multi-Adapter Serving": when the device is full the least recently used
// adapter that is not in use (not pinned) makes room; a hit refreshes its
// recency.  Only adapters that hold pages are eviction candidates (a rank-0
// adapter, which does not touch this projection, frees nothing).
//
// Placement state lives on the host (free pages as a map of free runs, so the
// lowest-numbered free pages are found by walking it in order; one page list,
// rank, pin count and last-use stamp per adapter).  A batch of loads is first
// played on a copy of that state, so a batch that cannot be placed changes
// nothing; then the device work is queued on the caller's stream:
// k_pool_rows writes the page-table rows and ranks, k_pool_pull copies the
// weights from pinned host memory into the pages.  Host memory the device
// cannot address (pageable) goes through hipMemcpyAsync instead, one copy per
// run of consecutive pages, and the call then waits for its copies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "lora_pool.h"
#include "kernels.hpp"

namespace {

struct State {
  std::map<int64_t, int64_t> free_runs;  // first page -> run length
  int64_t n_free = 0;
  std::vector<int32_t> rank;             // -1: not resident
  std::vector<int32_t> pins;
  std::vector<uint64_t> last_use;
  std::vector<std::vector<int32_t>> pages;
  uint64_t clock = 0;
  int64_t n_resident = 0;
  lora_pool_stats_t stats{};
};

}  // namespace

struct lora_pool {
  lora_pool_desc_t desc;
  bool device = false;  // false: accounting only
  std::mutex mu;
  State s;
};

namespace {

using lora::PoolPullArgs;
using lora::PoolRowsArgs;

struct LoadReq {
  int32_t adapter;
  int32_t rank;
  const uint8_t *A;
  const uint8_t *B;
};

int64_t adapter_bytes(const lora_pool_desc_t &d, int64_t r) {
  return r * (d.k + d.d) * d.elem_bytes;
}

int64_t pages_needed(const lora_pool_desc_t &d, int64_t r) {
  return (adapter_bytes(d, r) + d.page_bytes - 1) / d.page_bytes;
}

// Take the `n` lowest-numbered free pages (caller checked n <= n_free).
std::vector<int32_t> take_pages(State &s, int64_t n) {
  std::vector<int32_t> out;
  out.reserve((size_t)n);
  while ((int64_t)out.size() < n) {
    auto it = s.free_runs.begin();
    const int64_t first = it->first, len = it->second;
    const int64_t use = std::min<int64_t>(len, n - (int64_t)out.size());
    for (int64_t i = 0; i < use; ++i) out.push_back((int32_t)(first + i));
    s.free_runs.erase(it);
    if (use < len) s.free_runs.emplace(first + use, len - use);
  }
  s.n_free -= n;
  return out;
}

// Return one page, merging it with the free runs on either side.
void give_page(State &s, int64_t pg) {
  auto next = s.free_runs.lower_bound(pg);
  int64_t first = pg, len = 1;
  if (next != s.free_runs.begin()) {
    auto prev = std::prev(next);
    if (prev->first + prev->second == pg) {
      first = prev->first;
      len += prev->second;
      s.free_runs.erase(prev);
    }
  }
  if (next != s.free_runs.end() && next->first == pg + 1) {
    len += next->second;
    s.free_runs.erase(next);
  }
  s.free_runs.emplace(first, len);
  ++s.n_free;
}

void drop_adapter(State &s, int32_t a) {
  for (int32_t pg : s.pages[a]) give_page(s, pg);
  s.pages[a].clear();
  s.rank[a] = -1;
  --s.n_resident;
}

bool valid_id(const lora_pool_desc_t &d, int32_t a) { return a >= 0 && a < d.n_adapters; }

// Plays the loads on `s` in order.  Adapters of the batch are never evicted
// by later loads of the same batch.  Appends evicted adapters to `victims`.
lora_status_t place_batch(const lora_pool_desc_t &d, State &s, const LoadReq *req, int32_t n,
                          std::vector<int32_t> &victims) {
  std::vector<char> member((size_t)d.n_adapters, 0);
  for (int32_t i = 0; i < n; ++i) member[req[i].adapter] = 1;
  std::vector<int32_t> cand;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t a = req[i].adapter;
    const int64_t need = pages_needed(d, req[i].rank);
    const bool resident = s.rank[a] >= 0;
    if (!(resident && (int64_t)s.pages[a].size() == need)) {
      if (resident && s.pins[a] > 0) return LORA_ERR_ARG;  // pinned pages cannot move
      // Victims: unpinned adapters outside the batch that hold pages, least
      // recently used first, until enough pages would be free.
      int64_t avail = s.n_free + (resident ? (int64_t)s.pages[a].size() : 0);
      size_t first_victim = victims.size();
      if (avail < need) {
        cand.clear();
        for (int32_t b = 0; b < d.n_adapters; ++b)
          if (!member[b] && !s.pages[b].empty() && s.pins[b] == 0) cand.push_back(b);
        std::sort(cand.begin(), cand.end(),
                  [&](int32_t x, int32_t y) { return s.last_use[x] < s.last_use[y]; });
        for (int32_t b : cand) {
          if (avail >= need) break;
          victims.push_back(b);
          avail += (int64_t)s.pages[b].size();
        }
        if (avail < need) return LORA_ERR_PAGE;
      }
      if (resident) drop_adapter(s, a);
      for (size_t v = first_victim; v < victims.size(); ++v) {
        drop_adapter(s, victims[v]);
        ++s.stats.evictions;
      }
      s.pages[a] = take_pages(s, need);
      ++s.n_resident;
    }
    s.rank[a] = req[i].rank;
    s.last_use[a] = ++s.clock;
    ++s.stats.loads;
    s.stats.bytes_copied += adapter_bytes(d, req[i].rank);
  }
  return LORA_OK;
}

// Device-visible address of host memory the GPU can read directly (memory
// from hipHostMalloc), or nullptr (pageable memory, or not host memory).
const uint8_t *device_view(const void *ptr) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
    (void)hipGetLastError();  // an unregistered pointer is not an error here
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr || at.hostPointer == nullptr)
    return nullptr;
  return static_cast<const uint8_t *>(at.devicePointer) +
         (static_cast<const uint8_t *>(ptr) - static_cast<const uint8_t *>(at.hostPointer));
}

// Page-table rows (with ranks) of `adapters`, packed into as few k_pool_rows
// launches as the argument block allows.
hipError_t write_rows(const lora_pool_desc_t &d, const State &s, const std::vector<int32_t> &adapters,
                      hipStream_t st) {
  PoolRowsArgs r{};
  r.page_table = d.page_table;
  r.ranks = d.ranks;
  r.max_pages = d.max_pages;
  int32_t nv = 0;
  auto flush = [&]() -> hipError_t {
    const hipError_t e = lora::launch_pool_rows(r, st);
    r.n_rows = 0;
    nv = 0;
    return e;
  };
  for (int32_t a : adapters) {
    const std::vector<int32_t> &pg = s.pages[a];
    int32_t j = 0;
    do {
      if (r.n_rows == lora::kPoolRowsMax || nv == lora::kPoolRowVals) {
        const hipError_t e = flush();
        if (e != hipSuccess) return e;
      }
      const int32_t take = std::min<int32_t>((int32_t)pg.size() - j, lora::kPoolRowVals - nv);
      lora::PoolRow &row = r.row[r.n_rows++];
      row.adapter = a;
      row.rank = s.rank[a];
      row.n_vals = take;
      row.v0 = nv;
      row.j0 = j;
      row.last = j + take == (int32_t)pg.size();
      std::copy(pg.begin() + j, pg.begin() + j + take, r.v + nv);
      nv += take;
      j += take;
    } while (j < (int32_t)pg.size());
  }
  return r.n_rows > 0 ? flush() : hipSuccess;
}

int32_t log2_of(int64_t v) {
  int32_t l = 0;
  while (((int64_t)1 << l) < v) ++l;
  return l;
}

// Copy `bytes` host bytes to logical offset `off` of pages `pg` by DMA, one
// copy per run of consecutive physical pages.
hipError_t copy_logical(const lora_pool_desc_t &d, const std::vector<int32_t> &pg, int64_t off,
                        const uint8_t *src, int64_t bytes, hipStream_t st) {
  const int64_t pb = d.page_bytes;
  uint8_t *pool = static_cast<uint8_t *>(d.pool);
  while (bytes > 0) {
    const int64_t lp = off / pb;
    const int64_t in = off % pb;
    int64_t run_pages = 1;
    while (lp + run_pages < (int64_t)pg.size() && pg[lp + run_pages] == pg[lp] + run_pages &&
           run_pages * pb - in < bytes)
      ++run_pages;
    const int64_t n = std::min<int64_t>(bytes, run_pages * pb - in);
    const hipError_t e =
        hipMemcpyAsync(pool + (int64_t)pg[lp] * pb + in, src, (size_t)n, hipMemcpyDefault, st);
    if (e != hipSuccess) return e;
    off += n;
    src += n;
    bytes -= n;
  }
  return hipSuccess;
}

// Queue the device work of a placed batch: rows of victims and loaded
// adapters, then the weight copies.
lora_status_t queue_batch(const lora_pool_desc_t &d, const State &s, const LoadReq *req, int32_t n,
                          const std::vector<int32_t> &victims, hipStream_t st) {
  std::vector<int32_t> rows(victims);
  for (int32_t i = 0; i < n; ++i) rows.push_back(req[i].adapter);
  if (write_rows(d, s, rows, st) != hipSuccess) return LORA_ERR_HIP;
  PoolPullArgs p{};
  p.pool = static_cast<uint8_t *>(d.pool);
  p.page_table = d.page_table;
  p.max_pages = d.max_pages;
  p.log2_page = log2_of(d.page_bytes);
  p.log2_chunk = std::min<int32_t>(p.log2_page, 16);  // 64 KiB chunks inside a page
  bool wait = false;
  for (int32_t i = 0; i < n; ++i) {
    const LoadReq &q = req[i];
    if (q.rank == 0) continue;
    const int64_t a_bytes = (int64_t)q.rank * d.k * d.elem_bytes;
    const int64_t total = adapter_bytes(d, q.rank);
    const uint8_t *va = device_view(q.A);
    const uint8_t *vb = device_view(q.B);
    if (va == nullptr || vb == nullptr) {
      const std::vector<int32_t> &pg = s.pages[q.adapter];
      if (copy_logical(d, pg, 0, q.A, a_bytes, st) != hipSuccess ||
          copy_logical(d, pg, a_bytes, q.B, total - a_bytes, st) != hipSuccess)
        return LORA_ERR_HIP;
      wait = true;
      continue;
    }
    if (p.n_desc == lora::kPoolPullMax) {
      if (lora::launch_pool_pull(p, st) != hipSuccess) return LORA_ERR_HIP;
      p.n_desc = 0;
      p.n_chunks = 0;
    }
    lora::PoolPullDesc &D = p.d[p.n_desc++];
    D.a = va;
    D.b = vb;
    D.a_bytes = a_bytes;
    D.total = total;
    D.adapter = q.adapter;
    D.chunk0 = p.n_chunks;
    p.n_chunks += (int32_t)((total + ((int64_t)1 << p.log2_chunk) - 1) >> p.log2_chunk);
  }
  if (p.n_desc > 0 && lora::launch_pool_pull(p, st) != hipSuccess) return LORA_ERR_HIP;
  if (wait && hipStreamSynchronize(st) != hipSuccess) return LORA_ERR_HIP;
  return LORA_OK;
}

lora_status_t load_batch(lora_pool &p, const LoadReq *req, int32_t n, hipStream_t st) {
  const lora_pool_desc_t &d = p.desc;
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_id(d, req[i].adapter)) return LORA_ERR_ARG;
    if (req[i].rank < 0 || req[i].rank > d.max_rank) return LORA_ERR_RANK;
    if (p.device && req[i].rank > 0 &&
        (req[i].A == nullptr || req[i].B == nullptr ||
         (((uintptr_t)req[i].A | (uintptr_t)req[i].B) & (uintptr_t)(d.elem_bytes - 1)) != 0))
      return LORA_ERR_ARG;
    if (pages_needed(d, req[i].rank) > d.max_pages) return LORA_ERR_PAGE;
    for (int32_t j = 0; j < i; ++j)
      if (req[j].adapter == req[i].adapter) return LORA_ERR_ARG;
  }
  std::lock_guard<std::mutex> g(p.mu);
  State next = p.s;
  std::vector<int32_t> victims;
  const lora_status_t rc = place_batch(d, next, req, n, victims);
  if (rc != LORA_OK) return rc;
  p.s = std::move(next);
  if (!p.device) return LORA_OK;
  return queue_batch(d, p.s, req, n, victims, st);
}

}  // namespace

extern "C" {

lora_status_t lora_pool_create(const lora_pool_desc_t *desc, void *stream, lora_pool_t **out) {
  if (desc == nullptr || out == nullptr) return LORA_ERR_ARG;
  *out = nullptr;
  const lora_pool_desc_t &d = *desc;
  const int n_dev = (d.pool != nullptr) + (d.page_table != nullptr) + (d.ranks != nullptr);
  if (n_dev != 0 && n_dev != 3) return LORA_ERR_ARG;
  if (d.n_adapters < 1 || d.k < 1 || d.d < 1) return LORA_ERR_ARG;
  if (d.elem_bytes != 2 && d.elem_bytes != 4) return LORA_ERR_DTYPE;
  if (d.max_rank < 1 || d.max_rank > lora::kMaxRank) return LORA_ERR_RANK;
  if (d.n_pages < 1 || d.n_pages > INT32_MAX || d.page_bytes < 256 ||
      (d.page_bytes & (d.page_bytes - 1)) != 0 || d.max_pages < 1)
    return LORA_ERR_PAGE;
  if (n_dev == 3 && (((uintptr_t)d.pool & 255) != 0)) return LORA_ERR_ARG;
  lora_pool *p = new (std::nothrow) lora_pool;
  if (p == nullptr) return LORA_ERR_ARG;
  p->desc = d;
  p->device = n_dev == 3;
  State &s = p->s;
  s.free_runs.emplace(0, d.n_pages);
  s.n_free = d.n_pages;
  s.rank.assign((size_t)d.n_adapters, -1);
  s.pins.assign((size_t)d.n_adapters, 0);
  s.last_use.assign((size_t)d.n_adapters, 0);
  s.pages.resize((size_t)d.n_adapters);
  if (p->device) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (lora::launch_pool_fill(d.page_table, (int64_t)d.n_adapters * d.max_pages, -1, st) !=
            hipSuccess ||
        lora::launch_pool_fill(d.ranks, d.n_adapters, -1, st) != hipSuccess) {
      delete p;
      return LORA_ERR_HIP;
    }
  }
  *out = p;
  return LORA_OK;
}

void lora_pool_destroy(lora_pool_t *pool) { delete pool; }

lora_status_t lora_pool_adapters(const lora_pool_t *pool, lora_adapters_t *out) {
  if (pool == nullptr || out == nullptr) return LORA_ERR_ARG;
  const lora_pool_desc_t &d = pool->desc;
  *out = lora_adapters_t{};
  out->kind = LORA_ADAPTERS_POOL;
  out->n_adapters = d.n_adapters;
  out->max_rank = d.max_rank;
  out->max_pages = d.max_pages;
  out->ranks = d.ranks;
  out->pool = d.pool;
  out->page_table = d.page_table;
  out->page_bytes = d.page_bytes;
  out->n_pages = d.n_pages;
  return LORA_OK;
}

lora_status_t lora_pool_load(lora_pool_t *pool, int32_t adapter, int32_t rank, const void *host_A,
                             const void *host_B, void *stream) {
  if (pool == nullptr) return LORA_ERR_ARG;
  const LoadReq q{adapter, rank, static_cast<const uint8_t *>(host_A),
                  static_cast<const uint8_t *>(host_B)};
  return load_batch(*pool, &q, 1, static_cast<hipStream_t>(stream));
}

lora_status_t lora_pool_load_batch(lora_pool_t *pool, int32_t n, const int32_t *adapters,
                                   const int32_t *ranks, const void *const *host_A,
                                   const void *const *host_B, void *stream) {
  if (pool == nullptr || n < 0 || (n > 0 && (adapters == nullptr || ranks == nullptr)))
    return LORA_ERR_ARG;
  if (n > 0 && pool->device && (host_A == nullptr || host_B == nullptr)) return LORA_ERR_ARG;
  std::vector<LoadReq> req((size_t)n);
  for (int32_t i = 0; i < n; ++i)
    req[i] = LoadReq{adapters[i], ranks[i],
                     host_A ? static_cast<const uint8_t *>(host_A[i]) : nullptr,
                     host_B ? static_cast<const uint8_t *>(host_B[i]) : nullptr};
  return load_batch(*pool, req.data(), n, static_cast<hipStream_t>(stream));
}

lora_status_t lora_pool_evict(lora_pool_t *pool, int32_t adapter, void *stream) {
  if (pool == nullptr) return LORA_ERR_ARG;
  lora_pool &p = *pool;
  if (!valid_id(p.desc, adapter)) return LORA_ERR_ARG;
  std::lock_guard<std::mutex> g(p.mu);
  State &s = p.s;
  if (s.rank[adapter] < 0) return LORA_OK;
  if (s.pins[adapter] > 0) return LORA_ERR_ARG;
  drop_adapter(s, adapter);
  ++s.stats.evictions;
  if (!p.device) return LORA_OK;
  return write_rows(p.desc, s, {adapter}, static_cast<hipStream_t>(stream)) == hipSuccess
             ? LORA_OK
             : LORA_ERR_HIP;
}

lora_status_t lora_pool_touch(lora_pool_t *pool, const int32_t *adapters, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && adapters == nullptr)) return LORA_ERR_ARG;
  lora_pool &p = *pool;
  std::lock_guard<std::mutex> g(p.mu);
  for (int32_t i = 0; i < n; ++i)
    if (!valid_id(p.desc, adapters[i])) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (p.s.rank[adapters[i]] >= 0) p.s.last_use[adapters[i]] = ++p.s.clock;
  return LORA_OK;
}

lora_status_t lora_pool_pin(lora_pool_t *pool, const int32_t *adapters, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && adapters == nullptr)) return LORA_ERR_ARG;
  lora_pool &p = *pool;
  std::lock_guard<std::mutex> g(p.mu);
  for (int32_t i = 0; i < n; ++i)
    if (!valid_id(p.desc, adapters[i]) || p.s.rank[adapters[i]] < 0) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    ++p.s.pins[adapters[i]];
    p.s.last_use[adapters[i]] = ++p.s.clock;
  }
  return LORA_OK;
}

lora_status_t lora_pool_unpin(lora_pool_t *pool, const int32_t *adapters, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && adapters == nullptr)) return LORA_ERR_ARG;
  lora_pool &p = *pool;
  std::lock_guard<std::mutex> g(p.mu);
  std::vector<int32_t> count((size_t)p.desc.n_adapters, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_id(p.desc, adapters[i])) return LORA_ERR_ARG;
    if (++count[adapters[i]] > p.s.pins[adapters[i]]) return LORA_ERR_ARG;
  }
  for (int32_t i = 0; i < n; ++i) --p.s.pins[adapters[i]];
  return LORA_OK;
}

lora_status_t lora_pool_query(const lora_pool_t *pool, int32_t adapter, int32_t *resident,
                              int32_t *rank, int32_t *pins, int32_t *n_pages,
                              int32_t *pages_out) {
  if (pool == nullptr) return LORA_ERR_ARG;
  lora_pool &p = *const_cast<lora_pool *>(pool);
  if (!valid_id(p.desc, adapter)) return LORA_ERR_ARG;
  std::lock_guard<std::mutex> g(p.mu);
  const State &s = p.s;
  if (resident) *resident = s.rank[adapter] >= 0;
  if (rank) *rank = s.rank[adapter];
  if (pins) *pins = s.pins[adapter];
  const std::vector<int32_t> &pg = s.pages[adapter];
  if (n_pages) *n_pages = (int32_t)pg.size();
  if (pages_out)
    for (int32_t j = 0; j < p.desc.max_pages; ++j)
      pages_out[j] = j < (int32_t)pg.size() ? pg[j] : -1;
  return LORA_OK;
}

lora_status_t lora_pool_get_stats(const lora_pool_t *pool, lora_pool_stats_t *out) {
  if (pool == nullptr || out == nullptr) return LORA_ERR_ARG;
  lora_pool &p = *const_cast<lora_pool *>(pool);
  std::lock_guard<std::mutex> g(p.mu);
  *out = p.s.stats;
  out->free_pages = p.s.n_free;
  out->resident = p.s.n_resident;
  return LORA_OK;
}

}  // extern "C"
