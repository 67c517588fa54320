"""Reference model of adapter activation into a paged pool (plain Python).

TEST INFRASTRUCTURE ONLY: imported by the test suite alone.  It shares no
code with the HIP library and never imports it.

What it models, and where the pages say it:
  * "S-LoRA: what the paper actually says about serving thousands of LoRA
    adapters", section "Unified paging": an adapter's weights occupy
    fixed-size pages of one pool and the adapter keeps the list of its
    pages.  Reading taken here: the adapter's A (r x k) then B (d x r),
    unpadded, fill ceil(r (k + d) elem_bytes / page_bytes) pages; the lowest
    numbered free pages are taken (the pages leave the choice open; lowest
    first is the plainest deterministic one).
  * "Your LoRA Adapters Are Thrashing Your GPUs", section 05 "Multi-Adapter
    Serving": when the slots are full a new adapter evicts the least
    recently used one; pinned adapters stay resident and are never evicted.
  * "Multi-LoRA Adapter Caching in Production ...", section "Core Principle:
    Treat LoRA as a Tiered Cache": a hit refreshes the adapter's recency;
    an adapter that running work still uses is not evicted (here: pinned,
    with a reference count).
  * Batches (the pages do not define them; reading taken here): the loads
    of one batch run in order, none of them evicts an adapter of the same
    batch, and a batch that cannot be placed whole changes nothing -- the
    adapters a batch of requests needs are resident together or not at all.

Each operation returns the same status codes as the library's C ABI
(0 ok, 1 bad argument, 4 bad rank, 6 pages) and, on an error, changes
nothing.  ``mutant`` plants one deliberate mistake (pin tests only).
"""
from __future__ import annotations

import copy

OK, ERR_ARG, ERR_RANK, ERR_PAGE = 0, 1, 4, 6

MUTANTS = {
    1: "most recently used evicted",
    2: "pins ignored by eviction",
    3: "highest-numbered free pages taken",
    4: "page count rounded down",
    5: "a hit does not refresh recency",
    6: "a failed batch keeps its first loads",
    7: "a batch evicts its own adapters",
}


class PoolModel:
    def __init__(self, n_pages: int, page_bytes: int, n_adapters: int, max_pages: int,
                 max_rank: int, k: int, d: int, elem_bytes: int, mutant: int = 0):
        self.n_pages, self.page_bytes = n_pages, page_bytes
        self.n_adapters, self.max_pages, self.max_rank = n_adapters, max_pages, max_rank
        self.k, self.d, self.elem_bytes = k, d, elem_bytes
        self.mutant = mutant
        self.free = [True] * n_pages          # page -> free?
        self.rank = [-1] * n_adapters         # -1: not resident
        self.pins = [0] * n_adapters
        self.pages = [[] for _ in range(n_adapters)]
        self.last_use = [0] * n_adapters      # a larger value is more recent
        self.clock = 0
        self.loads = self.evictions = self.bytes_copied = 0
        self.evicted_log = []                 # adapters in eviction order

    # -- sizes ("Unified paging") -------------------------------------------
    def adapter_bytes(self, r: int) -> int:
        return r * (self.k + self.d) * self.elem_bytes

    def pages_needed(self, r: int) -> int:
        b = self.adapter_bytes(r)
        if self.mutant == 4:
            return b // self.page_bytes
        return -(-b // self.page_bytes)

    # -- helpers ------------------------------------------------------------
    def _tick(self, a: int) -> None:
        self.clock += 1
        self.last_use[a] = self.clock

    def resident(self, a: int) -> bool:
        return self.rank[a] >= 0

    def n_free(self) -> int:
        return sum(self.free)

    def _release(self, a: int) -> None:
        for p in self.pages[a]:
            self.free[p] = True
        self.pages[a] = []
        self.rank[a] = -1

    def _lru_order(self, protected):
        """Adapters that may be evicted, least recently used first: resident,
        holding pages (rank 0 frees nothing), not pinned, not protected."""
        cands = [a for a in range(self.n_adapters)
                 if a not in protected and self.pages[a] and (self.pins[a] == 0 or self.mutant == 2)]
        return sorted(cands, key=lambda a: self.last_use[a], reverse=(self.mutant == 1))

    # -- operations ---------------------------------------------------------
    def load(self, a: int, r: int) -> int:
        return self.load_batch([(a, r)])

    def load_batch(self, reqs) -> int:
        """Loads in order; adapters of the batch are not evicted for later
        ones of the batch; all or nothing (an error leaves the state as it
        was)."""
        reqs = [(int(a), int(r)) for a, r in reqs]
        for i, (a, r) in enumerate(reqs):
            if not 0 <= a < self.n_adapters:
                return ERR_ARG
            if not 0 <= r <= self.max_rank:
                return ERR_RANK
            if self.pages_needed(r) > self.max_pages:
                return ERR_PAGE
            if any(b == a for b, _ in reqs[:i]):
                return ERR_ARG
        members = {a for a, _ in reqs}
        if len(reqs) == 1:  # a single load fails before it changes anything
            return self._load_one(reqs[0][0], reqs[0][1], members)
        trial = self if self.mutant == 6 else copy.deepcopy(self)
        for a, r in reqs:
            rc = trial._load_one(a, r, {a} if self.mutant == 7 else members)
            if rc != OK:
                return rc
        self.__dict__.update(trial.__dict__)
        return OK

    def _load_one(self, a: int, r: int, protected) -> int:
        need = self.pages_needed(r)
        if not (self.resident(a) and len(self.pages[a]) == need):
            if self.resident(a) and self.pins[a] > 0:
                return ERR_ARG  # a pinned adapter's pages may not move
            avail = self.n_free() + (len(self.pages[a]) if self.resident(a) else 0)
            victims = []
            for v in self._lru_order(protected):
                if avail >= need:
                    break
                victims.append(v)
                avail += len(self.pages[v])
            if avail < need:
                return ERR_PAGE
            if self.resident(a):
                self._release(a)
            for v in victims:
                self._release(v)
                self.evictions += 1
                self.evicted_log.append(v)
            order = range(self.n_pages - 1, -1, -1) if self.mutant == 3 else range(self.n_pages)
            got = [p for p in order if self.free[p]][:need]
            for p in got:
                self.free[p] = False
            self.pages[a] = got
        self.rank[a] = r
        self._tick(a)
        self.loads += 1
        self.bytes_copied += self.adapter_bytes(r)
        return OK

    def evict(self, a: int) -> int:
        if not 0 <= a < self.n_adapters:
            return ERR_ARG
        if not self.resident(a):
            return OK
        if self.pins[a] > 0:
            return ERR_ARG
        self._release(a)
        self.evictions += 1
        self.evicted_log.append(a)
        return OK

    def touch(self, ids) -> int:
        if any(not 0 <= a < self.n_adapters for a in ids):
            return ERR_ARG
        for a in ids:
            if self.resident(a) and self.mutant != 5:
                self._tick(a)
        return OK

    def pin(self, ids) -> int:
        if any(not 0 <= a < self.n_adapters or not self.resident(a) for a in ids):
            return ERR_ARG
        for a in ids:
            self.pins[a] += 1
            self._tick(a)
        return OK

    def unpin(self, ids) -> int:
        if any(not 0 <= a < self.n_adapters for a in ids):
            return ERR_ARG
        for a in set(ids):
            if list(ids).count(a) > self.pins[a]:
                return ERR_ARG
        for a in ids:
            self.pins[a] -= 1
        return OK

    def query(self, a: int) -> dict:
        return {"resident": self.resident(a), "rank": self.rank[a], "pins": self.pins[a],
                "n_pages": len(self.pages[a]), "pages": list(self.pages[a])}

    def stats(self) -> dict:
        return {"loads": self.loads, "evictions": self.evictions,
                "bytes_copied": self.bytes_copied, "free_pages": self.n_free(),
                "resident": sum(1 for a in range(self.n_adapters) if self.resident(a))}

    def page_table(self):
        """The device page table the pool should hold: [n_adapters][max_pages]."""
        return [self.pages[a] + [-1] * (self.max_pages - len(self.pages[a]))
                for a in range(self.n_adapters)]
