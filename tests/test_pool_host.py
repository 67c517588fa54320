"""Adapter activation (paged pool manager) on the CPU.

1. The pool-policy model in oracle/pool_policy.py against what the pages
   print (tests/golden/lru_cascade.json) and hand-worked placements; every
   planted mistake in the model must fail one of these pins.
2. The library's manager (include/lora_pool.h) in accounting-only mode --
   the same placement / LRU / pinning code that drives the device copies,
   with no device memory -- against the model on seeded random operation
   sequences: every status, every adapter's pages and the counters must be
   identical.
"""
import json
import os

import numpy as np
import pytest

import lora_row_adapter_amd as lr
from oracle import pool_policy as pp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lru_cascade.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Pins of the model.  Each takes the model class's constructor (so the
# planted-mistake test can hand in a mutant) and raises AssertionError.
# ---------------------------------------------------------------------------

def one_slot_pool(make, slots, n_adapters):
    """Every adapter of rank 4 fills exactly one page: r (k + d) 2 B = 1 KiB."""
    return make(n_pages=slots, page_bytes=1024, n_adapters=n_adapters, max_pages=1, max_rank=4,
                k=64, d=64, elem_bytes=2)


def pin_eviction_cascade(make):
    g = golden()["eviction_cascade"]
    names = list(dict.fromkeys(g["initial_residents_lru_first"] +
                               [e["load"] for e in g["loads"]]))
    idx = {n: i for i, n in enumerate(names)}
    m = one_slot_pool(make, g["slots"], len(names))
    for n in g["initial_residents_lru_first"]:
        assert m.load(idx[n], 4) == pp.OK
    assert m.evicted_log == []
    for e in g["loads"]:
        before = len(m.evicted_log)
        assert m.load(idx[e["load"]], 4) == pp.OK
        got = [names[a] for a in m.evicted_log[before:]]
        assert got == [e["evicts"]], "load %s evicted %s, the page prints %s" % (
            e["load"], got, e["evicts"])


def pin_memory_budget(make):
    g = golden()["memory_budget"]
    page = 1 << 20
    for c in g["cases"]:
        # one adapter of adapter_mb (decimal) bytes: rank 1, k + d elements of 1 byte
        n_pages = g["available_gb"] * 10 ** 9 // page
        n = 400
        m = make(n_pages=n_pages, page_bytes=page, n_adapters=n, max_pages=1024, max_rank=1,
                 k=c["adapter_mb"] * 10 ** 6 // 2, d=c["adapter_mb"] * 10 ** 6 // 2, elem_bytes=1)
        a = 0
        while a < n and m.load(a, 1) == pp.OK and not m.evicted_log:
            a += 1
        # `a` adapters were resident when the next load first had to evict
        assert m.evicted_log == [0]
        printed = c["printed_slots"]
        assert abs(a - printed) <= 0.05 * printed, (a, printed)


def pin_pinned_burst(make):
    g = golden()["pinned_burst"]
    slots, hot, burst = g["slots"], g["hot"], g["burst"]
    for pinned in (0, 2):
        m = one_slot_pool(make, slots, hot + burst)
        for a in range(hot):
            assert m.load(a, 4) == pp.OK
        if pinned:
            assert m.pin(list(range(pinned))) == pp.OK
        for b in range(burst):
            assert m.load(hot + b, 4) == pp.OK
        alive = [a for a in range(hot) if m.query(a)["resident"]]
        assert alive == list(range(pinned)), (pinned, alive)
        assert m.stats()["resident"] == slots


def pin_lowest_pages_by_hand(make):
    # page 256 B; an adapter of rank r holds r (k + d) 2 = 128 r bytes:
    # r = 5 -> 640 B -> 3 pages, r = 8 -> 1024 B -> 4 pages.
    m = make(n_pages=10, page_bytes=256, n_adapters=6, max_pages=4, max_rank=8, k=32, d=32,
             elem_bytes=2)
    for a in range(3):
        assert m.load(a, 5) == pp.OK
    assert [m.query(a)["pages"] for a in range(3)] == [[0, 1, 2], [3, 4, 5], [6, 7, 8]]
    assert m.evict(1) == pp.OK
    assert m.load(3, 8) == pp.OK
    assert m.query(3)["pages"] == [3, 4, 5, 9]
    assert m.stats()["free_pages"] == 0
    # no page free: the least recently used (adapter 0) makes room
    assert m.load(4, 5) == pp.OK
    assert m.query(4)["pages"] == [0, 1, 2] and not m.query(0)["resident"]
    assert m.stats() == {"loads": 5, "evictions": 2, "bytes_copied": 640 * 4 + 1024,
                         "free_pages": 0, "resident": 3}


def pin_touch_refreshes(make):
    m = one_slot_pool(make, 4, 6)
    for a in range(4):
        assert m.load(a, 4) == pp.OK
    assert m.touch([0]) == pp.OK
    assert m.load(4, 4) == pp.OK
    assert not m.query(1)["resident"] and m.query(0)["resident"]


def pin_batch_by_hand(make):
    """A batch never evicts its own adapters, and fails whole."""
    m = one_slot_pool(make, 4, 8)
    for a in range(4):  # least recently used first: 0, 1, 2, 3
        assert m.load(a, 4) == pp.OK
    assert m.load_batch([(4, 4), (0, 4), (5, 4)]) == pp.OK
    # load 4 may not evict 0 (a member): 1 goes; 0 reloads in place; 5 evicts 2
    assert m.evicted_log == [1, 2]
    assert [a for a in range(8) if m.query(a)["resident"]] == [0, 3, 4, 5]
    assert m.pin([0, 4, 5]) == pp.OK
    # two new adapters, one unpinned slot (3): the second load fails, nothing changes
    before = [m.query(a) for a in range(8)], m.stats()
    assert m.load_batch([(6, 4), (7, 4)]) == pp.ERR_PAGE
    assert ([m.query(a) for a in range(8)], m.stats()) == before
    assert m.load_batch([(6, 4), (6, 4)]) == pp.ERR_ARG  # an adapter at most once


POOL_PINS = [pin_eviction_cascade, pin_memory_budget, pin_pinned_burst, pin_lowest_pages_by_hand,
             pin_touch_refreshes, pin_batch_by_hand]


@pytest.mark.parametrize("pin", POOL_PINS, ids=lambda f: f.__name__)
def test_pool_model_pin(pin):
    pin(pp.PoolModel)


@pytest.mark.parametrize("mutant", sorted(pp.MUTANTS),
                         ids=lambda m: pp.MUTANTS[m].replace(" ", "_"))
def test_pool_model_planted_mistake_is_caught(mutant):
    def make(**kw):
        return pp.PoolModel(mutant=mutant, **kw)

    caught = []
    for pin in POOL_PINS:
        try:
            pin(make)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % pp.MUTANTS[mutant]


def test_pool_model_invariants_random():
    """Pages of resident adapters are disjoint, sized by their rank, and with
    the free pages make up the whole pool; pinned adapters are never
    evicted; an evicted adapter was never more recently used than any
    unpinned adapter that stayed."""
    rng = np.random.default_rng(7)
    m = pp.PoolModel(n_pages=40, page_bytes=512, n_adapters=12, max_pages=16, max_rank=32, k=48,
                     d=80, elem_bytes=2)
    for _ in range(600):
        op = rng.integers(0, 5)
        a = int(rng.integers(0, 12))
        if op <= 1:
            before = list(m.last_use)
            was = [m.resident(b) for b in range(12)]
            log0 = len(m.evicted_log)
            if m.load(a, int(rng.integers(1, 33))) == pp.OK:
                for v in m.evicted_log[log0:]:
                    for s in range(12):
                        if s != a and was[s] and m.resident(s) and m.pins[s] == 0:
                            assert before[v] < before[s]
        elif op == 2:
            m.evict(a)
        elif op == 3 and m.resident(a):
            m.pin([a])
        elif op == 4 and m.pins[a] > 0:
            m.unpin([a])
        used = [p for b in range(12) for p in m.pages[b]]
        assert len(used) == len(set(used))
        assert len(used) + m.n_free() == 40
        for b in range(12):
            if m.resident(b):
                assert len(m.pages[b]) == m.pages_needed(m.rank[b])
            if m.pins[b] > 0:
                assert m.resident(b)


# ---------------------------------------------------------------------------
# The library's manager against the model (accounting-only mode).
# ---------------------------------------------------------------------------

def status_of(fn, *args):
    try:
        fn(*args)
        return 0
    except lr.LoraError as e:
        return e.status


def same_state(lib_pool, model, n_adapters):
    for a in range(n_adapters):
        assert lib_pool.query(a) == model.query(a), a
    assert lib_pool.stats() == model.stats()


GEOMS = [
    # n_pages, page_bytes, n_adapters, max_pages, max_rank, k, d, elem_bytes
    (64, 4096, 16, 64, 64, 512, 256, 2),
    (37, 256, 9, 40, 16, 40, 24, 4),
    (200, 65536, 24, 32, 64, 8192, 1024, 2),
]


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "pages%d_pb%d" % (g[0], g[1]))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_manager_matches_model(geom, seed):
    n_pages, pb, S, mp, R, k, d, eb = geom
    dtype = {2: "bf16", 4: "f32"}[eb]
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    lib_pool = lr.AdapterPool(n_pages, pb, S, mp, R, k, d, dtype=tdt, device=None)
    model = pp.PoolModel(n_pages, pb, S, mp, R, k, d, eb)
    rng = np.random.default_rng(100 + seed)
    for step in range(800):
        op = int(rng.integers(0, 9))
        a = int(rng.integers(-1, S + 1))  # includes out-of-range ids
        if op <= 2:
            r = int(rng.integers(-1, R + 2))  # includes rank 0 and bad ranks
            st_lib = status_of(lib_pool.load, a, None, None, r)
            st_mod = model.load(a, r)
        elif op == 3:
            st_lib, st_mod = status_of(lib_pool.evict, a), model.evict(a)
        elif op == 4:
            ids = [int(v) for v in rng.integers(0, S, size=int(rng.integers(0, 4)))]
            st_lib, st_mod = status_of(lib_pool.touch, ids), model.touch(ids)
        elif op == 5:
            ids = [int(v) for v in rng.integers(0, S, size=int(rng.integers(1, 3)))]
            st_lib, st_mod = status_of(lib_pool.pin, ids), model.pin(ids)
        elif op == 6:
            ids = [int(v) for v in rng.integers(0, S, size=int(rng.integers(1, 3)))]
            st_lib, st_mod = status_of(lib_pool.unpin, ids), model.unpin(ids)
        else:
            # batches, sometimes with a repeated id or a bad rank
            n = int(rng.integers(1, 5))
            reqs = [(int(rng.integers(0, S)), int(rng.integers(0, R + 1))) for _ in range(n)]
            if rng.random() < 0.1:
                reqs[-1] = (reqs[-1][0], R + 1)
            st_lib = status_of(lib_pool.load_batch, [(a_, None, None, r_) for a_, r_ in reqs])
            st_mod = model.load_batch(reqs)
        assert st_lib == st_mod, (step, op, a, st_lib, st_mod)
        if step % 16 == 0:
            same_state(lib_pool, model, S)
    same_state(lib_pool, model, S)
    assert model.stats()["evictions"] > 0  # the sequence exercised eviction


def test_manager_errors_and_edges():
    import torch
    P = lr.AdapterPool
    # geometry errors at creation
    for kw, status in ((dict(page_bytes=1000), 6), (dict(page_bytes=128), 6), (dict(n_pages=0), 6),
                       (dict(max_rank=0), 4), (dict(max_rank=257), 4), (dict(n_adapters=0), 1),
                       (dict(max_pages=0), 6)):
        args = dict(n_pages=8, page_bytes=4096, n_adapters=4, max_pages=8, max_rank=16, k=64, d=64)
        args.update(kw)
        with pytest.raises(lr.LoraError) as e:
            P(dtype=torch.bfloat16, device=None, **args)
        assert e.value.status == status, kw
    p = P(8, 1024, 4, 2, 16, 64, 64, dtype=torch.bfloat16, device=None)
    # rank 16 needs 16 * 128 * 2 = 4 KiB = 4 pages > max_pages 2
    with pytest.raises(lr.LoraError) as e:
        p.load(0, None, None, rank=16)
    assert e.value.status == 6
    p.load(0, None, None, rank=8)  # 2 pages
    p.pin([0])
    with pytest.raises(lr.LoraError) as e:
        p.evict(0)  # pinned
    assert e.value.status == 1
    with pytest.raises(lr.LoraError) as e:
        p.load(0, None, None, rank=2)  # pinned and would move (1 page)
    assert e.value.status == 1
    p.load(0, None, None, rank=7)  # pinned, same page count: reloaded in place
    assert p.query(0)["rank"] == 7 and p.query(0)["pages"] == [0, 1]
    with pytest.raises(lr.LoraError):
        p.unpin([0, 0])  # below zero: nothing changes
    assert p.query(0)["pins"] == 1
    p.unpin([0])
    with pytest.raises(lr.LoraError):
        p.pin([1])  # not resident
    p.evict(1)  # not resident: ok
    with pytest.raises(lr.LoraError):
        p.touch([4])
    # fill the pool: 8 pages = four adapters of 2 pages; all pinned -> no room
    for a in range(1, 4):
        p.load(a, None, None, rank=8)
    p.pin([0, 1, 2, 3])
    q = P(8, 1024, 5, 2, 16, 64, 64, dtype=torch.bfloat16, device=None)
    for a in range(4):
        q.load(a, None, None, rank=8)
    q.pin([0, 1, 2, 3])
    with pytest.raises(lr.LoraError) as e:
        q.load(4, None, None, rank=8)
    assert e.value.status == 6
    assert q.stats()["evictions"] == 0 and q.stats()["resident"] == 4
