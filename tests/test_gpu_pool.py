"""Adapter activation into a paged device pool, on the GPU, through the C ABI.

* After every load / evict the device page table and ranks equal the
  pool-policy model's (oracle/pool_policy.py) bit for bit, and every resident
  adapter's bytes, read back through the oracle's page translation, equal the
  host weights bit for bit.
* lora_linear over a managed pool gives the same bits as over stacked slots
  holding the same weights (same arithmetic, other addresses), and matches
  the fp64 oracle to the bf16 tolerance.
* An evicted adapter's rows are counted as bad ranks and get the base output.
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import DevWorkload, normwise, oracle_rows, say
from oracle import pool_policy as pp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


def logical_bytes(A: torch.Tensor, B: torch.Tensor) -> np.ndarray:
    """An adapter's logical byte space: A rows, then B rows (storage bytes)."""
    def raw(t):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint8).reshape(-1)
        return t.numpy().view(np.uint8).reshape(-1)
    return np.concatenate([raw(A), raw(B)])


def check_device_state(oracle_mod, pool: lr.AdapterPool, model: pp.PoolModel, blobs: dict):
    torch.cuda.synchronize()
    table = pool.page_table.cpu().numpy()
    assert np.array_equal(table, np.asarray(model.page_table(), np.int32))
    assert np.array_equal(pool.ranks.cpu().numpy(), np.asarray(model.rank, np.int32))
    buf = pool.pool.cpu().numpy()
    n_pages = buf.size // pool.page_bytes
    for a, blob in blobs.items():
        if not model.resident(a) or blob.size == 0:
            continue
        offs = np.arange(blob.size, dtype=np.int64)
        phys = oracle_mod.translate(table, pool.page_bytes, n_pages,
                                    np.full(blob.size, a, np.int32), offs)
        assert (phys >= 0).all(), a
        assert np.array_equal(buf[phys], blob), "adapter %d bytes differ" % a


def random_adapter(rng, r, k, d, dtype):
    A = torch.from_numpy(rng.standard_normal((r, k), dtype=np.float32) / np.sqrt(k)).to(dtype)
    B = torch.from_numpy(rng.standard_normal((d, r), dtype=np.float32) * 0.14).to(dtype)
    return A.contiguous(), B.contiguous()


@pytest.mark.parametrize("dtype,page_bytes", [(torch.bfloat16, 4096), (torch.float32, 65536)],
                         ids=["bf16_4k", "f32_64k"])
def test_pool_loads_match_model(oracle_mod, dtype, page_bytes):
    """Loads (pinned and pageable host memory), pins, touches, LRU and
    explicit evictions, a re-placement with a new rank: device state equals
    the model's after every step."""
    say("pool loads vs model %s %d" % (dtype, page_bytes))
    k, d, S, R = 1024, 768, 10, 64
    eb = torch.empty((), dtype=dtype).element_size()
    ranks = [4, 16, 64, 16, 8, 32, 64, 4, 0, 12]
    pages = [-(-r * (k + d) * eb // page_bytes) for r in ranks]
    n_pages = max(sum(pages) * 2 // 3, max(pages))  # too small for all: evictions happen
    pool = lr.AdapterPool(n_pages, page_bytes, S, 64, R, k, d, dtype=dtype, device="cuda")
    model = pp.PoolModel(n_pages, page_bytes, S, 64, R, k, d, eb)
    check_device_state(oracle_mod, pool, model, {})
    rng = np.random.default_rng(5)
    blobs = {}

    def load(a, r, pinned):
        if r == 0:  # does not touch this projection: no pages, nothing copied
            pool.load(a, None, None, rank=0)
            assert model.load(a, 0) == pp.OK
            blobs[a] = np.zeros(0, np.uint8)
            return
        A, B = random_adapter(rng, r, k, d, dtype)
        if pinned:
            A, B = A.pin_memory(), B.pin_memory()
        pool.load(a, A, B)
        assert model.load(a, r) == pp.OK
        blobs[a] = logical_bytes(A, B)
        if not pinned:
            A.zero_()  # the call has waited for a pageable source: reuse is safe
            B.zero_()

    for a, r in enumerate(ranks):
        load(a, r, pinned=(a % 2 == 0))
        check_device_state(oracle_mod, pool, model, blobs)
    assert model.stats()["evictions"] > 0
    pool.pin([7, 9])
    model.pin([7, 9])
    pool.touch([1, 3])
    model.touch([1, 3])
    for a, r in ((1, 16), (2, 64), (5, 8), (0, 32)):  # 5: rank change -> re-placed
        load(a, r, pinned=True)
        check_device_state(oracle_mod, pool, model, blobs)
    pool.evict(2)
    model.evict(2)
    pool.unpin([7])
    model.unpin([7])
    load(6, 64, pinned=False)
    check_device_state(oracle_mod, pool, model, blobs)
    assert pool.stats() == model.stats()
    for a in range(S):
        assert pool.query(a) == model.query(a)


@pytest.mark.parametrize("dtype,page_bytes", [(torch.bfloat16, 256), (torch.float32, 1 << 21)],
                         ids=["bf16_256", "f32_2m"])
def test_pool_batches_and_copy_paths(oracle_mod, dtype, page_bytes):
    """Batched loads through the copy kernel: sizes that are not multiples of
    16 bytes (d = 771), a source 2 bytes off 16-byte alignment (the
    element-wise path), pageable sources in the same batch (DMA fallback),
    evictions inside a batch; device state equals the model's each time."""
    say("pool batches %s %d" % (dtype, page_bytes))
    k, d, S, R = 520, 771, 8, 16
    eb = torch.empty((), dtype=dtype).element_size()
    ranks = [3, 16, 5, 1, 12, 7, 16, 2]
    pages = [-(-r * (k + d) * eb // page_bytes) for r in ranks]
    n_pages = max(sum(pages) * 3 // 4, max(pages) * 3)
    max_pages = max(pages)
    pool = lr.AdapterPool(n_pages, page_bytes, S, max_pages, R, k, d, dtype=dtype, device="cuda")
    model = pp.PoolModel(n_pages, page_bytes, S, max_pages, R, k, d, eb)
    rng = np.random.default_rng(11)
    blobs = {}

    def weights(a, r, kind):
        A, B = random_adapter(rng, r, k, d, dtype)
        if kind == "pinned":
            A, B = A.pin_memory(), B.pin_memory()
        elif kind == "offset":  # pinned, 2 bytes past a 16-byte boundary
            ba = torch.empty(A.numel() + 8, dtype=dtype).pin_memory()
            bb = torch.empty(B.numel() + 8, dtype=dtype).pin_memory()
            off = 1 if eb == 2 else 0
            ba[off:off + A.numel()].copy_(A.reshape(-1))
            bb[off:off + B.numel()].copy_(B.reshape(-1))
            A = ba[off:off + A.numel()].view(r, k)
            B = bb[off:off + B.numel()].view(d, r)
        blobs[a] = logical_bytes(A.contiguous(), B.contiguous())
        return (a, A, B)

    kinds = ["pinned", "offset", "pageable"]
    for rnd in range(4):
        ids = [int(x) for x in rng.permutation(S)[:3]]
        items = [weights(a, int(rng.choice(ranks)), kinds[(i + rnd) % 3]) for i, a in enumerate(ids)]
        pool.load_batch(items)
        assert model.load_batch([(a, A.shape[0]) for a, A, _ in items]) == pp.OK
        check_device_state(oracle_mod, pool, model, blobs)
    assert model.stats()["evictions"] > 0
    assert pool.stats() == model.stats()


def _managed_pool(w, proj, page_bytes, order, device="cuda", batch=False):
    """All adapters of a workload loaded through the manager, in `order`
    (one call per adapter, or one batch), then one evicted and reloaded."""
    eb = w.elem_bytes
    need = sum(-(-int(r) * (w.k + proj.d) * eb // page_bytes) for r in w.ranks)
    max_pages = max(-(-int(r) * (w.k + proj.d) * eb // page_bytes) for r in w.ranks)
    pool = lr.AdapterPool(need + 3, page_bytes, w.S, max_pages, w.max_rank, w.k, proj.d,
                          dtype=w.dtype, device=device)
    if batch:
        pool.load_batch([(int(s), proj.A[s].pin_memory(), proj.B[s].pin_memory()) for s in order])
    else:
        for s in order:
            pool.load(int(s), proj.A[s].pin_memory(), proj.B[s].pin_memory())
    first = int(order[0])
    pool.evict(first)
    pool.load(first, proj.A[first].pin_memory(), proj.B[first].pin_memory())
    return pool


def test_managed_pool_linear_matches_slots(oracle_mod):
    say("managed pool lora_linear vs slots")
    w = wl.custom(seed=71, M=300, k=1024, d=768, ranks=[4, 16, 64, 16, 8, 32], max_rank=64,
                  none_frac=0.1)
    p = w.projections[0]
    pool = _managed_pool(w, p, 4096, order=[3, 1, 5, 0, 4, 2])
    slots = DevWorkload(w, p)
    ad = pool.adapters()
    ws = lr.new_workspace(w.M, p.d, w.k, w.dtype, ad)
    ref = oracle_rows(oracle_mod, w, p)
    for path in (lr.PATH_AUTO, lr.PATH_GATHER, lr.PATH_SGMV):
        y = lr.lora_linear(slots.x, slots.W, ad, slots.ids, slots.scales, workspace=ws, path=path)
        torch.cuda.synchronize()
        chk = lr.lora_check(ws)
        assert chk == {"n_bad_ids": 0, "n_bad_ranks": 0, "n_bad_pages": 0, "n_sync_expired": 0}
        y_slot = slots.run(path=path)
        assert torch.equal(y, y_slot), path
        assert normwise(y.double().cpu().numpy(), ref) <= 2e-2


def test_evicted_adapter_rows_get_the_base(oracle_mod):
    say("evicted adapter rows")
    w = wl.custom(seed=72, M=256, k=512, d=384, ranks=[8, 16, 32, 4], max_rank=32, none_frac=0.1)
    p = w.projections[0]
    pool = _managed_pool(w, p, 4096, order=[0, 1, 2, 3])
    slots = DevWorkload(w, p)
    pool.evict(2)
    ad = pool.adapters()
    ws = lr.new_workspace(w.M, p.d, w.k, w.dtype, ad)
    y = lr.lora_linear(slots.x, slots.W, ad, slots.ids, slots.scales, workspace=ws)
    chk = lr.lora_check(ws)
    n2 = int((w.ids == 2).sum())
    assert chk == {"n_bad_ids": 0, "n_bad_ranks": n2, "n_bad_pages": 0, "n_sync_expired": 0}
    base = lr.lora_gemm(slots.x, slots.W)
    y_slot = slots.run()
    torch.cuda.synchronize()
    rows2 = torch.from_numpy(np.flatnonzero(w.ids == 2)).cuda()
    other = torch.from_numpy(np.flatnonzero(w.ids != 2)).cuda()
    assert torch.equal(y[rows2], base[rows2])
    assert torch.equal(y[other], y_slot[other])
    # reload (other pages now) and the rows are adapted again
    pool.load(2, p.A[2], p.B[2])
    y = lr.lora_linear(slots.x, slots.W, ad, slots.ids, slots.scales, workspace=ws)
    assert lr.lora_check(ws)["n_bad_ranks"] == 0
    assert torch.equal(y, y_slot)


def test_managed_pools_c3_sliced_match_slots(c3_workload):
    """The 70B-shaped q (8192 -> 8192) and v (8192 -> 1024) projections with
    their adapters activated through two managed pools of 64 KiB pages."""
    w = c3_workload
    say("c3 managed pools q+v")
    pq, pv = w.proj("q"), w.proj("v")
    order = np.argsort(-w.ranks, kind="stable")  # biggest first
    qpool = _managed_pool(w, pq, 65536, order)
    vpool = _managed_pool(w, pv, 65536, order, batch=True)
    dq, dv = DevWorkload(w, pq), DevWorkload(w, pv)
    W = torch.cat([dq.W, dv.W], 0).contiguous()
    managed = [lr.Slice(pq.d, qpool.adapters(), dq.scales), lr.Slice(pv.d, vpool.adapters(), dv.scales)]
    stacked = [lr.Slice(pq.d, dq.ad, dq.scales), lr.Slice(pv.d, dv.ad, dv.scales)]
    # 64 KiB pages hold whole 16 KiB A rows, so both calls fold the shrink
    # into the base GEMM: same arithmetic, other addresses
    y_m = lr.lora_linear_sliced(dq.x, W, managed, dq.ids)
    y_f = lr.lora_linear_sliced(dq.x, W, stacked, dq.ids)
    # and both with the shrink as its own kernel
    y_ms = lr.lora_linear_sliced(dq.x, W, managed, dq.ids, flags=lr.FLAG_SEPARATE_SHRINK)
    y_s = lr.lora_linear_sliced(dq.x, W, stacked, dq.ids, flags=lr.FLAG_SEPARATE_SHRINK)
    torch.cuda.synchronize()
    assert torch.equal(y_m, y_f)
    assert torch.equal(y_ms, y_s)
    assert normwise(y_s.double().cpu().numpy(), y_m.double().cpu().numpy()) <= 1e-2


@pytest.fixture(scope="module")
def c3_workload():
    return wl.c3_proj70b_bf16()
