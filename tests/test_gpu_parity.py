"""HIP path against the fp64 oracle, element by element, through the C ABI.

Tolerances (normwise max|y - ref| / max|ref| per output tensor): 1e-5 for the
fp32 workloads, 2e-2 for bf16 (fp32 accumulation; adapted bf16 rows are
rounded twice, after the base GEMM and after the expand).  Integer work (the
plan, page translation) is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import DevWorkload, TOL, assert_covers_present_adapters, normwise, oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# base GEMM
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,k,d", [(1, 64, 16), (37, 96, 40), (128, 256, 128), (300, 264, 129),
                                   (513, 1032, 260)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gemm_matches_fp64(M, k, d, dtype):
    say("gemm M=%d k=%d d=%d %s" % (M, k, d, dtype))
    g = torch.Generator().manual_seed(M * 7 + k)
    x = torch.randn(M, k, generator=g).to(dtype)
    W = (torch.randn(d, k, generator=g) / k ** 0.5).to(dtype)
    y = lr.lora_gemm(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    ref = x.double().numpy() @ W.double().numpy().T
    err = normwise(y.double().cpu().numpy(), ref)
    assert err <= TOL[dtype], err


def test_gemm_leading_dims():
    say("gemm strided views")
    g = torch.Generator().manual_seed(3)
    xb = torch.randn(70, 144, generator=g).to(torch.bfloat16)
    Wb = (torch.randn(50, 136, generator=g) / 12).to(torch.bfloat16)
    x = xb.cuda()[:, :128]
    W = Wb.cuda()[:, :128]
    ybuf = torch.full((70, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    y = ybuf[:, :50]
    lr.lora_gemm(x, W, y=y)
    torch.cuda.synchronize()
    ref = xb[:, :128].double().numpy() @ Wb[:, :128].double().numpy().T
    assert normwise(y.double().cpu().numpy(), ref) <= 2e-2
    assert bool((ybuf[:, 50:] == 7.0).all())  # columns past d untouched


# ---------------------------------------------------------------------------
# plan: bit-exact against the oracle
# ---------------------------------------------------------------------------

def _plan_case(oracle_mod, ids, S, ranks, R, pooled=None):
    dev = torch.device("cuda:0")
    ranks_t = torch.from_numpy(np.asarray(ranks, np.int32)).to(dev)
    k = d = 64
    if pooled is None:
        A = torch.zeros(S, R, k, dtype=torch.bfloat16, device=dev)
        B = torch.zeros(S, d, R, dtype=torch.bfloat16, device=dev)
        ad = lr.Adapters.slots(A, B, ranks_t)
        ref = oracle_mod.plan(ids, S, ranks, R)
    else:
        table, n_pages, P = pooled
        pool = torch.zeros(n_pages * P, dtype=torch.uint8, device=dev)
        ad = lr.Adapters.paged(pool, torch.from_numpy(table).to(dev), ranks_t, P, R)
        ref = oracle_mod.plan(ids, S, ranks, R, page_table=table, n_pages=n_pages, page_bytes=P,
                              k=k, d=d, elem_bytes=2)
    M = len(ids)
    ws = lr.new_workspace(M, d, k, torch.bfloat16, ad, device=dev)
    lr.lora_plan(torch.from_numpy(np.asarray(ids, np.int32)).to(dev), ad, k, d, torch.bfloat16, ws)
    got = lr.lora_plan_view(ws, M, ad)
    assert got["n_adapted"] == ref["n_adapted"]
    assert np.array_equal(got["perm"], ref["perm"])
    assert np.array_equal(got["seg_adapter"], ref["seg_adapter"])
    assert np.array_equal(got["seg_start"], ref["seg_start"])
    assert np.array_equal(got["seg_len"], ref["seg_len"])
    for key in ("n_bad_ids", "n_bad_ranks", "n_bad_pages"):
        assert got[key] == ref[key], key
    chk = lr.lora_check(ws)
    assert chk == {**{k_: ref[k_] for k_ in ("n_bad_ids", "n_bad_ranks", "n_bad_pages")},
                   "n_sync_expired": 0}
    # work items cover every adapted row exactly once
    assert got["items_gather"] == sum((l + 15) // 16 for l in ref["seg_len"])
    assert got["items_sgmv"] == sum((l + 63) // 64 for l in ref["seg_len"])


@pytest.mark.parametrize("M,S,seed", [(0, 3, 0), (1, 3, 1), (64, 4, 2), (255, 7, 3), (512, 12, 4),
                                      (2048, 1024, 5), (4097, 300, 6), (8192, 8, 7),
                                      (300, 5000, 9), (3000, 6000, 10)])
def test_plan_random_ids(oracle_mod, M, S, seed):
    say("plan M=%d S=%d" % (M, S))
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, S, size=M).astype(np.int32)
    if M > 4:
        ids[rng.integers(0, M, size=3)] = [-7, S, S + 100]   # invalid ids
    ranks = rng.integers(0, 17, size=S).astype(np.int32)
    ranks[0] = 20                                              # over max_rank
    _plan_case(oracle_mod, ids, S, ranks, 16)


def test_plan_structured(oracle_mod):
    for name, ids, S in [
        ("all none", np.full(100, -1, np.int32), 4),
        ("one adapter", np.zeros(777, np.int32), 2),
        ("sorted runs", np.repeat(np.arange(8, dtype=np.int32), 1024), 8),
        ("every row distinct", np.arange(1000, dtype=np.int32)[::-1].copy(), 1000),
        ("c3 ids", wl.c3_proj70b_bf16(M=512, k=64, d_q=64, d_v=64).ids, 12),
    ]:
        say("plan " + name)
        _plan_case(oracle_mod, ids, S, np.full(S, 8, np.int32), 16)


@pytest.mark.parametrize("M,S,k,d,dtype", [(512, 12, 256, 288, torch.bfloat16),
                                           (300, 8000, 64, 64, torch.bfloat16),
                                           (200, 9, 64, 64, torch.float32),
                                           (777, 40, 128, 96, torch.bfloat16)])
def test_plan_inside_linear(oracle_mod, M, S, k, d, dtype):
    # lora_linear computes the plan inside the base GEMM's launch (or just
    # before it): the plan it leaves in the workspace is the oracle's
    say("plan inside lora_linear M=%d S=%d k=%d d=%d %s" % (M, S, k, d, dtype))
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(M + S)
    ids = rng.integers(-1, S, size=M).astype(np.int32)
    ranks = rng.integers(0, 9, size=S).astype(np.int32)
    R = 8
    A = torch.zeros(S, R, k, dtype=dtype, device=dev)
    B = torch.zeros(S, d, R, dtype=dtype, device=dev)
    ranks_t = torch.from_numpy(ranks).to(dev)
    ad = lr.Adapters.slots(A, B, ranks_t)
    x = torch.randn(M, k, device=dev).to(dtype)
    W = torch.randn(d, k, device=dev).to(dtype)
    scales = torch.ones(S, dtype=torch.float32, device=dev)
    ws = lr.new_workspace(M, d, k, dtype, ad, device=dev)
    lr.lora_linear(x, W, ad, torch.from_numpy(ids).to(dev), scales, workspace=ws)
    got = lr.lora_plan_view(ws, M, ad)
    ref = oracle_mod.plan(ids, S, ranks, R)
    assert got["n_adapted"] == ref["n_adapted"]
    assert np.array_equal(got["perm"], ref["perm"])
    assert np.array_equal(got["seg_adapter"], ref["seg_adapter"])
    assert np.array_equal(got["seg_start"], ref["seg_start"])
    assert np.array_equal(got["seg_len"], ref["seg_len"])
    assert got["items_gather"] == sum((l + 15) // 16 for l in ref["seg_len"])


def test_plan_pool_pages(oracle_mod):
    say("plan pool page checks")
    rng = np.random.default_rng(8)
    S, P, n_pages = 20, 4096, 64
    k = d = 64
    ranks = rng.integers(1, 17, size=S).astype(np.int32)
    need = (ranks * (k + d) * 2 + P - 1) // P
    table = np.full((S, 4), -1, np.int32)
    for s in range(S):
        table[s, :need[s]] = rng.integers(0, n_pages, size=need[s])
    table[3, 0] = n_pages        # out of the pool
    table[5, need[5] - 1] = -2   # negative
    ids = rng.integers(-1, S, size=300).astype(np.int32)
    _plan_case(oracle_mod, ids, S, ranks, 16, pooled=(table, n_pages, P))


def test_translate_bit_exact(oracle_mod):
    say("translate")
    rng = np.random.default_rng(12)
    S, P, n_pages, max_pages = 30, 4096, 100, 6
    table = rng.integers(-1, n_pages + 2, size=(S, max_pages)).astype(np.int32)
    a = rng.integers(-2, S + 2, size=5000).astype(np.int32)
    off = rng.integers(-5, (max_pages + 1) * P, size=5000).astype(np.int64)
    dev = torch.device("cuda:0")
    pool = torch.zeros(n_pages * P, dtype=torch.uint8, device=dev)
    ad = lr.Adapters.paged(pool, torch.from_numpy(table).to(dev),
                           torch.ones(S, dtype=torch.int32, device=dev), P, 4)
    got = lr.lora_translate(ad, torch.from_numpy(a).to(dev), torch.from_numpy(off).to(dev))
    ok = (a >= 0) & (a < S)
    want = np.full(a.shape, -1, np.int64)
    want[ok] = oracle_mod.translate(table, P, n_pages, a[ok], off[ok])
    assert np.array_equal(got.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# the layer: full workloads (small ones whole, large ones on sampled rows)
# ---------------------------------------------------------------------------

def _check_full(oracle_mod, dw: DevWorkload, label: str, rows=None, path=lr.PATH_AUTO,
                cache=False):
    """Every row (rows=None) or the given rows against the oracle; cache=True
    memoises the oracle's full output for the large seeded workloads."""
    w, p = dw.w, dw.p
    say("layer %s (%s, M=%d k=%d d=%d, %s rows)" % (label, w.name, w.M, w.k, p.d,
                                                   "all" if rows is None else len(rows)))
    assert_covers_present_adapters(w, rows)
    y = dw.run(path=path).double().cpu().numpy()
    base = lr.lora_gemm(dw.x, dw.W)
    torch.cuda.synchronize()
    base = base.double().cpu().numpy()
    ref = oracle_rows(oracle_mod, w, p, rows, cache=cache)
    got = y if rows is None else y[rows]
    err = normwise(got, ref)
    say("  normwise error %.3g" % err)
    assert err <= TOL[w.dtype], err
    # rows with no adapter: exactly the base GEMM (bitwise)
    none = np.flatnonzero(w.ids < 0)
    assert np.array_equal(y[none], base[none])
    # the LoRA delta alone, on adapted rows (diagnostic bound)
    ids = w.ids if rows is None else w.ids[rows]
    adapted = ids >= 0
    if adapted.any():
        ref_base = oracle_rows(oracle_mod, w, p, rows, ids=np.full(w.M, -1, np.int32), cache=cache)
        d_got = (got - (base if rows is None else base[rows]))[adapted]
        d_ref = (ref - ref_base)[adapted]
        derr = normwise(d_got, d_ref)
        say("  delta normwise error %.3g" % derr)
        assert derr <= (5e-2 if w.dtype == torch.bfloat16 else 1e-4), derr
    return y


def test_c0_tiny_fp32(oracle_mod):
    w = wl.c0_tiny_fp32()
    _check_full(oracle_mod, DevWorkload(w, w.projections[0]), "c0")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_u1_distinct_scales(oracle_mod, dtype):
    w = wl.u1_scales(dtype=dtype)
    _check_full(oracle_mod, DevWorkload(w, w.projections[0]), "u1")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_u2_pool_small_pages(oracle_mod, dtype):
    w = wl.u2_pages(dtype=dtype)
    p = w.projections[0]
    y_pool = _check_full(oracle_mod, DevWorkload(w, p, pooled=True), "u2 pool 4KiB")
    y_slot = DevWorkload(w, p).run().double().cpu().numpy()
    assert np.array_equal(y_pool, y_slot)  # same arithmetic, other addresses


def test_c1_decode(oracle_mod):
    w = wl.c1_decode_bf16()
    _check_full(oracle_mod, DevWorkload(w, w.projections[0]), "c1")


@pytest.fixture(scope="module")
def c2():
    return wl.c2_prefill_bf16()


def test_c2_prefill(oracle_mod, c2):
    _check_full(oracle_mod, DevWorkload(c2, c2.projections[0]), "c2", cache=True)


@pytest.fixture(scope="module")
def c3():
    return wl.c3_proj70b_bf16()


@pytest.mark.parametrize("proj", ["q", "v"])
def test_c3_proj70b(oracle_mod, c3, proj):
    _check_full(oracle_mod, DevWorkload(c3, c3.proj(proj)), "c3 " + proj, cache=True)


@pytest.fixture(scope="module")
def c4():
    return wl.c4_paged_bf16()


def test_c4_paged(oracle_mod, c4):
    p = c4.projections[0]
    y_pool = _check_full(oracle_mod, DevWorkload(c4, p, pooled=True), "c4 pool 2MiB", cache=True)
    y_slot = DevWorkload(c4, p).run().double().cpu().numpy()
    assert np.array_equal(y_pool, y_slot)


@pytest.mark.parametrize("pname,path", [("gather", lr.PATH_GATHER), ("sgmv", lr.PATH_SGMV)],
                         ids=["gather", "sgmv"])
def test_u2_pages_at_c4_shape(oracle_mod, c4, pname, path):
    """Page crossing at the paged-pool shape ("S-LoRA: ...", "Unified
    paging"): d = k = 5120, rank 16, 4 KiB pages, so each adapter's 320 KiB
    [A | B] spans 80 pages at seeded physical positions (spare pool pages
    hold NaN).  Every row against the oracle, and bitwise equal to the same
    path over 2 MiB pages (one page per adapter): only addresses differ."""
    p = c4.projections[0]
    small = DevWorkload(c4, p, pooled=True, page_bytes=4096)
    assert int(small.table.shape[1]) == 80
    y4k = _check_full(oracle_mod, small, "u2 at c4 shape, 4 KiB pages " + pname, path=path,
                      cache=True)
    del small
    big = DevWorkload(c4, p, pooled=True)
    y2m = big.run(path=path).double().cpu().numpy()
    assert np.array_equal(y4k, y2m)


# ---------------------------------------------------------------------------
# invariants that need no oracle, and edge cases
# ---------------------------------------------------------------------------

def test_bitwise_invariants():
    w = wl.custom(seed=21, M=300, k=520, d=200, ranks=[4, 16, 7, 32, 1], max_rank=32)
    dw = DevWorkload(w, w.projections[0])
    say("invariants")
    y1 = dw.run().clone()
    y2 = dw.run().clone()
    assert torch.equal(y1, y2)                         # run to run
    y2x = dw.run(x=dw.x * 2).clone()
    assert torch.equal(y2x, y1 * 2)                    # power-of-two scaling is exact
    y3 = dw.run(flags=lr.FLAG_REUSE_PLAN).clone()      # plan reused from the last call
    assert torch.equal(y3, y1)
    # rank padding never reaches the output (kernels may load it inside a
    # 16-byte vector, but zero it before use), on every path
    nan_pad = DevWorkload(w, w.projections[0], pad_value=float("nan"))
    assert torch.equal(nan_pad.run(), y1)
    for path in (lr.PATH_GATHER, lr.PATH_SGMV):
        assert torch.equal(nan_pad.run(path=path), dw.run(path=path))


def test_sorted_and_unsorted_rows_agree():
    """Sorting rows by adapter changes no value ("Adapter Residency ...",
    section "Batch composition under many adapters")."""
    w = wl.custom(seed=5, M=200, k=256, d=96, ranks=[8, 8, 16, 4], max_rank=16)
    dw = DevWorkload(w, w.projections[0])
    say("row order")
    y = dw.run().clone()
    order = np.argsort(w.ids, kind="stable")
    o = torch.from_numpy(order).cuda()
    yp = dw.run(x=dw.x[o].contiguous(), ids=dw.ids[o].contiguous())
    assert torch.equal(yp, y[o])


@pytest.mark.parametrize("M,k,d,ranks", [
    (1, 64, 16, [4]),
    (17, 264, 41, [1, 2, 3, 5]),
    (130, 8, 8, [8, 8]),
    (64, 1024, 520, [64, 32, 16]),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_edge_shapes(oracle_mod, M, k, d, ranks, dtype):
    w = wl.custom(seed=M + k + d, M=M, k=k, d=d, ranks=ranks, max_rank=max(ranks), dtype=dtype)
    _check_full(oracle_mod, DevWorkload(w, w.projections[0]), "edge")


def test_empty_batch_and_all_none():
    w = wl.custom(seed=2, M=40, k=64, d=32, ranks=[4, 4], max_rank=4)
    dw = DevWorkload(w, w.projections[0])
    say("empty / all none")
    y0 = torch.empty(0, 32, dtype=torch.bfloat16, device="cuda")
    lr.lora_linear(dw.x[:0], dw.W, dw.ad, dw.ids[:0], dw.scales, y=y0, workspace=dw.ws)
    ids = torch.full((40,), -1, dtype=torch.int32, device="cuda")
    y = dw.run(ids=ids)
    assert torch.equal(y, lr.lora_gemm(dw.x, dw.W))


def test_bad_ids_and_ranks_are_counted_and_ignored(oracle_mod):
    w = wl.custom(seed=9, M=64, k=128, d=64, ranks=[4, 8, 40], max_rank=16)  # rank 40 > max
    ids = w.ids.copy()
    ids[[1, 2, 3]] = [-2, 3, 1000]
    dw = DevWorkload(w, w.projections[0])
    say("bad ids / ranks")
    y = dw.run(ids=torch.from_numpy(ids).cuda()).double().cpu().numpy()
    chk = lr.lora_check(dw.ws)
    assert chk["n_bad_ids"] == 3
    assert chk["n_bad_ranks"] == int((ids == 2).sum())
    eff = ids.copy()
    eff[(eff < -1) | (eff >= 3) | (eff == 2)] = -1
    ref = oracle_rows(oracle_mod, w, w.projections[0], ids=eff)
    assert normwise(y, ref) <= 2e-2


def test_row_chunks_beyond_plan_limit(oracle_mod):
    w = wl.custom(seed=33, M=8192 + 300, k=64, d=48, ranks=[4, 8, 16], max_rank=16)
    dw = DevWorkload(w, w.projections[0])
    say("row chunks M=%d" % w.M)
    y = dw.run().double().cpu().numpy()
    ref = oracle_rows(oracle_mod, w, w.projections[0])   # every row, both chunks
    assert normwise(y, ref) <= 2e-2


# ---------------------------------------------------------------------------
# both kernel families (VALU gather, MFMA segments) on every bf16 workload
# ---------------------------------------------------------------------------

PATHS = [("gather", lr.PATH_GATHER), ("sgmv", lr.PATH_SGMV)]


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_c1(oracle_mod, pname, path):
    w = wl.c1_decode_bf16()
    _check_full(oracle_mod, DevWorkload(w, w.projections[0]), "c1 " + pname, path=path)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_c2(oracle_mod, c2, pname, path):
    _check_full(oracle_mod, DevWorkload(c2, c2.projections[0]), "c2 " + pname, path=path,
                cache=True)


@pytest.mark.parametrize("proj", ["q", "v"])
@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_c3(oracle_mod, c3, pname, path, proj):
    _check_full(oracle_mod, DevWorkload(c3, c3.proj(proj)), "c3 %s %s" % (proj, pname), path=path,
                cache=True)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_c4_pool(oracle_mod, c4, pname, path):
    _check_full(oracle_mod, DevWorkload(c4, c4.projections[0], pooled=True), "c4 pool " + pname,
                path=path, cache=True)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_c4_slots(oracle_mod, c4, pname, path):
    _check_full(oracle_mod, DevWorkload(c4, c4.projections[0]), "c4 slots " + pname, path=path,
                cache=True)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_paths_small(oracle_mod, pname, path):
    for w, pooled in ((wl.u1_scales(dtype=torch.bfloat16), False),
                      (wl.u2_pages(dtype=torch.bfloat16), True),
                      (wl.custom(seed=41, M=300, k=264, d=130, ranks=[1, 3, 8, 17, 33, 64],
                                 max_rank=64), False),
                      (wl.custom(seed=42, M=1500, k=512, d=96, ranks=[8, 40, 16], max_rank=40,
                                 sorted_ids=True), False),
                      # pooled: ranks that are and are not multiples of 8, 16- and
                      # 64-row items
                      (wl.custom(seed=43, M=300, k=264, d=136, ranks=[1, 3, 8, 17, 32, 64],
                                 max_rank=64), True),
                      (wl.custom(seed=44, M=1500, k=512, d=96, ranks=[8, 40, 16], max_rank=40,
                                 sorted_ids=True), True)):
        _check_full(oracle_mod, DevWorkload(w, w.projections[0], pooled=pooled),
                    "%s %s" % (w.name, pname), path=path)


def test_sgmv_unsupported_combinations():
    say("sgmv unsupported")
    w = wl.custom(seed=3, M=32, k=64, d=32, ranks=[4, 4], max_rank=4, dtype=torch.float32)
    dw = DevWorkload(w, w.projections[0])
    with pytest.raises(lr.LoraError) as e:
        dw.run(path=lr.PATH_SGMV)
    assert e.value.status == 8
    w = wl.custom(seed=4, M=32, k=64, d=32, ranks=[4, 100], max_rank=128)
    dw = DevWorkload(w, w.projections[0])
    with pytest.raises(lr.LoraError) as e:
        dw.run(path=lr.PATH_SGMV)
    assert e.value.status == 8
    dw.run(path=lr.PATH_AUTO)  # falls to the VALU kernels


# ---------------------------------------------------------------------------
# several projections in one call
# ---------------------------------------------------------------------------

def _stacked(ws_list):
    return torch.cat([w for w in ws_list], dim=0).contiguous()


@pytest.mark.parametrize("pname,path", [("auto", lr.PATH_AUTO)] + PATHS,
                         ids=["auto", "gather", "sgmv"])
def test_sliced_c3_q_and_v(oracle_mod, c3, pname, path):
    say("sliced c3 q+v " + pname)
    pq, pv = c3.proj("q"), c3.proj("v")
    dq, dv = DevWorkload(c3, pq), DevWorkload(c3, pv)
    W = _stacked([dq.W, dv.W])
    slices = [lr.Slice(pq.d, dq.ad, dq.scales), lr.Slice(pv.d, dv.ad, dv.scales)]
    y = lr.lora_linear_sliced(dq.x, W, slices, dq.ids, path=path)
    torch.cuda.synchronize()
    base = lr.lora_gemm(dq.x, W)
    torch.cuda.synchronize()
    yq = y[:, :pq.d].double().cpu().numpy()
    yv = y[:, pq.d:].double().cpu().numpy()
    for name, got, p in (("q", yq, pq), ("v", yv, pv)):
        ref = oracle_rows(oracle_mod, c3, p, cache=True)   # every row, every adapter
        err = normwise(got, ref)
        say("  %s normwise error %.3g" % (name, err))
        assert err <= 2e-2
    none = np.flatnonzero(c3.ids < 0)
    assert torch.equal(y[none], base[none])
    # same as the q projection alone, to the bf16 tolerance
    y1 = dq.run(path=path)
    assert normwise(yq, y1.double().cpu().numpy()) <= 1e-2


def test_sliced_mixed_storage_and_rank_zero(oracle_mod):
    """Slice 0 in slots, slice 1 in a paged pool where adapter 2 has rank 0
    (it does not touch that projection)."""
    say("sliced mixed storage")
    M, k = 200, 256
    w0 = wl.custom(seed=61, M=M, k=k, d=96, ranks=[8, 16, 4, 32], max_rank=32)
    w1 = wl.custom(seed=61, M=M, k=k, d=40, ranks=[4, 8, 0, 16], max_rank=16)
    w1.x, w1.ids = w0.x, w0.ids
    d0 = DevWorkload(w0, w0.projections[0])
    d1 = DevWorkload(w1, w1.projections[0], pooled=True, page_bytes=4096)
    W = _stacked([d0.W, d1.W])
    slices = [lr.Slice(96, d0.ad, d0.scales), lr.Slice(40, d1.ad, d1.scales)]
    for path in (lr.PATH_GATHER, lr.PATH_SGMV):
        y = lr.lora_linear_sliced(d0.x, W, slices, d0.ids, path=path)
        torch.cuda.synchronize()
        y = y.double().cpu().numpy()
        assert normwise(y[:, :96], oracle_rows(oracle_mod, w0, w0.projections[0])) <= 2e-2
        assert normwise(y[:, 96:], oracle_rows(oracle_mod, w1, w1.projections[0])) <= 2e-2


@pytest.mark.parametrize("M,rmax", [(300, [64, 64, 64]), (300, [64, 32]), (2048, [64, 64, 64]),
                                    (2048, [16, 32, 16, 8])],
                         ids=["decode-3x64", "decode-64+32", "prefill-3x64", "prefill-4"])
def test_sliced_rank_blocks_per_workgroup(oracle_mod, M, rmax):
    """The shrink takes every slice's rank blocks in one workgroup where they
    fit 128 A rows (64 + 32, 16 + 32 + 16 + 8) and one workgroup per slice
    where they do not (3 x 64); decode-sized batches run 16-row items,
    prefill-sized runs (four adapters over 2048 rows) 64-row items.  Ragged
    k, ranks that are not multiples of 16, rank 0 in one slice; every slice
    of every row against the oracle, with and without the separate-shrink
    flag (no fold at these widths either way)."""
    say("sliced rank blocks M=%d %s" % (M, rmax))
    k = 520
    ds = [72, 40, 56, 24][:len(rmax)]
    S = 4 if M == 2048 else 9
    rng = np.random.default_rng(M + len(rmax))
    ws, devs = [], []
    for q, (r, d) in enumerate(zip(rmax, ds)):
        ranks = [int(v) for v in rng.integers(1, r + 1, size=S)]
        ranks[0] = r
        if q == 1:
            ranks[1] = 0
        w = wl.custom(seed=70 + q, M=M, k=k, d=d, ranks=ranks, max_rank=r)
        if ws:
            w.x, w.ids = ws[0].x, ws[0].ids
        ws.append(w)
        devs.append(DevWorkload(w, w.projections[0]))
    W = _stacked([dv.W for dv in devs])
    slices = [lr.Slice(d, dv.ad, dv.scales) for d, dv in zip(ds, devs)]
    for flags in (0, lr.FLAG_SEPARATE_SHRINK):
        y = lr.lora_linear_sliced(devs[0].x, W, slices, devs[0].ids, flags=flags)
        torch.cuda.synchronize()
        y = y.double().cpu().numpy()
        lo = 0
        for w, d in zip(ws, ds):
            err = normwise(y[:, lo:lo + d], oracle_rows(oracle_mod, w, w.projections[0]))
            say("  flags %d slice d=%d normwise %.3g" % (flags, d, err))
            assert err <= 2e-2
            lo += d
