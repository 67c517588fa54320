"""The shrink folded into the base GEMM, on the GPU, through the C ABI.

Where the base GEMM runs 128 x 144 or 64 x 64 tiles (bf16, adapters in
slots or in pages that hold whole A rows), each column tile also computes 16
columns of t = x A^T over the stacked (slice, adapter, rank) list -- and 16
more in a second pass where the list is longer than the first pass's
capacity -- and no shrink is launched.  Checked against the fp64 oracle
(normwise 2e-2, the layer's bf16 bound), against the same call with
LORA_FLAG_SEPARATE_SHRINK (t summed in another order: the two outputs differ
by bf16 rounding of y only), and through the library's own launch counters
(which kernels ran).  Shapes: 400 rows (three full 128-row tiles and a
16-row tail) and sum d = 9216, the range where 128 x 144 tiles are chosen;
decode sizes (64 to 256 rows, ragged columns) for the 64 x 64 tiles; k <= 512
keeps the oracle fast (the decode-4096 workload on sampled rows).
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import DevWorkload, normwise, oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


def launches(fn):
    """Run fn under the library's launch counters; kernel class -> launches."""
    with lr.Profiler():
        fn()
        torch.cuda.synchronize()
        prof = lr.Profiler.read(reset=True)
    return {k: prof[k]["launches"] for k in lr.KERNEL_CLASSES}


def sliced_pair(w):
    """Device slices for a two-projection workload (q then v)."""
    dev = torch.device("cuda")
    ranks = torch.from_numpy(w.ranks).to(dev)
    scales = torch.from_numpy(w.scales).to(dev)
    slices, keep = [], []
    for p in (w.proj("q"), w.proj("v")):
        A, B = wl.slots(w, p)
        A, B = A.to(dev), B.to(dev)
        keep.append((A, B))
        slices.append(lr.Slice(p.d, lr.Adapters.slots(A, B, ranks), scales))
    W = torch.cat([w.proj("q").W, w.proj("v").W], dim=0).contiguous().to(dev)
    return W, slices, keep


def test_two_slices_fused_matches_oracle(oracle_mod):
    """q + v slices with the 70B adapter set (ranks 4/16/64, sum 600 of a
    1024-column first pass)."""
    w = wl.c3_proj70b_bf16(M=400, k=512, d_q=8064, d_v=1152)
    W, slices, _keep = sliced_pair(w)
    x, ids = w.x.cuda(), torch.from_numpy(w.ids).cuda()
    out = {}
    for name, flags in (("fused", 0), ("separate", lr.FLAG_SEPARATE_SHRINK)):
        say("two slices, %s shrink" % name)
        res = {}
        cnt = launches(lambda: res.setdefault("y", lr.lora_linear_sliced(x, W, slices, ids, flags=flags)))
        out[name] = res["y"]
        assert cnt["gemm"] == 1 and cnt["sgmv_expand"] == 1, cnt
        assert cnt["sgmv_shrink"] == (0 if flags == 0 else 1), cnt
    for name, y in out.items():
        for p, lo in ((w.proj("q"), 0), (w.proj("v"), 8064)):
            ref = oracle_rows(oracle_mod, w, p)
            err = normwise(y[:, lo:lo + p.d].double().cpu().numpy(), ref)
            say("  %s %s normwise %.3g" % (name, p.name, err))
            assert err <= 2e-2
    # t summed in another order: y may differ in the last bf16 place only
    diff = normwise(out["fused"].double().cpu().numpy(), out["separate"].double().cpu().numpy())
    say("  fused vs separate normwise %.3g" % diff)
    assert diff <= 1e-2
    # rows without an adapter are the base GEMM bit for bit
    base = lr.lora_gemm(x, W)
    none = torch.from_numpy(np.flatnonzero(w.ids < 0)).cuda()
    assert torch.equal(out["fused"][none], base[none])


def test_small_adapter_set_one_pass(oracle_mod):
    """8 adapters x max_rank 64 = 512 <= 1024: one pass, no shrink launch."""
    w = wl.custom(seed=21, M=400, k=512, d=9216, ranks=[16, 64, 8, 0, 33, 64, 1, 16], max_rank=64,
                  none_frac=0.1)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    res = {}
    cnt = launches(lambda: res.setdefault("y", dw.run()))
    assert cnt["sgmv_shrink"] == 0 and cnt["gemm"] == 1 and cnt["sgmv_expand"] == 1, cnt
    err = normwise(res["y"].double().cpu().numpy(), oracle_rows(oracle_mod, w, p))
    say("no-shrink fused normwise %.3g" % err)
    assert err <= 2e-2
    ysep = dw.run(flags=lr.FLAG_SEPARATE_SHRINK)
    assert normwise(res["y"].double().cpu().numpy(), ysep.double().cpu().numpy()) <= 1e-2


def test_ranks_past_first_pass_use_the_second(oracle_mod):
    """20 adapters of rank 64 (sum 1280 > 1024): columns 1024.. come from
    the GEMM's second pass; still no shrink launch."""
    w = wl.custom(seed=22, M=400, k=512, d=9216, ranks=[64] * 20, max_rank=64, none_frac=0.05)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    res = {}
    cnt = launches(lambda: res.setdefault("y", dw.run()))
    assert cnt["sgmv_shrink"] == 0, cnt
    y = res["y"]
    err = normwise(y.double().cpu().numpy(), oracle_rows(oracle_mod, w, p))
    say("second pass normwise %.3g" % err)
    assert err <= 2e-2
    ysep = dw.run(flags=lr.FLAG_SEPARATE_SHRINK)
    assert normwise(y.double().cpu().numpy(), ysep.double().cpu().numpy()) <= 1e-2


def test_too_many_ranks_are_not_folded(oracle_mod):
    """40 adapters x max_rank 64 = 2560 > two passes of 1024: the shrink runs
    as its own kernel."""
    w = wl.custom(seed=25, M=400, k=256, d=9216, ranks=[64, 8] * 20, max_rank=64)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    res = {}
    cnt = launches(lambda: res.setdefault("y", dw.run()))
    assert cnt["sgmv_shrink"] == 1, cnt
    err = normwise(res["y"].double().cpu().numpy(), oracle_rows(oracle_mod, w, p))
    assert err <= 2e-2


def test_out_of_range_ranks_are_clamped_and_ignored(oracle_mod):
    """A rank above max_rank or below zero: the fold clamps it (no read past
    the slot) and the plan turns that adapter's rows into base rows.  With
    rank 64 clamped in, the sum (16 + 64 + 0 + 32) stays in one pass."""
    w = wl.custom(seed=23, M=400, k=512, d=9216, ranks=[16, 64, 8, 32], max_rank=64)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    dw.ranks[1] = 1000
    dw.ranks[2] = -3
    y = dw.run()
    ids = w.ids.copy()
    ids[np.isin(ids, [1, 2])] = -1
    err = normwise(y.double().cpu().numpy(), oracle_rows(oracle_mod, w, p, ids=ids))
    say("clamped ranks normwise %.3g" % err)
    assert err <= 2e-2
    base = lr.lora_gemm(dw.x, dw.W)
    bad = torch.from_numpy(np.flatnonzero(np.isin(w.ids, [1, 2]))).cuda()
    assert torch.equal(y[bad], base[bad])


def test_reuse_plan_with_fold():
    """A second call on the same ids with LORA_FLAG_REUSE_PLAN gives the same bits."""
    w = wl.custom(seed=24, M=400, k=512, d=9216, ranks=[16, 64, 8, 0, 33, 64, 1, 16], max_rank=64)
    dw = DevWorkload(w, w.projections[0])
    y1 = dw.run()
    y2 = dw.run(flags=lr.FLAG_REUSE_PLAN)
    assert torch.equal(y1, y2)


def pooled_pair(w, page_bytes):
    """Device slices for a two-projection workload with each slice's
    adapters in its own paged pool (seeded physical pages, NaN elsewhere)."""
    dev = torch.device("cuda")
    ranks = torch.from_numpy(w.ranks).to(dev)
    scales = torch.from_numpy(w.scales).to(dev)
    slices, keep = [], []
    for i, p in enumerate((w.proj("q"), w.proj("v"))):
        pool, table, _n = wl.pool(w, p, page_bytes=page_bytes, seed_offset=i)
        pool, table = pool.to(dev), table.to(dev)
        keep.append((pool, table))
        slices.append(lr.Slice(p.d, lr.Adapters.paged(pool, table, ranks, page_bytes, w.max_rank),
                               scales))
    W = torch.cat([w.proj("q").W, w.proj("v").W], dim=0).contiguous().to(dev)
    return W, slices, keep


@pytest.mark.parametrize("page_bytes", [4096, 1 << 20])
def test_two_slices_fused_from_pools(oracle_mod, page_bytes):
    """The fold reading A rows from paged pools ("S-LoRA: ...", "Unified
    paging"): pages a multiple of the 1 KiB A row (k = 512), so every row
    lies in one page; at 4 KiB an adapter's A spans up to 16 pages.  No
    shrink launched; every row against the oracle; bitwise equal to the
    same adapters in slots (same arithmetic, other addresses)."""
    w = wl.c3_proj70b_bf16(M=400, k=512, d_q=8064, d_v=1152)
    W, slices, _keep = pooled_pair(w, page_bytes)
    x, ids = w.x.cuda(), torch.from_numpy(w.ids).cuda()
    say("two pooled slices, fused shrink, %d-byte pages" % page_bytes)
    res = {}
    cnt = launches(lambda: res.setdefault("y", lr.lora_linear_sliced(x, W, slices, ids)))
    y = res["y"]
    assert cnt["gemm"] == 1 and cnt["sgmv_shrink"] == 0 and cnt["sgmv_expand"] == 1, cnt
    for p, lo in ((w.proj("q"), 0), (w.proj("v"), 8064)):
        ref = oracle_rows(oracle_mod, w, p)
        err = normwise(y[:, lo:lo + p.d].double().cpu().numpy(), ref)
        say("  %s normwise %.3g" % (p.name, err))
        assert err <= 2e-2
    Ws, sslices, _k2 = sliced_pair(w)
    ys = lr.lora_linear_sliced(x, Ws, sslices, ids)
    torch.cuda.synchronize()
    assert torch.equal(y, ys)


def test_fused_pool_bad_page_entry_reads_no_adapter():
    """A page-table entry outside the pool: the fold must not read through
    it (its rows read x, their t is unused), the plan counts the adapter's
    rows as bad pages and they get the base output."""
    w = wl.c3_proj70b_bf16(M=400, k=512, d_q=8064, d_v=1152)
    W, slices, keep = pooled_pair(w, 4096)
    x, ids = w.x.cuda(), torch.from_numpy(w.ids).cuda()
    table_q = keep[0][1]
    bad = 9  # a rank-64 adapter: its A rows sit in the fold's columns
    table_q[bad, 3] = 1 << 30
    say("fused pool, page entry outside the pool")
    ws = torch.zeros(lr.workspace_bytes_sliced(w.M, w.k, torch.bfloat16, slices),
                     dtype=torch.uint8, device="cuda")
    y = lr.lora_linear_sliced(x, W, slices, ids, workspace=ws)
    chk = lr.lora_check(ws)
    n_bad = int((w.ids == bad).sum())
    assert n_bad > 0 and chk["n_bad_pages"] == n_bad, chk
    base = lr.lora_gemm(x, W)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.flatnonzero(w.ids == bad)).cuda()
    assert torch.equal(y[rows], base[rows])


# ---------------------------------------------------------------------------
# The fold at decode sizes: 64 x 64 tiles.  Each column tile carries 16 t
# columns past its 64 W rows; column j of column tile tn is entry 16 tn + j
# (then cap + 16 tn + j for the second pass) of the list of every slot row
# (slice, adapter, rank < the slice's max_rank), so the columns past an
# adapter's rank are computed too and must never be read.
# ---------------------------------------------------------------------------

def check_fused_one(oracle_mod, w, pad, expect_shrink=0):
    p = w.projections[0]
    dw = DevWorkload(w, p, pad_value=pad)
    res = {}
    cnt = launches(lambda: res.setdefault("y", dw.run()))
    assert cnt["gemm"] == 1 and cnt["sgmv_expand"] == 1, cnt
    assert cnt["sgmv_shrink"] == expect_shrink, cnt
    y = res["y"]
    err = normwise(y.double().cpu().numpy(), oracle_rows(oracle_mod, w, p))
    say("  normwise %.3g" % err)
    assert err <= 2e-2
    ysep = dw.run(flags=lr.FLAG_SEPARATE_SHRINK)
    assert normwise(y.double().cpu().numpy(), ysep.double().cpu().numpy()) <= 1e-2
    base = lr.lora_gemm(dw.x, dw.W)
    torch.cuda.synchronize()
    none = torch.from_numpy(np.flatnonzero(w.ids < 0)).cuda()
    assert torch.equal(y[none], base[none])
    return dw, y


@pytest.mark.parametrize("M,k,d,ranks,R", [
    (200, 320, 1000, [16, 8, 0, 13, 16, 4], 16),   # ragged rows and columns, one pass
    (150, 128, 128, [16, 16, 16], 16),             # 48 entries past the 32-column first pass
    (64, 320, 64, [8, 3], 8),                      # one tile, the first pass exactly full
])
@pytest.mark.parametrize("pad", [0.0, float("nan")])
def test_decode_tiles_fused(oracle_mod, M, k, d, ranks, R, pad):
    """bf16 slots at shapes run as 64 x 64 tiles: no shrink launched; every
    row against the oracle; within bf16 rounding of the separate shrink;
    rows without an adapter bitwise the base GEMM.  pad = NaN fills the
    slots past each adapter's rank (A rows and B columns), which the fold
    multiplies into t columns that the expand must not read."""
    w = wl.custom(seed=40 + M + d, M=M, k=k, d=d, ranks=ranks, max_rank=R, none_frac=0.1)
    say("decode tiles fused: M=%d k=%d d=%d ranks=%s pad=%s" % (M, k, d, ranks, pad))
    check_fused_one(oracle_mod, w, pad)


def test_decode_tiles_fused_c1(oracle_mod):
    """The decode-4096 workload (256 rows, 4 slots of rank 16) on its
    benchmarked path: the shrink folded into the 64 x 64 GEMM; sampled rows
    of every adapter against the oracle."""
    w = wl.c1_decode_bf16()
    p = w.projections[0]
    dw = DevWorkload(w, p)
    res = {}
    cnt = launches(lambda: res.setdefault("y", dw.run()))
    assert cnt["gemm"] == 1 and cnt["sgmv_shrink"] == 0 and cnt["sgmv_expand"] == 1, cnt
    rows = np.concatenate([np.flatnonzero(w.ids == a)[:6] for a in range(-1, w.S)])
    ref = oracle_rows(oracle_mod, w, p, rows=rows)
    err = normwise(res["y"][torch.from_numpy(rows).cuda()].double().cpu().numpy(), ref)
    say("c1 fused sampled normwise %.3g" % err)
    assert err <= 2e-2


def test_decode_tiles_two_slices_two_passes(oracle_mod):
    """q + v slices with the 70B adapter set at 128 rows and sum d = 3072:
    48 column tiles, a 768-column first pass, 1536 slot rows -- the second
    pass carries half of them.  Slots, then the same adapters in 4 KiB
    pages (bitwise the same output)."""
    w = wl.c3_proj70b_bf16(M=128, k=256, d_q=2560, d_v=512)
    W, slices, _keep = sliced_pair(w)
    x, ids = w.x.cuda(), torch.from_numpy(w.ids).cuda()
    res = {}
    cnt = launches(lambda: res.setdefault("y", lr.lora_linear_sliced(x, W, slices, ids)))
    assert cnt["gemm"] == 1 and cnt["sgmv_shrink"] == 0 and cnt["sgmv_expand"] == 1, cnt
    y = res["y"]
    for p, lo in ((w.proj("q"), 0), (w.proj("v"), 2560)):
        err = normwise(y[:, lo:lo + p.d].double().cpu().numpy(), oracle_rows(oracle_mod, w, p))
        say("  %s normwise %.3g" % (p.name, err))
        assert err <= 2e-2
    Wp, pslices, _kp = pooled_pair(w, 4096)
    yp = lr.lora_linear_sliced(x, Wp, pslices, ids)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)


def test_decode_tiles_out_of_range_ranks(oracle_mod):
    """Ranks above max_rank or below zero at 64 x 64 tiles: the fold's list
    does not depend on them; the plan turns those adapters' rows into base
    rows."""
    w = wl.custom(seed=47, M=200, k=320, d=1000, ranks=[16, 16, 8, 4], max_rank=16)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    dw.ranks[1] = 1000
    dw.ranks[2] = -3
    y = dw.run()
    ids = w.ids.copy()
    ids[np.isin(ids, [1, 2])] = -1
    err = normwise(y.double().cpu().numpy(), oracle_rows(oracle_mod, w, p, ids=ids))
    assert err <= 2e-2
    base = lr.lora_gemm(dw.x, dw.W)
    bad = torch.from_numpy(np.flatnonzero(np.isin(w.ids, [1, 2]))).cuda()
    assert torch.equal(y[bad], base[bad])
