"""Where the layer's plan runs, and that it is the oracle's wherever it runs.

"Adapter Residency When One Replica Serves Many Fine-Tunes", section
"Batch composition under many adapters": the batch's rows are grouped by
adapter into segments before the LoRA kernels run.  The plan runs inside the
base GEMM's launch where that launch can carry it without slowing its tiles
-- split-K pairs (their first-arriving workgroup) and 64 x 64 tiles (one
more workgroup beside the tiles, two of that kernel's workgroups fitting on
a CU) -- and as its own kernel elsewhere.  Checked for each tile shape the
GEMM picks (64 x 64, 128 x 128, 256 x 128, 256 x 256, 256 x 160 and
128 x 144), at ragged sizes with bad ids and ranks planted:
  - the layer's output against the fp64 oracle on every row (normwise 2e-2);
  - the plan left in the workspace bit for bit against the oracle's plan
    (including the run of more than 64 adapters, whose plan takes the
    counting sort), and the bad-row counts lora_check reports;
  - the library's launch counters: a plan kernel exactly where the GEMM
    does not carry the plan.
Pools with a bad page entry, and HIP-graph replays with new ids contents
between replays on a workspace filled with random bytes beforehand, are
checked the same way.
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
    with lr.Profiler():
        fn()
        torch.cuda.synchronize()
        prof = lr.Profiler.read(reset=True)
    return {k: prof[k]["launches"] for k in lr.KERNEL_CLASSES}


def plan_of(dw):
    got = lr.lora_plan_view(dw.ws, dw.w.M, dw.ad)
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in got.items()}


def assert_plan_equal(got, ref):
    assert got["n_adapted"] == ref["n_adapted"]
    for key in ("perm", "seg_adapter", "seg_start", "seg_len"):
        assert np.array_equal(got[key], ref[key]), key
    for key in ("n_bad_ids", "n_bad_ranks", "n_bad_pages"):
        assert got[key] == ref[key], key


# (M, k, d, whether the GEMM launch carries the plan): the tile shape the
# base GEMM picks for it
SHAPES = [
    (300, 256, 1000, True),     # 64 x 64: one more workgroup beside the tiles
    (1000, 256, 2000, False),   # 128 x 128
    (3900, 256, 2000, False),   # 256 x 128
    (4000, 256, 4000, False),   # 256 x 256, two rounds of workgroups
    (1900, 256, 5120, False),   # 256 x 160
    (120, 256, 36864, False),   # 128 x 144 (one row tile: no split-K pairs)
    (512, 256, 9216, True),     # 256 x 144 split-K pairs
]


@pytest.mark.parametrize("M,k,d,carried", SHAPES,
                         ids=["t64", "t128", "t256x128", "t256", "t256x160", "t128x144", "split"])
@pytest.mark.parametrize("n_adapters", [6, 90], ids=["S6", "S90"])
def test_plan_every_tile(oracle_mod, M, k, d, carried, n_adapters):
    say("plan M=%d k=%d d=%d, %d adapters" % (M, k, d, n_adapters))
    R = 16
    rng = np.random.default_rng(M + n_adapters)
    ranks = [4, 16, 40, 8, 1, 12] + [int(r) for r in rng.integers(1, 17, size=n_adapters - 6)]
    w = wl.custom(seed=500 + M + n_adapters, M=M, k=k, d=d, ranks=ranks, max_rank=R)
    S = len(w.ranks)
    ids = w.ids.copy()
    ids[[0, 7, M - 1]] = [-5, S, S + 77]          # bad ids, the last row among them
    dw = DevWorkload(w, w.projections[0])
    ids_t = torch.from_numpy(ids).cuda()
    counts = launches(lambda: dw.run(ids=ids_t))
    say("  launches %s" % counts)
    assert counts["gemm"] == 1
    assert counts["plan"] == (0 if carried else 1)
    y = dw.run(ids=ids_t).clone()
    ref_plan = oracle_mod.plan(ids, S, w.ranks, R)
    assert_plan_equal(plan_of(dw), ref_plan)
    chk = lr.lora_check(dw.ws)
    assert chk["n_bad_ids"] == 3
    assert chk["n_bad_ranks"] == int((ids == 2).sum())
    eff = ids.copy()
    eff[(eff < -1) | (eff >= S) | (eff == 2)] = -1
    ref = oracle_rows(oracle_mod, w, w.projections[0], ids=eff)
    err = normwise(y.double().cpu().numpy(), ref)
    say("  normwise error %.3g" % err)
    assert err <= 2e-2
    # bitwise the same again (the workspace reused)
    assert torch.equal(dw.run(ids=ids_t), y)


def test_plan_in_gemm_pool_bad_page(oracle_mod):
    M, k, d = 300, 256, 1000   # 64 x 64 tiles: the plan rides in the GEMM launch
    say("plan carried by the GEMM, pool with a bad page entry")
    w = wl.custom(seed=71, M=M, k=k, d=d, ranks=[8, 16, 4, 12], max_rank=16, page_bytes=4096)
    dw = DevWorkload(w, w.projections[0], pooled=True, page_bytes=4096)
    table = dw.table.cpu().numpy().copy()
    n_pages = dw.pool.numel() // 4096
    table[1, 0] = n_pages                          # adapter 1 reads past the pool
    dw.table.copy_(torch.from_numpy(table))
    counts = launches(lambda: dw.run())
    assert counts["plan"] == 0
    y = dw.run().double().cpu().numpy()
    ref_plan = oracle_mod.plan(w.ids, len(w.ranks), w.ranks, 16, page_table=table,
                               n_pages=n_pages, page_bytes=4096, k=k, d=d, elem_bytes=2)
    assert_plan_equal(plan_of(dw), ref_plan)
    assert lr.lora_check(dw.ws)["n_bad_pages"] == int((w.ids == 1).sum())
    eff = w.ids.copy()
    eff[eff == 1] = -1
    err = normwise(y, oracle_rows(oracle_mod, w, w.projections[0], ids=eff))
    say("  normwise error %.3g" % err)
    assert err <= 2e-2


@pytest.mark.parametrize("M,k,d", [(300, 256, 1000), (1000, 256, 2000)],
                         ids=["carried", "own_kernel"])
def test_graph_replay_plan_in_gemm_new_ids(oracle_mod, M, k, d):
    say("graph replay of the layer M=%d d=%d, new ids between replays" % (M, d))
    w = wl.custom(seed=72, M=M, k=k, d=d, ranks=[4, 16, 8], max_rank=16)
    dw = DevWorkload(w, w.projections[0])
    # a workspace that was never cleared: the exchange words start anywhere
    g = torch.Generator().manual_seed(3)
    dw.ws.copy_(torch.randint(0, 256, (dw.ws.numel(),), generator=g, dtype=torch.uint8))
    rng = np.random.default_rng(72)
    id_sets = [w.ids] + [rng.integers(-1, 3, size=M).astype(np.int32) for _ in range(2)]
    eager = []
    for ids in id_sets:
        eager.append(dw.run(ids=torch.from_numpy(ids).cuda()).clone())
    for ids, y in zip(id_sets[:2], eager[:2]):
        err = normwise(y.double().cpu().numpy(), oracle_rows(oracle_mod, w, w.projections[0],
                                                             ids=ids))
        assert err <= 2e-2
    static_ids = torch.from_numpy(id_sets[0]).cuda()
    static_y = torch.empty_like(eager[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lr.lora_linear(dw.x, dw.W, dw.ad, static_ids, dw.scales, y=static_y, workspace=dw.ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lr.lora_linear(dw.x, dw.W, dw.ad, static_ids, dw.scales, y=static_y, workspace=dw.ws)
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 2, 2, 0, 1]):
        static_ids.copy_(torch.from_numpy(id_sets[i]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(static_y, eager[i])
        say("  replay %d (ids %d): bitwise equal to eager: %s" % (rep, i, same))
        assert same
        y2 = dw.run(ids=torch.from_numpy(id_sets[(i + 1) % 3]).cuda())
        assert torch.equal(y2, eager[(i + 1) % 3])
    del graph
