"""The layer under HIP-graph capture, and the split-K pairs' error path.

"LoRA Adapters: Many Models in One", "The model runner's part": the decode
step is captured once into a graph over static buffers and replayed with
new contents.  The benchmarked 70B q+v call runs its base GEMM as split-K
workgroup pairs that meet through words in the workspace; a replay reuses
the launch arguments captured once, so those words must come back to their
starting state after every launch.  Checked: one lora_linear_sliced call at
the 70B q+v shape (and one lora_gemm) captured, replayed with two different
x in turn -- with eager calls on the same workspace between replays -- and
every replay bitwise equal to the eager result for its x, which is itself
compared with the oracle on every row.

The pairs' bounded wait is exercised from the host: with the testing hook
set to 0 polls every second workgroup gives up at once (its tile is wrong,
every workgroup exits normally) and lora_check counts each pair once.
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import DevWorkload, normwise, oracle_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    lr.test_sync_spin_limit(-1)
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def c3():
    return wl.c3_proj70b_bf16()


def _other_x(w, seed):
    g = np.random.default_rng(np.random.SeedSequence(20261202 + 3 + 7919 * seed))
    return torch.from_numpy(g.standard_normal((w.M, w.k), dtype=np.float32)).to(torch.bfloat16)


def test_graph_replay_c3_sliced(oracle_mod, c3):
    say("graph capture of lora_linear_sliced at the 70B q+v shape")
    pq, pv = c3.proj("q"), c3.proj("v")
    dq, dv = DevWorkload(c3, pq), DevWorkload(c3, pv)
    W = torch.cat([dq.W, dv.W], dim=0).contiguous()
    slices = [lr.Slice(pq.d, dq.ad, dq.scales), lr.Slice(pv.d, dv.ad, dv.scales)]
    ws = torch.zeros(lr.workspace_bytes_sliced(c3.M, c3.k, torch.bfloat16, slices),
                     dtype=torch.uint8, device="cuda")
    xs = [dq.x, _other_x(c3, 1).cuda(), _other_x(c3, 2).cuda()]
    eager = []
    for x in xs:
        eager.append(lr.lora_linear_sliced(x, W, slices, dq.ids, workspace=ws).clone())
    torch.cuda.synchronize()
    # the eager results against the oracle, every row of both projections
    for i in (0, 1):
        for name, p, lo, hi in (("q", pq, 0, pq.d), ("v", pv, pq.d, pq.d + pv.d)):
            ref = oracle_full(oracle_mod, c3, p, x=xs[i].cpu())
            err = normwise(eager[i][:, lo:hi].double().cpu().numpy(), ref)
            say("  eager x%d %s normwise error %.3g" % (i, name, err))
            assert err <= 2e-2

    static_x = xs[0].clone()
    static_y = torch.empty_like(eager[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture's stream kind
        lr.lora_linear_sliced(static_x, W, slices, dq.ids, y=static_y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.lora_linear_sliced(static_x, W, slices, dq.ids, y=static_y, workspace=ws)
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 0, 1, 1, 0]):
        static_x.copy_(xs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(static_y, eager[i])
        say("  replay %d (x%d): bitwise equal to eager: %s" % (rep, i, same))
        assert same
        # eager work through the same workspace between replays (other epochs)
        y2 = lr.lora_linear_sliced(xs[2], W, slices, dq.ids, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y2, eager[2])
    assert lr.lora_check(ws)["n_sync_expired"] == 0
    del g


def test_graph_replay_split_gemm():
    M, k, d = 512, 8192, 9216
    say("graph capture of the split-K lora_gemm M=%d k=%d d=%d" % (M, k, d))
    n = lr.gemm_workspace_bytes(M, k, d, torch.bfloat16)
    assert n > 0
    gen = torch.Generator().manual_seed(77)
    W = (torch.randn(d, k, generator=gen) / k ** 0.5).to(torch.bfloat16).cuda()
    xs = [torch.randn(M, k, generator=gen).to(torch.bfloat16).cuda() for _ in range(2)]
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    eager = [lr.lora_gemm(x, W, workspace=ws).clone() for x in xs]
    torch.cuda.synchronize()
    for x, y in zip(xs, eager):  # textbook product, sampled rows of each row tile
        rows = torch.tensor([0, 1, 255, 256, 300, 511])
        ref = x[rows].double().cpu().numpy() @ W.double().cpu().numpy().T
        assert normwise(y[rows.cuda()].double().cpu().numpy(), ref) <= 2e-2
    static_x, static_y = xs[0].clone(), torch.empty_like(eager[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lr.lora_gemm(static_x, W, y=static_y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.lora_gemm(static_x, W, y=static_y, workspace=ws)
    for rep, i in enumerate([0, 1, 1, 0, 1]):
        static_x.copy_(xs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_y, eager[i]), "replay %d" % rep
        lr.lora_gemm(xs[1 - i], W, workspace=ws)
        torch.cuda.synchronize()
    assert lr.lora_check(ws)["n_sync_expired"] == 0
    del g


def test_split_wait_expiry_is_counted(c3):
    """With the wait bound forced to 0 polls every pair's second half gives
    up at once: each pair is counted exactly once, for lora_gemm in its own
    workspace and for the layer in its plan header; with the default bound
    the results are bitwise those of before and the counts stay."""
    M, k, d = 512, 512, 9216
    say("split-K wait expiry forced from the host")
    P = ((M + 255) // 256) * ((d + 143) // 144)
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(M, k, generator=gen).to(torch.bfloat16).cuda()
    W = (torch.randn(d, k, generator=gen) / k ** 0.5).to(torch.bfloat16).cuda()
    ws = torch.zeros(lr.gemm_workspace_bytes(M, k, d, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    y0 = lr.lora_gemm(x, W, workspace=ws).clone()
    assert lr.lora_check(ws)["n_sync_expired"] == 0
    lr.test_sync_spin_limit(0)
    try:
        lr.lora_gemm(x, W, workspace=ws)
        torch.cuda.synchronize()
    finally:
        lr.test_sync_spin_limit(-1)
    assert lr.lora_check(ws)["n_sync_expired"] == P
    y1 = lr.lora_gemm(x, W, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0)
    assert lr.lora_check(ws)["n_sync_expired"] == P

    # the layer: counted in the workspace's plan header
    w = wl.custom(seed=90, M=M, k=k, d=d, ranks=[4, 16, 64], max_rank=64)
    dw = DevWorkload(w, w.projections[0])
    ref = dw.run().clone()
    assert lr.lora_check(dw.ws)["n_sync_expired"] == 0
    lr.test_sync_spin_limit(0)
    try:
        dw.run()
    finally:
        lr.test_sync_spin_limit(-1)
    assert lr.lora_check(dw.ws)["n_sync_expired"] == P
    assert torch.equal(dw.run(), ref)
