"""The merged single-adapter weight (lora_merge) on the GPU against the fp64
oracle, through the C ABI.

Tolerances: bf16 W' is one RNE rounding of W + coef*s*BA with an fp32 sum,
so each element is within half a bf16 ulp (2^-8 relative) of the fp64 value
plus the fp32 summation error; checked as |W' - ref| <= 2^-8 |ref| + 1e-6
max|ref| elementwise.  fp32: normwise 1e-5.  The layer over the merged
weight (lora_gemm) is held to the layer's tolerance (2e-2 bf16).
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


def check_merged(got: torch.Tensor, ref: np.ndarray, dtype, what: str):
    g = got.double().cpu().numpy()
    if dtype == torch.bfloat16:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.max(np.abs(ref))
        bad = np.abs(g - ref) > bound
        assert not bad.any(), "%s: %d elements off by more than half a bf16 ulp" % (what, int(bad.sum()))
    else:
        err = normwise(g, ref)
        assert err <= 1e-5, "%s: normwise %g" % (what, err)


CASES = [
    # seed, d, k, ranks, max_rank, dtype
    (1, 256, 256, [4, 16, 64, 1], 64, torch.bfloat16),
    (2, 300, 520, [33, 7, 0, 64], 64, torch.bfloat16),     # ragged d and k tails, rank 0
    (3, 136, 1024, [100, 5, 128], 128, torch.bfloat16),   # ranks above 64
    (4, 200, 264, [8, 31, 64], 64, torch.float32),
    (5, 70, 260, [3, 96], 96, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "s%d_%dx%d_%s" % (c[0], c[1], c[2], str(c[5])[6:]))
@pytest.mark.parametrize("pooled", [False, True], ids=["slots", "pool"])
def test_merge_matches_oracle(oracle_mod, case, pooled):
    seed, d, k, ranks, R, dtype = case
    w = wl.custom(seed=seed, M=64, k=k, d=d, ranks=ranks, max_rank=R, dtype=dtype)
    p = w.projections[0]
    dw = DevWorkload(w, p, pooled=pooled, page_bytes=4096 if pooled else None)
    for s in range(w.S):
        for coef in (1.0, -1.0):
            say("merge %s %s adapter %d coef %g" % (case[:3], "pool" if pooled else "slots", s, coef))
            out = lr.lora_merge(dw.W, dw.ad, s, dw.scales, coef=coef)
            torch.cuda.synchronize()
            ref = oracle_mod.merge(p.W, p.A[s], p.B[s], float(w.scales[s]), coef=coef)
            check_merged(out, ref, dtype, "adapter %d coef %g" % (s, coef))
            if ranks[s] == 0:
                assert torch.equal(out, dw.W)


def test_merge_in_place_and_strided():
    w = wl.custom(seed=7, M=64, k=512, d=384, ranks=[16, 64], max_rank=64)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    ref = lr.lora_merge(dw.W, dw.ad, 1, dw.scales)
    Wc = dw.W.clone()
    lr.lora_merge(Wc, dw.ad, 1, dw.scales, out=Wc)
    assert torch.equal(Wc, ref)
    # leading dimensions larger than k on both sides
    big = torch.zeros(384, 640, dtype=torch.bfloat16, device="cuda")
    big[:, :512] = dw.W
    outb = torch.full((384, 576), 7.0, dtype=torch.bfloat16, device="cuda")
    lr.lora_merge(big[:, :512], dw.ad, 1, dw.scales, out=outb[:, :512])
    torch.cuda.synchronize()
    assert torch.equal(outb[:, :512], ref)
    assert torch.all(outb[:, 512:] == 7.0)  # nothing written past k


def test_merged_layer_matches_oracle(oracle_mod):
    """One adapter carries every row: lora_gemm over the merged weight gives
    the layer (oracle) to the layer's tolerance, and matches lora_linear."""
    w = wl.custom(seed=8, M=256, k=1024, d=768, ranks=[16, 64], max_rank=64)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    for s in range(w.S):
        say("merged layer adapter %d" % s)
        Wm = lr.lora_merge(dw.W, dw.ad, s, dw.scales)
        y = lr.lora_gemm(dw.x, Wm)
        ids = np.full(w.M, s, np.int32)
        ref = oracle_rows(oracle_mod, w, p, ids=ids)
        assert normwise(y.double().cpu().numpy(), ref) <= 2e-2
        y_add = dw.run(ids=torch.from_numpy(ids).cuda())
        assert normwise(y.double().cpu().numpy(), y_add.double().cpu().numpy()) <= 2e-2


def test_merge_device_errors_copy_w():
    w = wl.custom(seed=9, M=64, k=256, d=128, ranks=[8, 16], max_rank=16)
    p = w.projections[0]
    dw = DevWorkload(w, p)
    dw.ranks[1] = 17  # above max_rank
    out = lr.lora_merge(dw.W, dw.ad, 1, dw.scales)
    torch.cuda.synchronize()
    assert torch.equal(out, dw.W)
    dp = DevWorkload(w, p, pooled=True, page_bytes=4096)
    dp.table[0, 0] = -1  # a missing page
    out = lr.lora_merge(dp.W, dp.ad, 0, dp.scales)
    torch.cuda.synchronize()
    assert torch.equal(out, dp.W)
    dp.table[0, 0] = int(dp.pool.numel() // 4096)  # a page past the pool
    out = lr.lora_merge(dp.W, dp.ad, 0, dp.scales)
    torch.cuda.synchronize()
    assert torch.equal(out, dp.W)


@pytest.fixture(scope="module")
def c3():
    return wl.c3_proj70b_bf16()


@pytest.mark.parametrize("proj", ["q", "v"])
def test_merge_c3_sampled(oracle_mod, c3, proj):
    """The 70B shapes (8192 x 8192 and 1024 x 8192), each rank of the set, on
    sampled rows of W' (the merge is row-independent)."""
    p = c3.proj(proj)
    dw = DevWorkload(c3, p)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, p.d - 1], rng.integers(0, p.d, 30)]))
    for s in (0, 3, 9):  # ranks 4, 16, 64
        say("c3 %s merge adapter %d (rank %d)" % (proj, s, c3.ranks[s]))
        out = lr.lora_merge(dw.W, dw.ad, s, dw.scales)
        torch.cuda.synchronize()
        ref = oracle_mod.merge(p.W[rows], p.A[s], p.B[s][rows], float(c3.scales[s]))
        check_merged(out[torch.from_numpy(rows).cuda()], ref, torch.bfloat16, "c3 %s adapter %d" % (proj, s))
