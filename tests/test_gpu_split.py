"""Split-K workgroup pairs of the base GEMM (256 x 144 tiles, each computed by
two workgroups over the two halves of k; the second to arrive adds the
first one's fp32 partial from the workspace), and the unsplit 256 x 160
tiles of the same eight-wave kernel.

They run where the GEMM would otherwise use 128 x 144 tiles with more than
one 128-row tile -- e.g. 385..512 rows with d in (8192, 9216] -- and only
with a workspace of lora_gemm_workspace_bytes.  Checked here against a
textbook fp64 product (numpy) and against the unsplit tiles of the same
shape: the results agree to the bf16 tolerance (another fp32 summation
order), repeated calls through one workspace stay bitwise equal (the
arrival order of the two halves does not change the sum), and a workspace
full of arbitrary bytes needs no clearing.
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from gpu_helpers import normwise, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


def _operands(M, k, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, k, generator=g).to(torch.bfloat16)
    W = (torch.randn(d, k, generator=g) / k ** 0.5).to(torch.bfloat16)
    return x, W


def _ref(x, W):
    return x.double().numpy() @ W.double().numpy().T


def _no_workspace():
    return torch.empty(0, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("M,k,d", [(512, 256, 9216), (400, 384, 9216), (385, 256, 8352),
                                   (512, 1024, 9216)])
def test_split_pairs_match_fp64_and_unsplit(M, k, d):
    say("split gemm M=%d k=%d d=%d" % (M, k, d))
    n = lr.gemm_workspace_bytes(M, k, d, torch.bfloat16)
    assert n > 0, "shape expected to run split-K pairs"
    x, W = _operands(M, k, d, M + k + d)
    xd, Wd = x.cuda(), W.cuda()
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    y_split = lr.lora_gemm(xd, Wd, workspace=ws)
    y_plain = lr.lora_gemm(xd, Wd, workspace=_no_workspace())
    torch.cuda.synchronize()
    ref = _ref(x, W)
    e_split = normwise(y_split.double().cpu().numpy(), ref)
    e_plain = normwise(y_plain.double().cpu().numpy(), ref)
    say("  split %.3g unsplit %.3g" % (e_split, e_plain))
    assert e_split <= TOL and e_plain <= TOL
    # the two summation orders differ by at most a couple of bf16 ulps
    assert normwise(y_split.double().cpu().numpy(), y_plain.double().cpu().numpy()) <= 2e-2


def test_split_repeated_calls_are_bitwise_stable_with_dirty_workspace():
    M, k, d = 512, 512, 9216
    say("split gemm repeated calls, workspace of random bytes")
    n = lr.gemm_workspace_bytes(M, k, d, torch.bfloat16)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    xs = [_operands(M, k, d, 100 + i) for i in range(3)]
    W = xs[0][1].cuda()
    first = []
    for rep in range(2):
        for i, (x, _) in enumerate(xs):
            y = lr.lora_gemm(x.cuda(), W, workspace=ws)
            torch.cuda.synchronize()
            if rep == 0:
                assert normwise(y.double().cpu().numpy(), _ref(x, xs[0][1])) <= TOL
                first.append(y.clone())
            else:
                assert torch.equal(y, first[i]), "call %d changed bits" % i


def test_small_workspace_falls_back_to_unsplit_tiles():
    M, k, d = 512, 256, 9216
    say("split gemm, workspace one byte short")
    n = lr.gemm_workspace_bytes(M, k, d, torch.bfloat16)
    x, W = _operands(M, k, d, 7)
    xd, Wd = x.cuda(), W.cuda()
    short = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    y_short = lr.lora_gemm(xd, Wd, workspace=short)
    y_plain = lr.lora_gemm(xd, Wd, workspace=_no_workspace())
    torch.cuda.synchronize()
    assert torch.equal(y_short, y_plain)


@pytest.mark.parametrize("M,k,d", [(2048, 256, 5120), (1900, 320, 5120)])
def test_wide_tiles_match_fp64(M, k, d):
    """Unsplit 256 x 160 tiles (2048 rows x 5120 columns: 256 tiles), with a
    ragged last row tile; no workspace involved."""
    say("wide-tile gemm M=%d k=%d d=%d" % (M, k, d))
    assert lr.gemm_workspace_bytes(M, k, d, torch.bfloat16) == 0
    x, W = _operands(M, k, d, 17 + M)
    y = lr.lora_gemm(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    assert normwise(y.double().cpu().numpy(), _ref(x, W)) <= TOL


def test_layer_none_rows_equal_split_gemm_bitwise():
    """lora_linear's base step is the same split launch (its workspace holds
    the GEMM region), so rows without an adapter equal lora_gemm bitwise."""
    M, k, d, S, R = 512, 256, 9216, 3, 16
    say("layer none rows vs split gemm")
    x, W = _operands(M, k, d, 11)
    g = torch.Generator().manual_seed(5)
    A = (torch.randn(S, R, k, generator=g) / k ** 0.5).to(torch.bfloat16)
    B = (torch.randn(S, d, R, generator=g) * 0.1).to(torch.bfloat16)
    ids = torch.randint(-1, S, (M,), generator=g, dtype=torch.int32)
    ad = lr.Adapters.slots(A.cuda(), B.cuda(), torch.full((S,), R, dtype=torch.int32, device="cuda"))
    scales = torch.full((S,), 2.0, device="cuda")
    y = lr.lora_linear(x.cuda(), W.cuda(), ad, ids.cuda(), scales)
    base = lr.lora_gemm(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    none = (ids == -1).nonzero().flatten().cuda()
    assert none.numel() > 0
    assert torch.equal(y[none], base[none])
    # adapted rows: base + 2 (x A^T) B^T, fp64 reference
    xa = x.double().numpy()
    ref = _ref(x, W)
    for s in range(S):
        rows = (ids == s).nonzero().flatten().numpy()
        t = xa[rows] @ A[s].double().numpy().T
        ref[rows] += 2.0 * (t @ B[s].double().numpy().T)
    assert normwise(y.double().cpu().numpy(), ref) <= TOL
