"""Quantized base weights (INT8 per-row scales, INT4 per-row-and-group
scales) on the GPU against the fp64 oracle, through the C ABI.

The oracle dequantizes exactly (oracle.dequant_int8 / dequant_int4) and runs
the layer in fp64.  Tolerance: normwise 2e-2, as for every bf16 output of the
layer (INT8 weights are exact in bf16 and the row scale multiplies the fp32
sum; INT4 weights are rounded once to bf16 after scaling, a relative error of
at most 2^-9 per weight).  Rows without an adapter equal lora_gemm_q bitwise.
"""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import normwise, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


def make_q(w, fmt, group, names=None):
    q, s = wl.quantized_base(w, fmt, group=group, names=names)
    qw = lr.QWeight(lr.W_INT8 if fmt == "int8" else lr.W_INT4, q.cuda(), s.cuda(), w.k,
                    group=group if fmt == "int4" else 0)
    return qw, q.numpy(), s.numpy()


def dequant(oracle_mod, fmt, q, s, group, k):
    if fmt == "int8":
        return oracle_mod.dequant_int8(q.view(np.int8), s)
    return oracle_mod.dequant_int4(q, s, group, k)


GEMM_CASES = [
    # seed, M, k, d, fmt, group
    # small shapes run 64 x 64 tiles; the 70B test below runs 128 x 144
    (1, 37, 256, 200, "int8", 0),     # ragged M and d
    (2, 300, 1024, 288, "int8", 0),
    (3, 64, 512, 96, "int8", 0),
    (4, 37, 256, 200, "int4", 64),
    (5, 300, 1024, 288, "int4", 128),
    (6, 130, 768, 150, "int4", 256),
    (7, 1024, 256, 2048, "int8", 0),   # 128 x 128 tiles (two rounds of 64 x 64 would cost more)
    (8, 1024, 256, 2048, "int4", 64),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "%s_g%d_%dx%dx%d" % (c[4], c[5], c[1], c[2], c[3]))
def test_gemm_q_matches_oracle(oracle_mod, case):
    seed, M, k, d, fmt, group = case
    say("gemm_q %s" % (case,))
    w = wl.custom(seed=seed, M=M, k=k, d=d, ranks=[4], max_rank=4)
    qw, q, s = make_q(w, fmt, group or 128)
    x = w.x.cuda()
    y = lr.lora_gemm_q(x, qw)
    torch.cuda.synchronize()
    Wd = dequant(oracle_mod, fmt, q, s, group or 128, k)
    ref = w.x.double().numpy() @ Wd.T
    err = normwise(y.double().cpu().numpy(), ref)
    say("  normwise error %.3g" % err)
    assert err <= 2e-2


@pytest.mark.parametrize("fmt,group", [("int8", 0), ("int4", 128)])
def test_linear_q_layer(oracle_mod, fmt, group):
    """The whole layer over a quantized base: every row against the oracle
    layer with the exactly dequantized weight; none rows bitwise equal to
    lora_gemm_q; every path."""
    w = wl.custom(seed=11, M=300, k=1024, d=288, ranks=[4, 16, 64, 8], max_rank=64, none_frac=0.1)
    p = w.projections[0]
    qw, q, s = make_q(w, fmt, group or 128)
    Wd = dequant(oracle_mod, fmt, q, s, group or 128, w.k)
    A, B = wl.slots(w, p)
    ad = lr.Adapters.slots(A.cuda(), B.cuda(), torch.from_numpy(w.ranks).cuda())
    scales = torch.from_numpy(w.scales).cuda()
    x, ids = w.x.cuda(), torch.from_numpy(w.ids).cuda()
    ref = oracle_mod.lora_linear(w.x, Wd, p.A, p.B, w.scales.astype(np.float64), w.ids,
                                 max_rank=w.max_rank)
    base = lr.lora_gemm_q(x, qw)
    for path in (lr.PATH_AUTO, lr.PATH_GATHER, lr.PATH_SGMV):
        say("linear_q %s path %d" % (fmt, path))
        y = lr.lora_linear_sliced_q(x, qw, [lr.Slice(p.d, ad, scales)], ids, path=path)
        torch.cuda.synchronize()
        assert normwise(y.double().cpu().numpy(), ref) <= 2e-2
        none = torch.from_numpy(np.flatnonzero(w.ids < 0)).cuda()
        assert torch.equal(y[none], base[none])


@pytest.fixture(scope="module")
def c3():
    return wl.c3_proj70b_bf16()


@pytest.mark.parametrize("fmt,group", [("int8", 0), ("int4", 128)])
def test_linear_q_c3(oracle_mod, c3, fmt, group):
    """The 70B q+v pair with an INT8 / INT4 stacked base weight, every row
    (so every adapter) against the oracle layer over the exactly dequantized
    weight."""
    say("c3 quantized %s" % fmt)
    pq, pv = c3.proj("q"), c3.proj("v")
    qw, q, s = make_q(c3, fmt, group or 128, names=["q", "v"])
    dev = torch.device("cuda")
    ranks = torch.from_numpy(c3.ranks).to(dev)
    scales = torch.from_numpy(c3.scales).to(dev)
    slices = []
    for p in (pq, pv):
        A, B = wl.slots(c3, p)
        slices.append(lr.Slice(p.d, lr.Adapters.slots(A.to(dev), B.to(dev), ranks), scales))
    x, ids = c3.x.to(dev), torch.from_numpy(c3.ids).to(dev)
    y = lr.lora_linear_sliced_q(x, qw, slices, ids)
    torch.cuda.synchronize()
    if fmt == "int8":
        Wd = oracle_mod.dequant_int8(q.view(np.int8), s)
    else:
        Wd = oracle_mod.dequant_int4(q, s, group, c3.k)
    for name, p, lo, hi in (("q", pq, 0, pq.d), ("v", pv, pq.d, pq.d + pv.d)):
        ref = oracle_mod.lora_linear(c3.x, Wd[lo:hi], p.A, p.B, c3.scales.astype(np.float64),
                                     c3.ids, max_rank=c3.max_rank)
        err = normwise(y[:, lo:hi].double().cpu().numpy(), ref)
        say("  %s normwise error %.3g" % (name, err))
        assert err <= 2e-2


def test_q_argument_errors():
    x = torch.zeros(8, 128, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(64, 128, dtype=torch.uint8, device="cuda")
    s = torch.ones(64, device="cuda")
    bad = [
        lr.QWeight(lr.W_INT4, q[:, :64], torch.ones(64, 2, device="cuda"), 128, group=96),  # group % 64
        lr.QWeight(lr.W_INT4, q[:, :64], torch.ones(64, 1, device="cuda"), 128, group=256),  # k % group
        lr.QWeight(3, q, s, 128),                                                         # format
    ]
    for qw in bad:
        with pytest.raises(lr.LoraError):
            lr.lora_gemm_q(x, qw)
    with pytest.raises(lr.LoraError):  # k not a multiple of 64
        lr.lora_gemm_q(torch.zeros(8, 96, dtype=torch.bfloat16, device="cuda"),
                       lr.QWeight(lr.W_INT8, q, s, 96))
