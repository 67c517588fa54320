"""lora_linear_sliced_noalloc: the layer without a workspace argument, over
the library's static per-GPU scratch array (for callers that cannot
allocate).  Its output must be the workspace entry point's, bit for bit (the
same kernels run; only where the plan runs differs), on consecutive calls
whose sizes shrink -- the array keeps the previous call's contents -- and a
call too large for the array must be refused before anything is launched."""
import numpy as np
import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl
from gpu_helpers import DevWorkload, normwise, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    torch.cuda.set_device(0)
    lr.load_library()
    yield
    torch.cuda.synchronize()


def _pair(w):
    pq, pv = w.proj("q"), w.proj("v")
    dq, dv = DevWorkload(w, pq), DevWorkload(w, pv)
    W = torch.cat([dq.W, dv.W], dim=0).contiguous()
    slices = [lr.Slice(pq.d, dq.ad, dq.scales), lr.Slice(pv.d, dv.ad, dv.scales)]
    return dq, W, slices


def test_noalloc_matches_workspace_entry(oracle_mod):
    w = wl.c3_proj70b_bf16()
    dq, W, slices = _pair(w)
    d_total = W.shape[0]
    # 512 rows (split-K pairs, shrink folded into the GEMM), then 200 and 37
    # rows of the same batch (other tiles), then 512 again
    for M in (512, 200, 37, 512):
        say("noalloc vs workspace entry, 70B q+v shape, M=%d" % M)
        x, ids = dq.x[:M].contiguous(), dq.ids[:M].contiguous()
        need = lr.workspace_bytes_sliced(M, w.k, torch.bfloat16, slices)
        assert need <= lr.NOALLOC_SCRATCH_BYTES
        ref = lr.lora_linear_sliced(x, W, slices, ids)
        y = torch.full((M, d_total), float("nan"), dtype=torch.bfloat16, device="cuda")
        lr.lora_linear_sliced_noalloc(x, W, slices, ids, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), "M=%d differs from lora_linear_sliced" % M
        if M == 37:  # and the oracle, every row of both projections
            for name, lo, hi in (("q", 0, 8192), ("v", 8192, 9216)):
                p = w.proj(name)
                r = oracle_mod.lora_linear(w.x[:M], p.W, p.A, p.B, w.scales.astype(np.float64),
                                           w.ids[:M], max_rank=w.max_rank)
                assert normwise(y[:, lo:hi].double().cpu().numpy(), r) <= 2e-2


def test_noalloc_paths_and_pool():
    """Both kernel families and a paged pool, two calls in a row."""
    w = wl.custom(seed=55, M=300, k=512, d=384, ranks=[4, 16, 64, 8], max_rank=64)
    p = w.projections[0]
    for pooled in (False, True):
        dw = DevWorkload(w, p, pooled=pooled)
        sl = [lr.Slice(p.d, dw.ad, dw.scales)]
        for path in (lr.PATH_GATHER, lr.PATH_SGMV, lr.PATH_AUTO):
            for M in (300, 123):
                say("noalloc pooled=%s path=%d M=%d" % (pooled, path, M))
                x, ids = dw.x[:M].contiguous(), dw.ids[:M].contiguous()
                ref = lr.lora_linear_sliced(x, dw.W, sl, ids, path=path)
                y = torch.empty(M, p.d, dtype=torch.bfloat16, device="cuda")
                lr.lora_linear_sliced_noalloc(x, dw.W, sl, ids, y=y, path=path)
                torch.cuda.synchronize()
                assert torch.equal(y, ref)


def test_noalloc_refuses_calls_past_its_array():
    """8192 rows of the 70B q+v pair need more than the array holds: the
    call returns LORA_ERR_WORKSPACE and y is left as it was (real, in-bounds
    buffers are passed all the same)."""
    say("noalloc size limit")
    w = wl.c3_proj70b_bf16(M=64)
    dq, W, slices = _pair(w)
    M = 8192
    assert lr.workspace_bytes_sliced(M, w.k, torch.bfloat16, slices) > lr.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(M, w.k, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(M, dtype=torch.int32, device="cuda")
    y = torch.full((M, W.shape[0]), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lr.LoraError) as e:
        lr.lora_linear_sliced_noalloc(x, W, slices, ids, y=y)
    assert e.value.status == 5  # LORA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
