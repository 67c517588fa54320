"""Glue for the GPU tests: move seeded workloads to the device, call the
library through its binding, and compare with the oracle."""
import hashlib
import sys

import numpy as np
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import workloads as wl

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def normwise(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(a - ref))) if ref.size else 0.0
    return diff / den if den > 0 else diff


class DevWorkload:
    """A workload's tensors on cuda:0 (one projection)."""

    def __init__(self, w: wl.Workload, proj: wl.Projection, pooled: bool = False,
                 page_bytes=None, pad_value: float = 0.0):
        dev = torch.device("cuda:0")
        self.w, self.p = w, proj
        self.x = w.x.to(dev)
        self.W = proj.W.to(dev)
        self.ids = torch.from_numpy(w.ids).to(dev)
        self.scales = torch.from_numpy(w.scales).to(dev)
        self.ranks = torch.from_numpy(w.ranks).to(dev)
        if pooled:
            pool, table, n_pages = wl.pool(w, proj, page_bytes=page_bytes)
            self.pool, self.table = pool.to(dev), table.to(dev)
            self.page_bytes = int(page_bytes or w.page_bytes)
            self.ad = lr.Adapters.paged(self.pool, self.table, self.ranks, self.page_bytes, w.max_rank)
        else:
            A, B = wl.slots(w, proj, pad_value=pad_value)
            self.A, self.B = A.to(dev), B.to(dev)
            self.ad = lr.Adapters.slots(self.A, self.B, self.ranks)
        self.ws = lr.new_workspace(w.M, proj.d, w.k, w.dtype, self.ad, device=dev)

    def run(self, x=None, ids=None, path=lr.PATH_AUTO, flags=0, y=None):
        x = self.x if x is None else x
        ids = self.ids if ids is None else ids
        out = lr.lora_linear(x, self.W, self.ad, ids, self.scales, y=y, workspace=self.ws,
                             path=path, flags=flags)
        torch.cuda.synchronize()
        return out


_ORACLE_CACHE = {}
_ORACLE_CACHE_MAX = 8


def _digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if hasattr(a, "detach"):
            a = a.detach().cpu().contiguous()
            a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
            a = a.numpy()
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def oracle_full(oracle, w, proj, ids=None, x=None):
    """fp64 oracle output for every row, memoised on the exact inputs (a
    digest of x, W, every A and B, the scales and the ids), so the large
    workloads are computed once per session however many tests compare
    against them."""
    ids = w.ids if ids is None else np.asarray(ids, np.int32)
    x = w.x if x is None else x
    key = _digest(x, proj.W, w.scales, ids, np.asarray([w.max_rank]),
                  *[a for a in proj.A], *[b for b in proj.B])
    hit = _ORACLE_CACHE.get(key)
    if hit is None:
        hit = oracle.lora_linear(x, proj.W, proj.A, proj.B, w.scales.astype(np.float64), ids,
                                 max_rank=w.max_rank)
        if len(_ORACLE_CACHE) >= _ORACLE_CACHE_MAX:
            _ORACLE_CACHE.pop(next(iter(_ORACLE_CACHE)))
        _ORACLE_CACHE[key] = hit
    return hit


def oracle_rows(oracle, w, proj, rows=None, ids=None, cache=False):
    """fp64 oracle output for the given rows (all rows when None).  With
    cache=True every row is computed once (oracle_full) and indexed."""
    ids = w.ids if ids is None else ids
    if cache:
        full = oracle_full(oracle, w, proj, ids=ids)
        return full if rows is None else full[np.asarray(rows)]
    if rows is None:
        return oracle.lora_linear(w.x, proj.W, proj.A, proj.B, w.scales.astype(np.float64), ids,
                                  max_rank=w.max_rank)
    rows = np.asarray(rows)
    return oracle.lora_linear(w.x[torch.from_numpy(rows)], proj.W, proj.A, proj.B,
                              w.scales.astype(np.float64), ids[rows], max_rank=w.max_rank)


def assert_covers_present_adapters(w, rows=None) -> None:
    """Every adapter some row uses has at least one row among those compared."""
    ids = np.asarray(w.ids)
    present = set(np.unique(ids[ids >= 0]).tolist())
    seen = present if rows is None else set(np.unique(ids[np.asarray(rows)]).tolist())
    missing = sorted(present - seen)
    assert not missing, "adapters never compared with the oracle: %s" % missing[:20]
