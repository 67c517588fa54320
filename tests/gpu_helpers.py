"""Glue for the GPU tests: move seeded workloads to the device, call the
library through its binding, and compare with the oracle."""
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


def oracle_rows(oracle, w, proj, rows=None, ids=None):
    """fp64 oracle output for the given rows (all rows when None)."""
    ids = w.ids if ids is None else ids
    if rows is None:
        return oracle.lora_linear(w.x, proj.W, proj.A, proj.B, w.scales.astype(np.float64), ids,
                                  max_rank=w.max_rank)
    rows = np.asarray(rows)
    return oracle.lora_linear(w.x[torch.from_numpy(rows)], proj.W, proj.A, proj.B,
                              w.scales.astype(np.float64), ids[rows], max_rank=w.max_rank)


def sample_rows(w, n: int, seed: int = 0) -> np.ndarray:
    """Rows to check at full size: both ends, every segment boundary region,
    none rows, and a seeded random remainder."""
    rng = np.random.default_rng(seed)
    M = w.M
    pick = {0, M - 1, M // 2}
    none = np.flatnonzero(w.ids < 0)
    pick.update(none[:4].tolist())
    change = np.flatnonzero(np.diff(w.ids) != 0)
    pick.update(change[:8].tolist())
    pick.update((change[:8] + 1).tolist())
    while len(pick) < min(n, M):
        pick.add(int(rng.integers(0, M)))
    return np.array(sorted(pick), dtype=np.int64)
