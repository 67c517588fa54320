"""Seeded synthetic inputs for the multi-adapter LoRA linear layer.

This module draws inputs and lays them out; it holds none of the layer's
arithmetic.  Both the HIP path (tests, benchmark) and the fp64 oracle are fed
from it, and it imports neither.

Value recipe: x ~ N(0, 1); W and A ~ N(0, 1/k) (second argument = variance);
B ~ N(0, 0.02) (variance).  Values are drawn in fp32 from
``numpy.random.default_rng(SeedSequence(20261202 + index))`` with spawned child
streams in the order x, W, A, B, structure (ids / lengths / adapters), and
rounded to bf16 by round-to-nearest-even where the workload is bf16.

Named workloads (shapes follow the pages' deployments: a 70B-class model with
hidden size 8192 and Q/V adapters of rank 4/16/64, S-LoRA-style thousands of
adapters in a paged pool, d = k = 4096 with rank 16):

  c0_tiny_fp32     d=k=256, 64 rows, 4 adapters r=8, alpha=16, fp32
  c1_decode_bf16   d=k=4096, 256 rows, 4 adapters r=16, alpha=32
  c2_prefill_bf16  d=k=4096, 8 x 1024 rows, ranks {8,8,16,16,32,32,64,64}, alpha=2r
  c3_proj70b_bf16  k=8192, q d=8192 and v d=1024, 512 rows, 12 adapters
                   ranks {4 x3, 16 x6, 64 x3}, alpha=2r, Zipf(1.1), 51 rows none
  c4_paged_bf16    d=k=5120, 2048 rows from 256 sequences of 1..32 tokens,
                   1024 adapters r=16, alpha=32, Zipf(1.0), 2 MiB pages
  u1_scales        c0 shapes, 5 adapters r={4,8,16,32,64}, alpha=16 fixed
                   (scales 4, 2, 1, 0.5, 0.25 -- catches a wrong-slot scale)
  u2_pages         c0 shapes in a pool of 4 KiB pages (adapters cross pages)
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

BASE_SEED = 20261202
B_VAR = 0.02
BF16_NAN_BITS = 0x7FC0
F32_NAN_BITS = 0x7FC00000


@dataclasses.dataclass
class Projection:
    """One adapted linear: base weight W [d, k] and logical adapters."""
    name: str
    d: int
    W: torch.Tensor                 # [d, k], storage dtype, CPU
    A: List[torch.Tensor]           # A[s]: [r_s, k]
    B: List[torch.Tensor]           # B[s]: [d, r_s]


@dataclasses.dataclass
class Workload:
    name: str
    index: int
    dtype: torch.dtype
    M: int
    k: int
    ranks: np.ndarray               # int32 [S]
    alphas: np.ndarray              # float32 [S]
    scales: np.ndarray              # float32 [S] = alpha / r (true rank)
    max_rank: int
    ids: np.ndarray                 # int32 [M], -1 = none
    x: torch.Tensor                 # [M, k]
    projections: List[Projection]
    seq_lens: Optional[np.ndarray] = None
    page_bytes: Optional[int] = None
    pool_slack: float = 1.25
    notes: str = ""

    @property
    def S(self) -> int:
        return int(self.ranks.size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == torch.float32 else 2

    def proj(self, name: str) -> Projection:
        for p in self.projections:
            if p.name == name:
                return p
        raise KeyError(name)


def _rng_streams(index: int, n: int = 6):
    ss = np.random.SeedSequence(BASE_SEED + index)
    return [np.random.default_rng(c) for c in ss.spawn(n)]


def _to_storage(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).contiguous()


def _normal(rng: np.random.Generator, shape, var: float, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        a *= np.float32(np.sqrt(var))
    return _to_storage(a, dtype)


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Finite Zipf popularity over n items in listed order: p_i ~ (i+1)^-s."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-float(s))
    return w / w.sum()


def _build(name: str, index: int, dtype: torch.dtype, M: int, k: int, proj_dims: Dict[str, int],
           ranks, alphas, max_rank: int, ids_fn, page_bytes: Optional[int] = None,
           seq_lens=None, notes: str = "") -> Workload:
    rx, rw, ra, rb, rs = _rng_streams(index, 5)
    ranks = np.asarray(ranks, np.int32)
    alphas = np.asarray(alphas, np.float32)
    # alpha / r with the true rank; an adapter of rank 0 adds nothing and
    # gets scale 0 (no division by zero)
    scales = np.where(ranks > 0, alphas / np.maximum(ranks, 1).astype(np.float32),
                      np.float32(0)).astype(np.float32)
    ids, seq = ids_fn(rs)
    x = _normal(rx, (M, k), 1.0, dtype)
    projections = []
    for pname, d in proj_dims.items():
        W = _normal(rw, (d, k), 1.0 / k, dtype)
        A = [_normal(ra, (int(r), k), 1.0 / k, dtype) for r in ranks]
        B = [_normal(rb, (d, int(r)), B_VAR, dtype) for r in ranks]
        projections.append(Projection(pname, d, W, A, B))
    return Workload(name, index, dtype, M, k, ranks, alphas, scales, max_rank,
                    np.asarray(ids, np.int32), x, projections,
                    seq_lens=seq if seq is not None else seq_lens, page_bytes=page_bytes,
                    notes=notes)


def _uniform_ids(M: int, S: int):
    def f(rng):
        return rng.integers(-1, S, size=M, dtype=np.int64).astype(np.int32), None
    return f


def c0_tiny_fp32(M: int = 64, d: int = 256, k: int = 256) -> Workload:
    return _build("c0_tiny_fp32", 0, torch.float32, M, k, {"out": d}, [8] * 4, [16.0] * 4, 8,
                  _uniform_ids(M, 4))


def c1_decode_bf16(M: int = 256, d: int = 4096, k: int = 4096) -> Workload:
    return _build("c1_decode_bf16", 1, torch.bfloat16, M, k, {"out": d}, [16] * 4, [32.0] * 4,
                  16, _uniform_ids(M, 4))


def c2_prefill_bf16(n_seq: int = 8, seq_len: int = 1024, d: int = 4096, k: int = 4096) -> Workload:
    ranks = [8, 8, 16, 16, 32, 32, 64, 64][:n_seq] if n_seq <= 8 else None
    M = n_seq * seq_len

    def ids_fn(rng):
        ids = np.repeat(np.arange(n_seq, dtype=np.int32), seq_len)
        return ids, np.full(n_seq, seq_len, np.int64)

    return _build("c2_prefill_bf16", 2, torch.bfloat16, M, k, {"out": d}, ranks,
                  [2.0 * r for r in ranks], 64, ids_fn)


C3_RANKS = [4, 4, 4, 16, 16, 16, 16, 16, 16, 64, 64, 64]


def c3_proj70b_bf16(M: int = 512, k: int = 8192, d_q: int = 8192, d_v: int = 1024,
                    none_frac: float = 0.10, zipf_s: float = 1.1) -> Workload:
    S = len(C3_RANKS)

    def ids_fn(rng):
        n_none = int(round(none_frac * M))
        ids = np.empty(M, np.int32)
        none_rows = rng.choice(M, size=n_none, replace=False)
        mask = np.zeros(M, bool)
        mask[none_rows] = True
        ids[mask] = -1
        ids[~mask] = rng.choice(S, size=M - n_none, p=zipf_probs(S, zipf_s)).astype(np.int32)
        return ids, None

    return _build("c3_proj70b_bf16", 3, torch.bfloat16, M, k, {"q": d_q, "v": d_v}, C3_RANKS,
                  [2.0 * r for r in C3_RANKS], 64, ids_fn,
                  notes="Zipf popularity in listed adapter order; none rows at seeded positions")


def seq_lengths(rng: np.random.Generator, n_seq: int, total: int, max_len: int) -> np.ndarray:
    """Every sequence starts at one token; the remaining tokens go one at a
    time to uniformly chosen sequences still below max_len."""
    lens = np.ones(n_seq, np.int64)
    for _ in range(total - n_seq):
        open_ = np.flatnonzero(lens < max_len)
        lens[open_[rng.integers(0, open_.size)]] += 1
    return lens


def c4_paged_bf16(n_seq: int = 256, total: int = 2048, d: int = 5120, k: int = 5120,
                  n_adapters: int = 1024, page_bytes: int = 2 << 20, zipf_s: float = 1.0) -> Workload:
    def ids_fn(rng):
        lens = seq_lengths(rng, n_seq, total, 32)
        ad = rng.choice(n_adapters, size=n_seq, p=zipf_probs(n_adapters, zipf_s)).astype(np.int32)
        return np.repeat(ad, lens).astype(np.int32), lens

    return _build("c4_paged_bf16", 4, torch.bfloat16, total, k, {"out": d}, [16] * n_adapters,
                  [32.0] * n_adapters, 16, ids_fn, page_bytes=page_bytes,
                  notes="per-sequence Zipf(1.0) adapter; sequences in generation order")


def u1_scales(dtype: torch.dtype = torch.float32, M: int = 64, d: int = 256, k: int = 256) -> Workload:
    ranks = [4, 8, 16, 32, 64]
    return _build("u1_scales", 100, dtype, M, k, {"out": d}, ranks, [16.0] * 5, 64,
                  _uniform_ids(M, 5))


def u2_pages(dtype: torch.dtype = torch.float32, page_bytes: int = 4096, M: int = 64, d: int = 256,
             k: int = 256) -> Workload:
    ranks = [4, 8, 16, 8, 12]
    return _build("u2_pages", 101, dtype, M, k, {"out": d}, ranks, [16.0] * 5, 16,
                  _uniform_ids(M, 5), page_bytes=page_bytes)


def custom(seed: int, M: int, k: int, d: int, ranks, max_rank: int, dtype=torch.bfloat16,
           alphas=None, none_frac: Optional[float] = None, page_bytes: Optional[int] = None,
           sorted_ids: bool = False) -> Workload:
    """Free-form workload for edge cases (ragged sizes, odd ranks, ...)."""
    ranks = list(ranks)
    S = len(ranks)
    if alphas is None:
        alphas = [2.0 * r if r > 0 else 1.0 for r in ranks]

    def ids_fn(rng):
        ids = rng.integers(-1, S, size=M, dtype=np.int64).astype(np.int32)
        if none_frac is not None:
            ids = rng.integers(0, max(S, 1), size=M, dtype=np.int64).astype(np.int32)
            ids[rng.random(M) < none_frac] = -1
        if sorted_ids:
            ids = np.sort(ids)
        return ids, None

    safe = np.asarray([max(r, 1) for r in ranks], np.float32)
    w = _build("custom", 1000 + int(seed), dtype, M, k, {"out": d}, [max(r, 0) for r in ranks],
               alphas, max_rank, ids_fn, page_bytes=page_bytes)
    w.scales = (np.asarray(alphas, np.float32) / safe).astype(np.float32)
    w.page_bytes = page_bytes or 4096
    return w


WORKLOADS = {
    "c0_tiny_fp32": c0_tiny_fp32,
    "c1_decode_bf16": c1_decode_bf16,
    "c2_prefill_bf16": c2_prefill_bf16,
    "c3_proj70b_bf16": c3_proj70b_bf16,
    "c4_paged_bf16": c4_paged_bf16,
    "u1_scales": u1_scales,
    "u2_pages": u2_pages,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)


# ----------------------------------------------------------------------------
# Layouts handed to the library.  These move bytes; they compute nothing.
# ----------------------------------------------------------------------------

def slots(w: Workload, proj: Projection, R: Optional[int] = None, pad_value: float = 0.0):
    """Stacked, rank-padded slots: A_slots [S, R, k], B_slots [S, d, R].

    An adapter whose rank exceeds R (an invalid set, for error tests) keeps
    only its first R rows here."""
    R = w.max_rank if R is None else R
    S, k, d = w.S, w.k, proj.d
    A = torch.full((S, R, k), pad_value, dtype=w.dtype)
    B = torch.full((S, d, R), pad_value, dtype=w.dtype)
    for s in range(S):
        r = min(int(w.ranks[s]), R)
        if r:
            A[s, :r, :] = proj.A[s][:r]
            B[s, :, :r] = proj.B[s][:, :r]
    return A.contiguous(), B.contiguous()


def _storage_bytes(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint8).reshape(-1)
    return t.numpy().view(np.uint8).reshape(-1)


def pool(w: Workload, proj: Projection, page_bytes: Optional[int] = None,
         slack: Optional[float] = None, seed_offset: int = 0):
    """Paged pool: each adapter's logical byte space (A rows, then B rows,
    both unpadded) cut into page_bytes pages placed at seeded physical pages.
    Unused pages hold NaN so a wrong translation shows up in the output.
    Physical pages are a permutation drawn from
    SeedSequence(20261202 + index + 7919 * (seed_offset + 1)).

    Returns (pool uint8 [n_pages * page_bytes], page_table int32 [S, max_pages], n_pages)."""
    P = int(page_bytes or w.page_bytes)
    slack = w.pool_slack if slack is None else slack
    eb = w.elem_bytes
    blobs = []
    for s in range(w.S):
        blobs.append(np.concatenate([_storage_bytes(proj.A[s]), _storage_bytes(proj.B[s])])
                     if w.ranks[s] else np.zeros(0, np.uint8))
    pages_of = [(b.size + P - 1) // P for b in blobs]
    max_pages = max(max(pages_of), 1)
    need = int(sum(pages_of))
    n_pages = max(int(np.ceil(need * slack)), need, 1)
    rng = np.random.default_rng(np.random.SeedSequence(BASE_SEED + w.index + 7919 * (seed_offset + 1)))
    phys = rng.permutation(n_pages)
    buf = np.empty(n_pages * P, np.uint8)
    nan = np.array([BF16_NAN_BITS if eb == 2 else F32_NAN_BITS],
                   np.uint16 if eb == 2 else np.uint32).view(np.uint8)
    buf.reshape(-1, eb)[:] = nan
    table = np.full((w.S, max_pages), -1, np.int32)
    nxt = 0
    for s, b in enumerate(blobs):
        for j in range(pages_of[s]):
            p = int(phys[nxt])
            nxt += 1
            table[s, j] = p
            chunk = b[j * P:(j + 1) * P]
            buf[p * P:p * P + chunk.size] = chunk
    return torch.from_numpy(buf), torch.from_numpy(table), n_pages


def algorithmic_bytes(w: Workload, proj: Projection) -> Dict[str, float]:
    """Bytes and flops the layer must move or do on this instance: real
    ranks, each present adapter's A and B once, x once, adapted y rows read
    and written once, t in fp32."""
    e = w.elem_bytes
    ids = w.ids
    valid = ids >= 0
    Ma = int(valid.sum())
    present = np.unique(ids[valid])
    r_rows = int(w.ranks[ids[valid]].sum()) if Ma else 0
    r_present = int(w.ranks[present].sum()) if present.size else 0
    k, d, M = w.k, proj.d, w.M
    return {
        "M": M, "M_a": Ma, "n_present": int(present.size),
        "shrink_bytes": Ma * k * e + r_present * k * e + r_rows * 4,
        "shrink_flops": 2.0 * k * r_rows,
        "expand_bytes": r_present * d * e + r_rows * 4 + 2 * Ma * d * e,
        "expand_flops": 2.0 * d * r_rows,
        "gemm_flops": 2.0 * M * d * k,
        "gemm_bytes": (M * k + d * k + M * d) * e,
    }


def quantized_base(w: Workload, fmt: str, group: int = 128, names=None):
    """Seeded quantized base weights for the workload's projections, stacked
    by rows in `names` order (default: all).  Symmetric formats:
      int8: q uniform in [-127, 127], one scale per row;
      int4: q uniform in [-8, 7], two per byte (element 2i in the low nibble),
            one scale per row and k-group.
    Scales are sqrt(3 / k) / qmax times U(0.5, 1.5), so the weights have
    about the variance 1/k of the bf16 workloads.  Draws come from
    SeedSequence(20261202 + index + 104729); nothing is computed from the
    bf16 weights.  Returns (q uint8 [d, ldq], scales float32: [d] for int8,
    [d, k / group] for int4)."""
    names = [p.name for p in w.projections] if names is None else list(names)
    d = sum(w.proj(n).d for n in names)
    k = w.k
    rng = np.random.default_rng(np.random.SeedSequence(BASE_SEED + w.index + 104729))
    if fmt == "int8":
        q = rng.integers(-127, 128, size=(d, k), dtype=np.int64).astype(np.int8)
        s = (np.sqrt(3.0 / k) / 127.0 * rng.uniform(0.5, 1.5, size=d)).astype(np.float32)
        return torch.from_numpy(q.view(np.uint8).copy()), torch.from_numpy(s)
    if fmt == "int4":
        if k % group or group % 64:
            raise ValueError("group must be a multiple of 64 dividing k")
        v = rng.integers(-8, 8, size=(d, k), dtype=np.int64)
        u = (v & 0xF).astype(np.uint8)
        packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
        s = (np.sqrt(3.0 / k) / 8.0 * rng.uniform(0.5, 1.5, size=(d, k // group))).astype(np.float32)
        return torch.from_numpy(packed), torch.from_numpy(s)
    raise ValueError(fmt)
