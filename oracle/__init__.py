"""fp64 CPU oracle for the multi-adapter LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (``lora_row_adapter_amd``) and never imports it; the product
path never imports this package.

The arithmetic lives in ``lora_oracle.c`` (plain fp64 loops, gcc, OpenMP over
rows only).  This module builds it, loads it with ctypes and converts numpy or
torch inputs to the contiguous fp64 / int32 arrays it reads.  Function-level
citations are in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")

ROW_ADAPTED, ROW_NONE, ROW_BAD_ID, ROW_BAD_RANK, ROW_BAD_PAGE = 0, 1, 2, 3, 4

_lib = None


def build(force: bool = True, out: str | None = None, mutant: int = 0,
          sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp -ffp-contract=off).

    ``mutant`` > 0 builds a copy with one planted mistake (pin tests only);
    ``sanitize`` builds it under AddressSanitizer and UndefinedBehaviorSanitizer
    (the loading process preloads gcc's libasan)."""
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer", "-g"] if sanitize else [])
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c99", "-Wall", "-Werror", "-DORACLE_MUTANT=%d" % int(mutant)] + san + [
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def use_library(path: str | None) -> None:
    """Point this module at another build of the oracle (pin tests use it to
    load a mutant); None returns to the normal build."""
    global _lib, _lib_path
    _lib = None
    _lib_path = path or _LIB


_lib_path = _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_lib_path):
        build(out=_lib_path)
    lib = ctypes.CDLL(_lib_path)
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_adapter_params.argtypes = [i64, i64, i64]
    lib.oracle_adapter_params.restype = i64
    lib.oracle_adapter_offset.argtypes = [i64, i64, i64, i32, i64, i64]
    lib.oracle_adapter_offset.restype = i64
    lib.oracle_translate.argtypes = [p, i32, i64, i64, p, p, i64, p]
    lib.oracle_translate.restype = i64
    lib.oracle_plan.argtypes = [i64, p, i32, p, i32, p, i32, i64, i64, i64, i64, i64,
                                p, p, p, p, p, p, p]
    lib.oracle_plan.restype = i64
    lib.oracle_lora_linear.argtypes = [i64, i64, i64, p, p, i32, p, i32, p, p, p, p, p, p,
                                       p, i32]
    lib.oracle_lora_linear.restype = None
    lib.oracle_merge.argtypes = [i64, i64, i64, p, p, p, ctypes.c_double, ctypes.c_double, p, i32]
    lib.oracle_merge.restype = None
    lib.oracle_threads.argtypes = [i32]
    lib.oracle_threads.restype = i32
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: exact upcast of the stored values
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def threads_used(n: int) -> int:
    return int(_load().oracle_threads(int(n)))


def adapter_params(d: int, k: int, r: int) -> int:
    return int(_load().oracle_adapter_params(d, k, r))


def adapter_offset(r: int, k: int, elem_bytes: int, which: str, row: int, col: int) -> int:
    return int(_load().oracle_adapter_offset(r, k, elem_bytes, 0 if which == "A" else 1, row, col))


def translate(page_table, page_bytes: int, n_pages: int, adapter, logical_off):
    """Logical byte offsets -> physical pool byte offsets (-1 when invalid)."""
    pt = _i32(page_table)
    if pt.ndim != 2:
        raise ValueError("page_table must be [n_adapters, max_pages]")
    a = _i32(adapter).reshape(-1)
    off = np.ascontiguousarray(np.asarray(logical_off, dtype=np.int64).reshape(-1))
    if a.shape != off.shape:
        raise ValueError("adapter and logical_off differ in length")
    out = np.empty_like(off)
    _load().oracle_translate(_ptr(pt), pt.shape[1], int(page_bytes), int(n_pages), _ptr(a),
                             _ptr(off), off.size, _ptr(out))
    return out


def plan(ids, n_adapters: int, ranks, max_rank: int, page_table=None, n_pages: int = 0,
         page_bytes: int = 0, k: int = 0, d: int = 0, elem_bytes: int = 2) -> dict:
    """Row classes, stable adapter-sorted permutation and segment table."""
    ids_ = _i32(ids).reshape(-1)
    rk = _i32(ranks).reshape(-1)
    if rk.size != n_adapters:
        raise ValueError("ranks must have n_adapters entries")
    M = ids_.size
    row_class = np.empty(M, np.int32)
    perm = np.empty(max(M, 1), np.int32)
    nseg_cap = max(min(M, n_adapters), 1)
    seg_a = np.empty(nseg_cap, np.int32)
    seg_s = np.empty(nseg_cap, np.int32)
    seg_l = np.empty(nseg_cap, np.int32)
    n_seg = np.zeros(1, np.int64)
    counts = np.zeros(3, np.int64)
    if page_table is not None:
        pt = _i32(page_table)
        pt_ptr, max_pages = _ptr(pt), pt.shape[1]
    else:
        pt, pt_ptr, max_pages = None, None, 0
    n_ad = _load().oracle_plan(M, _ptr(ids_), int(n_adapters), _ptr(rk), int(max_rank), pt_ptr,
                               int(max_pages), int(n_pages), int(page_bytes), int(k), int(d),
                               int(elem_bytes), _ptr(row_class), _ptr(perm), _ptr(seg_a),
                               _ptr(seg_s), _ptr(seg_l), _ptr(n_seg), _ptr(counts))
    ns = int(n_seg[0])
    return {
        "row_class": row_class,
        "perm": perm[:n_ad].copy(),
        "n_adapted": int(n_ad),
        "seg_adapter": seg_a[:ns].copy(),
        "seg_start": seg_s[:ns].copy(),
        "seg_len": seg_l[:ns].copy(),
        "n_bad_ids": int(counts[0]),
        "n_bad_ranks": int(counts[1]),
        "n_bad_pages": int(counts[2]),
    }


def lora_linear(x, W, A_list, B_list, scales, ids, max_rank: int | None = None,
                n_threads: int | None = None) -> np.ndarray:
    """y = x W^T + scale_s (x A_s^T) B_s^T per row (fp64).

    A_list[s] is r_s x k and B_list[s] is d x r_s (logical, unpadded); ids[m]
    = -1 selects no adapter."""
    x64, W64 = _f64(x), _f64(W)
    if x64.ndim != 2 or W64.ndim != 2 or x64.shape[1] != W64.shape[1]:
        raise ValueError("x must be [M,k] and W [d,k]")
    M, k = x64.shape
    d = W64.shape[0]
    S = len(A_list)
    if len(B_list) != S:
        raise ValueError("A_list and B_list differ in length")
    ranks = np.zeros(max(S, 1), np.int32)
    a_parts, b_parts, a_off, b_off = [], [], np.zeros(max(S, 1), np.int64), np.zeros(max(S, 1), np.int64)
    ao = bo = 0
    for s in range(S):
        a = _f64(A_list[s])
        b = _f64(B_list[s])
        r = a.shape[0]
        if a.shape != (r, k) or b.shape != (d, r):
            raise ValueError("adapter %d has A %s, B %s; expected (r,%d), (%d,r)" % (s, a.shape, b.shape, k, d))
        ranks[s] = r
        a_off[s], b_off[s] = ao, bo
        a_parts.append(a.reshape(-1))
        b_parts.append(b.reshape(-1))
        ao += a.size
        bo += b.size
    A = np.ascontiguousarray(np.concatenate(a_parts)) if a_parts and ao else np.zeros(1)
    B = np.ascontiguousarray(np.concatenate(b_parts)) if b_parts and bo else np.zeros(1)
    sc = _f64(scales).reshape(-1) if S else np.zeros(1)
    ids_ = _i32(ids).reshape(-1)
    if ids_.size != M:
        raise ValueError("ids must have M entries")
    if max_rank is None:
        max_rank = int(ranks.max()) if S else 0
    y = np.empty((M, d), np.float64)
    nt = default_threads() if n_threads is None else int(n_threads)
    _load().oracle_lora_linear(M, k, d, _ptr(x64), _ptr(W64), S, _ptr(ranks), int(max_rank),
                               _ptr(a_off), _ptr(b_off), _ptr(A), _ptr(B), _ptr(sc), _ptr(ids_),
                               _ptr(y), nt)
    return y


def merge(W, A, B, scale: float, coef: float = 1.0, n_threads: int | None = None) -> np.ndarray:
    """W + coef * scale * B A in fp64 (W [d,k], A [r,k], B [d,r])."""
    W64, A64, B64 = _f64(W), _f64(A), _f64(B)
    d, k = W64.shape
    r = A64.shape[0] if A64.ndim == 2 else 0
    if A64.shape != (r, k) or B64.shape != (d, r):
        raise ValueError("A must be [r,%d] and B [%d,r]" % (k, d))
    if r == 0:
        A64, B64 = np.zeros(1), np.zeros(1)
    out = np.empty((d, k), np.float64)
    nt = default_threads() if n_threads is None else int(n_threads)
    _load().oracle_merge(d, k, r, _ptr(W64), _ptr(np.ascontiguousarray(A64)),
                         _ptr(np.ascontiguousarray(B64)), float(scale), float(coef), _ptr(out), nt)
    return out


def dequant_int8(q, scales) -> np.ndarray:
    """W[n, j] = scales[n] * q[n, j] in fp64 (q int8 [d, k], scales [d]).

    "Your LoRA Adapters Are Thrashing Your GPUs", section 02: an INT8 base
    weight; the symmetric per-output-row reading."""
    q = np.asarray(q)
    if q.dtype != np.int8:
        q = q.view(np.int8) if q.dtype == np.uint8 else q.astype(np.int8)
    s = np.asarray(scales, np.float64).reshape(-1)
    if s.size != q.shape[0]:
        raise ValueError("one scale per row")
    return q.astype(np.float64) * s[:, None]


def unpack_int4(packed, k: int) -> np.ndarray:
    """Signed 4-bit values of a packed row-major [d, >= k/2] byte array:
    element 2i of a row is the low nibble of byte i, element 2i + 1 the high
    nibble, both two's complement (-8 .. 7).  Returns int8 [d, k]."""
    b = np.asarray(packed).astype(np.uint8)[:, : k // 2]
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((b.shape[0], k), np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_int4(packed, scales, group: int, k: int) -> np.ndarray:
    """W[n, j] = scales[n, j // group] * q[n, j] in fp64.

    "Your LoRA Adapters Are Thrashing Your GPUs", section 02: an INT4 base
    weight; the symmetric reading with one scale per row and k-group."""
    q = unpack_int4(packed, k).astype(np.float64)
    s = np.asarray(scales, np.float64).reshape(q.shape[0], k // group)
    return q * np.repeat(s, group, axis=1)
