"""ctypes binding of liblora_row.so (declared in include/lora_row.h).

Argument marshalling only: torch tensors are checked for device, dtype and
layout, and their device pointers, leading dimensions and the current HIP
stream are handed to the C entry points of the same names.  Every step of
the layer runs in the library's HIP kernels.  If the library is missing the
call raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "liblora_row.so"

PATH_AUTO, PATH_GATHER, PATH_SGMV = 0, 1, 2
FLAG_REUSE_PLAN = 1
FLAG_SEPARATE_SHRINK = 2
KIND_SLOTS, KIND_POOL = 0, 1
PLAN_MAX_ROWS = 8192
KERNEL_CLASSES = ("plan", "gemm", "shrink", "expand", "sgmv_shrink", "sgmv_expand")

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class LoraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_str(status), status))


class _CAdapters(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("n_adapters", ctypes.c_int32),
        ("max_rank", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("ranks", ctypes.c_void_p),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("pool", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_bytes", ctypes.c_int64),
        ("n_pages", ctypes.c_int64),
    ]


class _CSlice(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int64),
        ("scales", ctypes.c_void_p),
        ("adapters", _CAdapters),
    ]


class _CPlanView(ctypes.Structure):
    _fields_ = [
        ("counters", ctypes.c_void_p),
        ("perm", ctypes.c_void_p),
        ("seg_adapter", ctypes.c_void_p),
        ("seg_start", ctypes.c_void_p),
        ("seg_len", ctypes.c_void_p),
        ("capacity_rows", ctypes.c_int64),
    ]


class _CProfile(ctypes.Structure):
    _fields_ = [
        ("ms", ctypes.c_double * 6),
        ("launches", ctypes.c_int64 * 6),
        ("dropped", ctypes.c_int64),
    ]


class _CQWeight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("ldq", ctypes.c_int64),
        ("scales", ctypes.c_void_p),
    ]


class _CPoolDesc(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("ranks", ctypes.c_void_p),
        ("n_pages", ctypes.c_int64),
        ("page_bytes", ctypes.c_int64),
        ("n_adapters", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("max_rank", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("k", ctypes.c_int64),
        ("d", ctypes.c_int64),
    ]


class _CPoolStats(ctypes.Structure):
    _fields_ = [
        ("loads", ctypes.c_int64),
        ("evictions", ctypes.c_int64),
        ("bytes_copied", ctypes.c_int64),
        ("free_pages", ctypes.c_int64),
        ("resident", ctypes.c_int64),
    ]


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                           " (the HIP path has no fallback)" % path)
    lib = ctypes.CDLL(path)
    i32, i64, u32, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t
    pad = ctypes.POINTER(_CAdapters)
    lib.lora_abi_version.argtypes = []
    lib.lora_abi_version.restype = i32
    lib.lora_status_str.argtypes = [i32]
    lib.lora_status_str.restype = ctypes.c_char_p
    lib.lora_workspace_bytes.argtypes = [i64, i64, i64, i32, pad]
    lib.lora_workspace_bytes.restype = sz
    lib.lora_gemm.argtypes = [i32, i64, i64, i64, p, i64, p, i64, p, i64, p, sz, p]
    lib.lora_gemm.restype = i32
    lib.lora_gemm_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.lora_gemm_workspace_bytes.restype = sz
    lib.lora_linear.argtypes = [i32, i64, i64, i64, p, i64, p, i64, pad, p, p, p, i64, p, sz, i32,
                                u32, p]
    lib.lora_linear.restype = i32
    psl = ctypes.POINTER(_CSlice)
    lib.lora_workspace_bytes_sliced.argtypes = [i64, i64, i32, i32, psl]
    lib.lora_workspace_bytes_sliced.restype = sz
    lib.lora_linear_sliced.argtypes = [i32, i64, i64, p, i64, p, i64, i32, psl, p, p, i64, p, sz,
                                       i32, u32, p]
    lib.lora_linear_sliced.restype = i32
    lib.lora_linear_sliced_noalloc.argtypes = [i32, i64, i64, p, i64, p, i64, i32, psl, p, p, i64,
                                               i32, u32, p]
    lib.lora_linear_sliced_noalloc.restype = i32
    lib.lora_plan.argtypes = [i64, i64, i64, i32, pad, p, p, sz, p]
    lib.lora_plan.restype = i32
    lib.lora_plan_view.argtypes = [p, sz, i64, pad, ctypes.POINTER(_CPlanView)]
    lib.lora_plan_view.restype = i32
    pqw = ctypes.POINTER(_CQWeight)
    lib.lora_gemm_q.argtypes = [i64, i64, i64, p, i64, pqw, p, i64, p]
    lib.lora_gemm_q.restype = i32
    lib.lora_linear_sliced_q.argtypes = [i64, i64, p, i64, pqw, i32, ctypes.POINTER(_CSlice), p, p,
                                         i64, p, sz, i32, u32, p]
    lib.lora_linear_sliced_q.restype = i32
    lib.lora_merge.argtypes = [i32, i64, i64, p, i64, pad, i32, p, ctypes.c_float, p, i64, p]
    lib.lora_merge.restype = i32
    lib.lora_translate.argtypes = [pad, p, p, i64, p, p]
    lib.lora_translate.restype = i32
    lib.lora_check.argtypes = [p, p, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64),
                               ctypes.POINTER(i64)]
    lib.lora_check.restype = i32
    lib.lora_test_sync_spin_limit.argtypes = [i32]
    lib.lora_test_sync_spin_limit.restype = i32
    lib.lora_profile_enable.argtypes = [i32]
    lib.lora_profile_enable.restype = i32
    lib.lora_profile_read.argtypes = [ctypes.POINTER(_CProfile), i32]
    lib.lora_profile_read.restype = i32
    pi32 = ctypes.POINTER(i32)
    lib.lora_pool_create.argtypes = [ctypes.POINTER(_CPoolDesc), p, ctypes.POINTER(p)]
    lib.lora_pool_create.restype = i32
    lib.lora_pool_destroy.argtypes = [p]
    lib.lora_pool_destroy.restype = None
    lib.lora_pool_adapters.argtypes = [p, pad]
    lib.lora_pool_adapters.restype = i32
    lib.lora_pool_load.argtypes = [p, i32, i32, p, p, p]
    lib.lora_pool_load.restype = i32
    lib.lora_pool_load_batch.argtypes = [p, i32, pi32, pi32, ctypes.POINTER(p), ctypes.POINTER(p), p]
    lib.lora_pool_load_batch.restype = i32
    lib.lora_pool_evict.argtypes = [p, i32, p]
    lib.lora_pool_evict.restype = i32
    for name in ("lora_pool_touch", "lora_pool_pin", "lora_pool_unpin"):
        getattr(lib, name).argtypes = [p, pi32, i32]
        getattr(lib, name).restype = i32
    lib.lora_pool_query.argtypes = [p, i32, pi32, pi32, pi32, pi32, pi32]
    lib.lora_pool_query.restype = i32
    lib.lora_pool_get_stats.argtypes = [p, ctypes.POINTER(_CPoolStats)]
    lib.lora_pool_get_stats.restype = i32
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().lora_abi_version())


def status_str(status: int) -> str:
    try:
        return load_library().lora_status_str(int(status)).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "status %d" % status


def _check(status: int, what: str) -> None:
    if status != 0:
        raise LoraError(status, what)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)
    return _DTYPES[t.dtype]


def _rows(t: torch.Tensor, name: str):
    """(pointer, leading dimension) of a row-major 2-D device tensor."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.stride(1) != 1:
        raise ValueError("%s must have unit stride along its last dimension" % name)
    return t.data_ptr(), t.stride(0)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))
    return t.data_ptr()


class Adapters:
    """An adapter set: stacked rank-padded slots or a paged pool.

    Holds references to the device tensors so they outlive the descriptor."""

    def __init__(self, kind: int, ranks: torch.Tensor, max_rank: int, A=None, B=None, pool=None,
                 page_table=None, page_bytes: int = 0, n_pages: int = 0):
        self.kind = kind
        self.ranks = ranks
        self.max_rank = int(max_rank)
        self.A, self.B, self.pool, self.page_table = A, B, pool, page_table
        self.page_bytes = int(page_bytes)
        self.n_pages = int(n_pages)
        self.n_adapters = int(ranks.numel())
        c = _CAdapters()
        c.kind = kind
        c.n_adapters = self.n_adapters
        c.max_rank = self.max_rank
        c.ranks = _dev(ranks, "ranks", torch.int32)
        if kind == KIND_SLOTS:
            c.A = _dev(A, "A")
            c.B = _dev(B, "B")
        else:
            if page_table.dim() != 2 or page_table.shape[0] != self.n_adapters:
                raise ValueError("page_table must be [n_adapters, max_pages]")
            c.pool = _dev(pool, "pool")
            c.page_table = _dev(page_table, "page_table", torch.int32)
            c.max_pages = int(page_table.shape[1])
            c.page_bytes = self.page_bytes
            c.n_pages = self.n_pages
        self._c = c

    @classmethod
    def slots(cls, A: torch.Tensor, B: torch.Tensor, ranks: torch.Tensor) -> "Adapters":
        """A [S, R, k], B [S, d, R], ranks int32 [S] (device)."""
        if A.dim() != 3 or B.dim() != 3 or A.shape[0] != B.shape[0] or A.shape[1] != B.shape[2]:
            raise ValueError("slots must be A [S, R, k] and B [S, d, R]")
        if A.dtype != B.dtype:
            raise TypeError("A and B differ in dtype")
        return cls(KIND_SLOTS, ranks, A.shape[1], A=A, B=B)

    @classmethod
    def paged(cls, pool: torch.Tensor, page_table: torch.Tensor, ranks: torch.Tensor,
              page_bytes: int, max_rank: int) -> "Adapters":
        """pool: device bytes [n_pages * page_bytes]; page_table int32 [S, max_pages]."""
        if pool.numel() * pool.element_size() % page_bytes:
            raise ValueError("pool size is not a whole number of pages")
        n_pages = pool.numel() * pool.element_size() // page_bytes
        return cls(KIND_POOL, ranks, max_rank, pool=pool, page_table=page_table,
                   page_bytes=page_bytes, n_pages=n_pages)

    def ref(self):
        return ctypes.byref(self._c)


class AdapterPool:
    """Adapter activation into a paged device pool (include/lora_pool.h).

    With ``device`` set, the pool bytes, page table and ranks are allocated
    here as torch tensors and handed to the manager; ``adapters()`` is the
    POOL adapter set lora_linear reads.  With ``device=None`` the manager
    runs in accounting-only mode (placement, LRU and pinning decisions with
    no device memory)."""

    def __init__(self, n_pages: int, page_bytes: int, n_adapters: int, max_pages: int,
                 max_rank: int, k: int, d: int, dtype: torch.dtype = torch.bfloat16,
                 device=None, stream=None):
        lib = load_library()
        self.dtype = dtype
        self.k, self.d = int(k), int(d)
        self.max_pages = int(max_pages)
        self.page_bytes = int(page_bytes)
        c = _CPoolDesc()
        c.n_pages, c.page_bytes = int(n_pages), self.page_bytes
        c.n_adapters, c.max_pages, c.max_rank = int(n_adapters), self.max_pages, int(max_rank)
        c.elem_bytes = torch.empty((), dtype=dtype).element_size()
        c.k, c.d = self.k, self.d
        self.pool = self.page_table = self.ranks = None
        if device is not None:
            self.pool = torch.empty(int(n_pages) * self.page_bytes, dtype=torch.uint8, device=device)
            self.page_table = torch.empty((int(n_adapters), self.max_pages), dtype=torch.int32,
                                          device=device)
            self.ranks = torch.empty(int(n_adapters), dtype=torch.int32, device=device)
            c.pool = self.pool.data_ptr()
            c.page_table = self.page_table.data_ptr()
            c.ranks = self.ranks.data_ptr()
        self._desc = c
        self._inflight = []  # (event, host A, host B) of pinned loads not yet reached
        h = ctypes.c_void_p()
        st = _stream_ptr(stream) if device is not None else 0
        _check(lib.lora_pool_create(ctypes.byref(c), st, ctypes.byref(h)), "lora_pool_create")
        self._h = h

    def __del__(self):
        for ev, _ in getattr(self, "_inflight", []):
            try:
                ev.synchronize()
            except Exception:  # pragma: no cover - interpreter shutdown
                pass
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.lora_pool_destroy(h)
            self._h = None

    def _stream(self, stream) -> int:
        return _stream_ptr(stream) if self.pool is not None else 0

    def adapters(self) -> Adapters:
        """The POOL adapter set over this manager's device tensors."""
        if self.pool is None:
            raise ValueError("an accounting-only pool has no device adapter set")
        return Adapters.paged(self.pool, self.page_table, self.ranks, self.page_bytes,
                              self._desc.max_rank)

    def _weights(self, A, B, rank):
        """(rank, A pointer, B pointer) after checking the host tensors."""
        if A is None:
            if rank is None:
                raise ValueError("rank is needed when no weights are given")
            return int(rank), 0, 0
        if A.is_cuda or B.is_cuda:
            raise ValueError("A and B are host tensors")
        if A.dtype != self.dtype or B.dtype != self.dtype:
            raise TypeError("A and B must be %s" % self.dtype)
        if A.dim() != 2 or B.dim() != 2 or A.shape[1] != self.k or B.shape[0] != self.d \
                or B.shape[1] != A.shape[0]:
            raise ValueError("A must be [r, %d] and B [%d, r]" % (self.k, self.d))
        if not (A.is_contiguous() and B.is_contiguous()):
            raise ValueError("A and B must be contiguous")
        return int(A.shape[0] if rank is None else rank), A.data_ptr(), B.data_ptr()

    def _keep_alive(self, tensors, stream):
        # Pinned sources are read by the device after the call returns: keep
        # the tensors alive until the stream has passed the copy (torch's
        # pinned-memory cache would otherwise hand the block to the next
        # pin_memory() call).
        pinned = [t for t in tensors if t is not None and t.is_pinned()]
        if pinned and self.pool is not None:
            ev = torch.cuda.Event()
            ev.record(stream if stream is not None else torch.cuda.current_stream())
            self._inflight.append((ev, pinned))

    def load(self, adapter: int, A: Optional[torch.Tensor], B: Optional[torch.Tensor],
             rank: Optional[int] = None, stream=None) -> None:
        """Make ``adapter`` resident: A [r, k] and B [d, r], host tensors in
        the pool's dtype (pinned ones are read by the device asynchronously)."""
        r, pa, pb = self._weights(A, B, rank)
        self._inflight = [e for e in self._inflight if not e[0].query()]
        _check(_lib.lora_pool_load(self._h, int(adapter), r, pa, pb, self._stream(stream)),
               "lora_pool_load")
        self._keep_alive([A, B], stream)

    def load_batch(self, items, stream=None) -> None:
        """Several loads in one call (all or nothing).  items: (adapter, A, B)
        or (adapter, None, None, rank) tuples."""
        n = len(items)
        ids = (ctypes.c_int32 * n)()
        ranks = (ctypes.c_int32 * n)()
        pa = (ctypes.c_void_p * n)()
        pb = (ctypes.c_void_p * n)()
        keep = []
        for i, it in enumerate(items):
            A, B = it[1], it[2]
            r, a_ptr, b_ptr = self._weights(A, B, it[3] if len(it) > 3 else None)
            ids[i], ranks[i], pa[i], pb[i] = int(it[0]), r, a_ptr, b_ptr
            keep += [A, B]
        self._inflight = [e for e in self._inflight if not e[0].query()]
        _check(_lib.lora_pool_load_batch(self._h, n, ids, ranks, pa, pb, self._stream(stream)),
               "lora_pool_load_batch")
        self._keep_alive(keep, stream)

    def evict(self, adapter: int, stream=None) -> None:
        _check(_lib.lora_pool_evict(self._h, int(adapter), self._stream(stream)), "lora_pool_evict")

    def _ids(self, fn, ids, what):
        arr = (ctypes.c_int32 * len(ids))(*[int(i) for i in ids])
        _check(fn(self._h, arr, len(ids)), what)

    def touch(self, ids) -> None:
        self._ids(_lib.lora_pool_touch, ids, "lora_pool_touch")

    def pin(self, ids) -> None:
        self._ids(_lib.lora_pool_pin, ids, "lora_pool_pin")

    def unpin(self, ids) -> None:
        self._ids(_lib.lora_pool_unpin, ids, "lora_pool_unpin")

    def query(self, adapter: int) -> dict:
        res, rank, pins, npg = (ctypes.c_int32() for _ in range(4))
        pages = (ctypes.c_int32 * self.max_pages)()
        _check(_lib.lora_pool_query(self._h, int(adapter), ctypes.byref(res), ctypes.byref(rank),
                                    ctypes.byref(pins), ctypes.byref(npg), pages), "lora_pool_query")
        return {"resident": bool(res.value), "rank": rank.value, "pins": pins.value,
                "n_pages": npg.value, "pages": list(pages)[:npg.value]}

    def stats(self) -> dict:
        st = _CPoolStats()
        _check(_lib.lora_pool_get_stats(self._h, ctypes.byref(st)), "lora_pool_get_stats")
        return {name: getattr(st, name) for name, _ in _CPoolStats._fields_}


class Slice:
    """One projection of a multi-slice call: width d, its adapter set and
    its per-adapter scales (device fp32 [n_adapters])."""

    def __init__(self, d: int, adapters: Adapters, scales: torch.Tensor):
        self.d = int(d)
        self.adapters = adapters
        self.scales = scales

    def c(self) -> _CSlice:
        c = _CSlice()
        c.d = self.d
        c.scales = _dev(self.scales, "scales", torch.float32)
        c.adapters = self.adapters._c
        return c


def _slice_array(slices):
    arr = (_CSlice * len(slices))()
    for i, sl in enumerate(slices):
        arr[i] = sl.c()
    return arr


def workspace_bytes_sliced(max_rows: int, k: int, dtype: torch.dtype, slices) -> int:
    arr = _slice_array(slices)
    n = load_library().lora_workspace_bytes_sliced(int(max_rows), int(k), _DTYPES[dtype], len(slices), arr)
    if n == 0:
        raise LoraError(1, "lora_workspace_bytes_sliced")
    return int(n)


def workspace_bytes(max_rows: int, d: int, k: int, dtype: torch.dtype, adapters: Adapters) -> int:
    n = load_library().lora_workspace_bytes(int(max_rows), int(d), int(k), _DTYPES[dtype], adapters.ref())
    if n == 0:
        raise LoraError(1, "lora_workspace_bytes")
    return int(n)


def new_workspace(max_rows: int, d: int, k: int, dtype: torch.dtype, adapters: Adapters,
                  device=None) -> torch.Tensor:
    n = workspace_bytes(max_rows, d, k, dtype, adapters)
    # zero-filled once: the library's sticky error words start at 0
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def gemm_workspace_bytes(M: int, k: int, d: int, dtype: torch.dtype) -> int:
    """Workspace bytes lora_gemm uses for this shape (0: none needed)."""
    return int(load_library().lora_gemm_workspace_bytes(int(M), int(k), int(d), _DTYPES[dtype]))


def lora_gemm(x: torch.Tensor, W: torch.Tensor, y: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = x W^T on the device (base projection only).  Without a workspace
    one of lora_gemm_workspace_bytes bytes is allocated (torch) for the call."""
    lib = load_library()
    if y is None:
        y = torch.empty((x.shape[0], W.shape[0]), dtype=x.dtype, device=x.device)
    xp, ldx = _rows(x, "x")
    wp, ldw = _rows(W, "W")
    yp, ldy = _rows(y, "y")
    if W.dtype != x.dtype or y.dtype != x.dtype:
        raise TypeError("x, W, y must share a dtype")
    if workspace is None:
        n = gemm_workspace_bytes(x.shape[0], x.shape[1], W.shape[0], x.dtype)
        if n > 0:
            workspace = torch.zeros(n, dtype=torch.uint8, device=x.device)
    wsp, wsn = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib.lora_gemm(_dtype_code(x), x.shape[0], x.shape[1], W.shape[0], xp, ldx, wp, ldw,
                         yp, ldy, wsp, wsn, _stream_ptr(stream)), "lora_gemm")
    return y


def lora_linear(x: torch.Tensor, W: torch.Tensor, adapters: Adapters, adapter_ids: torch.Tensor,
                scales: torch.Tensor, y: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, path: int = PATH_AUTO, flags: int = 0,
                stream=None) -> torch.Tensor:
    """y = x W^T + scale_s (x A_s^T) B_s^T per row (s = adapter_ids[m], -1 = none)."""
    lib = load_library()
    M, k = x.shape
    d = W.shape[0]
    if y is None:
        y = torch.empty((M, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, d, k, x.dtype, adapters, device=x.device)
    xp, ldx = _rows(x, "x")
    wp, ldw = _rows(W, "W")
    yp, ldy = _rows(y, "y")
    if W.dtype != x.dtype or y.dtype != x.dtype:
        raise TypeError("x, W, y must share a dtype")
    if adapters.kind == KIND_SLOTS and adapters.A.dtype != x.dtype:
        raise TypeError("adapter slots must have x's dtype")
    if adapter_ids.numel() != M:
        raise ValueError("adapter_ids must have one entry per row")
    st = lib.lora_linear(_dtype_code(x), M, k, d, xp, ldx, wp, ldw, adapters.ref(),
                         _dev(adapter_ids, "adapter_ids", torch.int32),
                         _dev(scales, "scales", torch.float32), yp, ldy,
                         _dev(workspace, "workspace"), workspace.numel(), int(path), int(flags),
                         _stream_ptr(stream))
    _check(st, "lora_linear")
    return y


def lora_linear_sliced(x: torch.Tensor, W: torch.Tensor, slices, adapter_ids: torch.Tensor,
                       y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       path: int = PATH_AUTO, flags: int = 0, stream=None) -> torch.Tensor:
    """Several LoRA projections of the same x in one call.

    W is the slices' base weights stacked by rows, [sum d_i, k]; y is
    [M, sum d_i] with slice i in its own column range."""
    lib = load_library()
    M, k = x.shape
    d_total = sum(sl.d for sl in slices)
    if W.shape[0] != d_total:
        raise ValueError("W must stack the slices' weights: %d rows expected" % d_total)
    if y is None:
        y = torch.empty((M, d_total), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.zeros(workspace_bytes_sliced(M, k, x.dtype, slices), dtype=torch.uint8,
                                device=x.device)
    xp, ldx = _rows(x, "x")
    wp, ldw = _rows(W, "W")
    yp, ldy = _rows(y, "y")
    if W.dtype != x.dtype or y.dtype != x.dtype:
        raise TypeError("x, W, y must share a dtype")
    if adapter_ids.numel() != M:
        raise ValueError("adapter_ids must have one entry per row")
    arr = _slice_array(slices)
    st = lib.lora_linear_sliced(_dtype_code(x), M, k, xp, ldx, wp, ldw, len(slices), arr,
                                _dev(adapter_ids, "adapter_ids", torch.int32), yp, ldy,
                                _dev(workspace, "workspace"), workspace.numel(), int(path),
                                int(flags), _stream_ptr(stream))
    _check(st, "lora_linear_sliced")
    return y


def lora_linear_sliced_noalloc(x: torch.Tensor, W: torch.Tensor, slices, adapter_ids: torch.Tensor,
                               y: torch.Tensor, path: int = PATH_AUTO, flags: int = 0,
                               stream=None) -> torch.Tensor:
    """lora_linear_sliced without a workspace: the library's static per-GPU
    scratch array (LORA_NOALLOC_SCRATCH_BYTES) stands in for it and the call
    allocates nothing.  y is the caller's [M, sum d_i] output."""
    lib = load_library()
    M, k = x.shape
    d_total = sum(sl.d for sl in slices)
    if W.shape[0] != d_total:
        raise ValueError("W must stack the slices' weights: %d rows expected" % d_total)
    xp, ldx = _rows(x, "x")
    wp, ldw = _rows(W, "W")
    yp, ldy = _rows(y, "y")
    if W.dtype != x.dtype or y.dtype != x.dtype:
        raise TypeError("x, W, y must share a dtype")
    if adapter_ids.numel() != M or y.shape[0] != M:
        raise ValueError("adapter_ids and y must have one entry per row")
    arr = _slice_array(slices)
    st = lib.lora_linear_sliced_noalloc(_dtype_code(x), M, k, xp, ldx, wp, ldw, len(slices), arr,
                                        _dev(adapter_ids, "adapter_ids", torch.int32), yp, ldy,
                                        int(path), int(flags), _stream_ptr(stream))
    _check(st, "lora_linear_sliced_noalloc")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20  # LORA_NOALLOC_SCRATCH_BYTES


def lora_plan(adapter_ids: torch.Tensor, adapters: Adapters, k: int, d: int, dtype: torch.dtype,
              workspace: torch.Tensor, stream=None) -> None:
    lib = load_library()
    _check(lib.lora_plan(adapter_ids.numel(), int(k), int(d), _DTYPES[dtype], adapters.ref(),
                         _dev(adapter_ids, "adapter_ids", torch.int32), _dev(workspace, "workspace"),
                         workspace.numel(), _stream_ptr(stream)), "lora_plan")


def lora_plan_view(workspace: torch.Tensor, M: int, adapters: Adapters) -> dict:
    """Copies of the plan arrays in the workspace (synchronises)."""
    lib = load_library()
    v = _CPlanView()
    _check(lib.lora_plan_view(_dev(workspace, "workspace"), workspace.numel(), int(M), adapters.ref(),
                              ctypes.byref(v)), "lora_plan_view")
    base = workspace.data_ptr()

    def arr(ptr, n):
        off = int(ptr) - base
        return workspace[off:off + 4 * n].view(torch.int32).cpu().numpy().copy()

    counters = arr(v.counters, 8)
    n_ad, n_seg = int(counters[3]), int(counters[4])
    return {
        "n_bad_ids": int(counters[0]), "n_bad_ranks": int(counters[1]),
        "n_bad_pages": int(counters[2]), "n_adapted": n_ad, "n_segments": n_seg,
        "items_gather": int(counters[5]), "items_sgmv": int(counters[6]), "rows": int(counters[7]),
        "perm": arr(v.perm, n_ad), "seg_adapter": arr(v.seg_adapter, n_seg),
        "seg_start": arr(v.seg_start, n_seg), "seg_len": arr(v.seg_len, n_seg),
    }


W_INT8, W_INT4 = 1, 2


class QWeight:
    """A quantized base weight (include/lora_row.h, lora_qweight_t): packed
    q as a device uint8 tensor [d, ldq bytes] and fp32 scales ([d] for INT8,
    [d, k / group] for INT4)."""

    def __init__(self, fmt: int, q: torch.Tensor, scales: torch.Tensor, k: int, group: int = 0):
        if q.dtype not in (torch.uint8, torch.int8) or q.dim() != 2:
            raise TypeError("q must be a 2-D uint8 / int8 tensor")
        if q.stride(1) != 1:
            raise ValueError("q rows must be contiguous")
        self.fmt, self.q, self.scales, self.k, self.group = int(fmt), q, scales, int(k), int(group)
        self.d = int(q.shape[0])
        c = _CQWeight()
        c.format = self.fmt
        c.group = self.group
        if not q.is_cuda:
            raise ValueError("q must be a device tensor")
        c.q = q.data_ptr()
        c.ldq = q.stride(0) * q.element_size()
        c.scales = _dev(scales, "scales", torch.float32)
        self._c = c

    def ref(self):
        return ctypes.byref(self._c)


def lora_gemm_q(x: torch.Tensor, W: QWeight, y: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """y = x dequant(W)^T (bf16 x and y)."""
    lib = load_library()
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((x.shape[0], W.d), dtype=x.dtype, device=x.device)
    xp, ldx = _rows(x, "x")
    yp, ldy = _rows(y, "y")
    _check(lib.lora_gemm_q(x.shape[0], x.shape[1], W.d, xp, ldx, W.ref(), yp, ldy,
                           _stream_ptr(stream)), "lora_gemm_q")
    return y


def lora_linear_sliced_q(x: torch.Tensor, W: QWeight, slices, adapter_ids: torch.Tensor,
                         y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         path: int = PATH_AUTO, flags: int = 0, stream=None) -> torch.Tensor:
    """lora_linear_sliced over a quantized stacked base weight (bf16)."""
    lib = load_library()
    M, k = x.shape
    d_total = sum(sl.d for sl in slices)
    if W.d != d_total:
        raise ValueError("W must stack the slices' weights: %d rows expected" % d_total)
    if y is None:
        y = torch.empty((M, d_total), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.zeros(workspace_bytes_sliced(M, k, x.dtype, slices), dtype=torch.uint8,
                                device=x.device)
    xp, ldx = _rows(x, "x")
    yp, ldy = _rows(y, "y")
    if adapter_ids.numel() != M:
        raise ValueError("adapter_ids must have one entry per row")
    arr = _slice_array(slices)
    st = lib.lora_linear_sliced_q(M, k, xp, ldx, W.ref(), len(slices), arr,
                                  _dev(adapter_ids, "adapter_ids", torch.int32), yp, ldy,
                                  _dev(workspace, "workspace"), workspace.numel(), int(path),
                                  int(flags), _stream_ptr(stream))
    _check(st, "lora_linear_sliced_q")
    return y


def lora_merge(W: torch.Tensor, adapters: Adapters, adapter: int, scales: torch.Tensor,
               coef: float = 1.0, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """W' = W + coef * scales[adapter] * B_a A_a (out=W merges in place)."""
    lib = load_library()
    if out is None:
        out = torch.empty_like(W)
    wp, ldw = _rows(W, "W")
    op, ldo = _rows(out, "out")
    if out.dtype != W.dtype or out.shape != W.shape:
        raise TypeError("out must match W in dtype and shape")
    if adapters.kind == KIND_SLOTS and adapters.A.dtype != W.dtype:
        raise TypeError("adapter slots must have W's dtype")
    _check(lib.lora_merge(_dtype_code(W), W.shape[0], W.shape[1], wp, ldw, adapters.ref(),
                          int(adapter), _dev(scales, "scales", torch.float32), float(coef), op, ldo,
                          _stream_ptr(stream)), "lora_merge")
    return out


def lora_translate(adapters: Adapters, adapter: torch.Tensor, logical_off: torch.Tensor,
                   stream=None) -> torch.Tensor:
    lib = load_library()
    n = adapter.numel()
    if logical_off.numel() != n:
        raise ValueError("adapter and logical_off differ in length")
    out = torch.empty(n, dtype=torch.int64, device=adapter.device)
    _check(lib.lora_translate(adapters.ref(), _dev(adapter, "adapter", torch.int32),
                              _dev(logical_off, "logical_off", torch.int64), n,
                              _dev(out, "phys_off"), _stream_ptr(stream)), "lora_translate")
    return out


def lora_check(workspace: torch.Tensor, stream=None) -> dict:
    """Device error counters of a workspace (synchronises the stream)."""
    lib = load_library()
    a, b, c, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.lora_check(_dev(workspace, "workspace"), _stream_ptr(stream), ctypes.byref(a),
                          ctypes.byref(b), ctypes.byref(c), ctypes.byref(e)), "lora_check")
    return {"n_bad_ids": a.value, "n_bad_ranks": b.value, "n_bad_pages": c.value,
            "n_sync_expired": e.value}


def test_sync_spin_limit(polls: int) -> None:
    """Testing hook: bound of the split-K pairs' wait (0: every wait expires,
    counted; negative: the default)."""
    _check(load_library().lora_test_sync_spin_limit(int(polls)), "lora_test_sync_spin_limit")


class Profiler:
    """Per-kernel GPU time from events the library records around each launch."""

    def __enter__(self):
        lib = load_library()
        _check(lib.lora_profile_read(None, 1), "lora_profile_read")
        _check(lib.lora_profile_enable(1), "lora_profile_enable")
        return self

    def __exit__(self, *exc):
        load_library().lora_profile_enable(0)
        return False

    @staticmethod
    def read(reset: bool = False) -> dict:
        p = _CProfile()
        _check(load_library().lora_profile_read(ctypes.byref(p), int(reset)), "lora_profile_read")
        return {name: {"ms": p.ms[i], "launches": p.launches[i]}
                for i, name in enumerate(KERNEL_CLASSES)} | {"dropped": p.dropped}
