"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before launching
anything (no compute calls here)."""
import ctypes
import glob
import os
import re

import pytest
import torch

import lora_row_adapter_amd as lr
from lora_row_adapter_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b(lora_\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.endswith("_t")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("lora_linear", "lora_gemm", "lora_gemm_workspace_bytes", "lora_plan", "lora_plan_view", "lora_translate",
                     "lora_check", "lora_workspace_bytes", "lora_abi_version", "lora_status_str",
                     "lora_profile_enable", "lora_profile_read", "lora_pool_create",
                     "lora_pool_load", "lora_pool_evict", "lora_pool_pin", "lora_pool_unpin",
                     "lora_pool_touch", "lora_pool_query", "lora_pool_get_stats",
                     "lora_pool_adapters", "lora_pool_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lr.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_and_status_strings():
    assert lr.abi_version() == 3
    assert lr.status_str(0) == "ok"
    assert "workspace" in lr.status_str(5)


def _slots_struct(S=4, R=16, kind=0, A=16, Bp=16, ranks=64, pool=0, table=0, page_bytes=0,
                  n_pages=0, max_pages=0):
    c = B._CAdapters()
    c.kind, c.n_adapters, c.max_rank, c.max_pages = kind, S, R, max_pages
    c.ranks, c.A, c.B, c.pool, c.page_table = ranks, A, Bp, pool, table
    c.page_bytes, c.n_pages = page_bytes, n_pages
    return c


def test_workspace_bytes_host_only():
    lib = lr.load_library()
    c = _slots_struct(S=12, R=64)
    n = lib.lora_workspace_bytes(512, 8192, 8192, 1, ctypes.byref(c))
    assert n > 0 and n % 256 == 0
    # monotone in rows; capped at the plan limit
    n2 = lib.lora_workspace_bytes(1024, 8192, 8192, 1, ctypes.byref(c))
    assert n2 > n
    assert lib.lora_workspace_bytes(8192, 1, 1, 1, ctypes.byref(c)) == \
        lib.lora_workspace_bytes(100000, 1, 1, 1, ctypes.byref(c))
    # invalid descriptors -> 0
    assert lib.lora_workspace_bytes(512, 8192, 8192, 1, None) == 0
    bad = _slots_struct(R=0)
    assert lib.lora_workspace_bytes(512, 8192, 8192, 1, ctypes.byref(bad)) == 0
    bad = _slots_struct(R=300)
    assert lib.lora_workspace_bytes(512, 8192, 8192, 1, ctypes.byref(bad)) == 0
    assert lib.lora_workspace_bytes(512, 8192, 8192, 7, ctypes.byref(c)) == 0
    pool = _slots_struct(kind=1, A=0, Bp=0, pool=256, table=64, page_bytes=3000, n_pages=4,
                         max_pages=1)
    assert lib.lora_workspace_bytes(512, 64, 64, 1, ctypes.byref(pool)) == 0  # not a power of two


def _linear(lib, c, dtype=1, M=4, k=64, d=64, x=256, ldx=64, W=512, ldw=64, ids=1024,
            scales=2048, y=4096, ldy=64, ws=8192, ws_bytes=1 << 30, path=0, flags=0):
    return lib.lora_linear(dtype, M, k, d, x, ldx, W, ldw, ctypes.byref(c) if c else None, ids,
                           scales, y, ldy, ws, ws_bytes, path, flags, None)


def test_linear_rejects_bad_arguments_on_host():
    lib = lr.load_library()
    c = _slots_struct()
    assert _linear(lib, c, dtype=5) == 3                  # dtype
    assert _linear(lib, c, ldx=32) == 2                   # ldx < k
    assert _linear(lib, c, k=60, ldx=64, ldw=64) == 2     # k not a multiple of 8 (bf16)
    assert _linear(lib, c, x=258) == 2                    # misaligned x
    assert _linear(lib, c, x=0) == 1                      # null x
    assert _linear(lib, None) == 1                        # null adapters
    assert _linear(lib, c, ids=0) == 1                    # null ids
    assert _linear(lib, c, ws=8200) == 5                  # workspace misaligned
    assert _linear(lib, c, ws_bytes=100) == 5             # workspace too small
    assert _linear(lib, c, path=9) == 1                   # bad path
    assert _linear(lib, c, flags=4) == 1                  # unknown flag
    assert _linear(lib, c, M=9000, flags=1) == 1          # plan reuse across row chunks
    assert _linear(lib, c, M=-1) == 2
    assert _linear(lib, c, M=0) == 0                      # empty batch is a no-op
    assert _linear(lib, _slots_struct(R=0)) == 4          # max_rank
    assert _linear(lib, _slots_struct(A=24)) == 2         # misaligned slots
    assert _linear(lib, _slots_struct(kind=3)) == 1


def test_gemm_and_misc_reject_bad_arguments_on_host():
    lib = lr.load_library()
    assert lib.lora_gemm(1, 4, 64, 64, 0, 64, 512, 64, 1024, 64, None, 0, None) == 1
    assert lib.lora_gemm(1, 4, 64, 64, 256, 64, 512, 64, 1024, 32, None, 0, None) == 2
    assert lib.lora_gemm(1, 0, 64, 64, 0, 64, 0, 64, 0, 64, None, 0, None) == 0
    # a misaligned workspace is refused before any launch
    assert lib.lora_gemm(1, 4, 64, 64, 256, 64, 512, 64, 1024, 64, 4096 + 16, 1 << 20, None) == 5
    assert lib.lora_check(None, None, None, None, None, None) == 1
    c = _slots_struct()
    assert lib.lora_translate(ctypes.byref(c), 16, 16, 4, 16, None) == 1   # slots have no pages
    v = B._CPlanView()
    assert lib.lora_plan_view(256, 1 << 30, 100, ctypes.byref(c), ctypes.byref(v)) == 0
    assert v.capacity_rows == 100 and v.counters == 256 and v.perm > v.counters
    assert lib.lora_plan(9000, 64, 64, 1, ctypes.byref(c), 16, 256, 1 << 30, None) == 2
    assert lib.lora_profile_enable(0) == 0
    p = B._CProfile()
    assert lib.lora_profile_read(ctypes.byref(p), 1) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="not built"):
        B.load_library()


def test_gemm_workspace_sizes():
    """Split-K pairs (256 x 144 tiles, two k halves) at shapes that would run
    128 x 144 tiles with more than 128 rows: a 256-byte header (the expired
    wait counter), per pair 8 waves x 2 x 10 MFMA blocks of 64 lanes x 16
    bytes, plus 16 bytes of arrival/ready words, each region 256-byte
    aligned."""
    bf16 = 1
    pairs = 2 * 64  # 512 rows, d = 9216
    part = pairs * 8 * 2 * 10 * 64 * 16
    assert lr.gemm_workspace_bytes(512, 8192, 9216, torch.bfloat16) == 256 + part + 2048
    assert lr.gemm_workspace_bytes(128, 8192, 9216, torch.bfloat16) == 0   # one row tile
    assert lr.gemm_workspace_bytes(512, 8192, 4096, torch.bfloat16) == 0   # not a 144-column shape
    assert lr.gemm_workspace_bytes(512, 8192, 9216, torch.float32) == 0
    assert lr.gemm_workspace_bytes(400, 8192, 9216, torch.bfloat16) == 256 + part + 2048  # ragged rows
    assert lr.gemm_workspace_bytes(384, 8192, 9216, torch.bfloat16) == 0  # 128 x 128 tiles fit one round
    lib = lr.load_library()
    assert lib.lora_gemm_workspace_bytes(512, 8192 + 64, 9216, bf16) == 0  # k halves not 64-aligned
    # the layer's workspace holds the GEMM region of every chunk it may run
    c = _slots_struct(S=12, R=64)
    small = lib.lora_workspace_bytes(128, 9216, 8192, bf16, ctypes.byref(c))
    full = lib.lora_workspace_bytes(512, 9216, 8192, bf16, ctypes.byref(c))
    assert full >= small + part
    # fp32 layers run no split GEMM
    assert lib.lora_workspace_bytes(512, 9216, 8192, 0, ctypes.byref(c)) < small + part
