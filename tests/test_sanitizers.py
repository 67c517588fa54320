"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host side -- argument checks of every entry point, workspace
layout, the adapter pool manager in accounting-only mode -- is built with
ASan + UBSan (lora_row_adapter_amd.build.build_sanitized) and the host tests
run against that build in a subprocess that preloads clang's ASan runtime.
The fp64 oracle is built the same way with gcc and its pins run against it.
Any sanitizer report fails the run (halt on the first error)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_OPTS = {
    "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run(env_extra, tests, timeout=900):
    env = dict(os.environ)
    env.update(SAN_OPTS)
    env.update(env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd + tests, env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_library_host_code_under_asan_ubsan(tmp_path):
    from lora_row_adapter_amd import build
    build.build_sanitized(str(tmp_path))
    rc, out = _run({"LD_PRELOAD": build.clang_asan_runtime(), "LORA_TEST_LIB_DIR": str(tmp_path)},
                   ["tests/test_abi_host.py", "tests/test_pool_host.py"])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
    assert " passed" in out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "liblora_oracle_san.so"), sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    rc, out = _run({"LD_PRELOAD": libasan, "LORA_TEST_ORACLE_LIB": lib},
                   ["tests/test_oracle_pins.py", "-k", "test_pin"])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
    assert " passed" in out
