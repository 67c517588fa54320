"""Build liblora_row.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in _build/ (in parallel), then
linked into lora_row_adapter_amd/liblora_row.so.  Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblora_row.so")
SOURCES = ["lora_api.cpp", "plan.hip", "gemm.hip", "lora_gather.hip", "lora_sgmv.hip",
           "pool.hip", "pool_mgr.cpp", "merge.hip", "gemm_q.hip", "noalloc.hip"]
ARCH = os.environ.get("LORA_ROW_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags():
    return ["--offload-arch=%s" % ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
            # no packed-fp32 instructions anywhere in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def clang_asan_runtime() -> str:
    """The ASan runtime of the ROCm clang that hipcc drives (preloaded by a
    process that loads a sanitized build)."""
    import glob
    for c in sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")):
        return c
    raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")


def build_sanitized(out_dir: str) -> str:
    """The library with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code as usual), as
    out_dir/liblora_row.so.  The sanitizer runtime is not linked in: the
    process that loads it preloads clang_asan_runtime()."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
           "-g"]

    def comp(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [hipcc()] + common_flags() + san + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                  "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("sanitized hipcc failed for %s:\n%s" % (src, r.stdout + r.stderr))
        return obj
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(comp, SOURCES))
    lib = os.path.join(out_dir, "liblora_row.so")
    cmd = [hipcc(), "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    build(verbose=True)
