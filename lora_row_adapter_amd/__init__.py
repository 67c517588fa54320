"""Multi-adapter LoRA linear layer for AMD MI355X (gfx950).

The product is the C-ABI library ``liblora_row.so`` (HIP kernels for CDNA4),
declared in ``include/lora_row.h``; this package is a thin ctypes binding
with the same entry-point names.  The library is loaded on first use and its
absence is an error: there is no fallback.
"""
from ._binding import (  # noqa: F401
    FLAG_REUSE_PLAN, FLAG_SEPARATE_SHRINK, KERNEL_CLASSES, PATH_AUTO, PATH_GATHER, PATH_SGMV, PLAN_MAX_ROWS, AdapterPool,
    Adapters, QWeight, W_INT4, W_INT8, lora_gemm_q, lora_linear_sliced_q,
    LoraError, Profiler, Slice, abi_version, library_path, load_library, lora_check, lora_gemm,
    lora_linear, lora_linear_sliced, lora_linear_sliced_noalloc, NOALLOC_SCRATCH_BYTES, lora_merge, lora_plan, lora_plan_view, lora_translate, new_workspace,
    status_str, workspace_bytes, workspace_bytes_sliced, gemm_workspace_bytes, test_sync_spin_limit,
)
