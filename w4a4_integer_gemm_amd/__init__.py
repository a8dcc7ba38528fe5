"""FoldQuant W8A8/W4A4 integer linear layers for AMD Instinct MI355X (gfx950).

The layer (the vla.cpp FoldQuant page's act + gemm nodes) runs in libfq.so:
hand-written HIP kernels behind the C ABI declared in include/fq.h.  This
package only loads that library and marshals arguments; torch provides device
memory and streams.
"""
from ._binding import (E2M3, FqError, abi_version, fq_act_bytes, fq_dequant_rows, fq_device_init, fq_fold_gain, fq_geglu,
                       fq_gemm, fq_gemm_heads, fq_test_hook,
                       fq_linear, fq_linear_heads, fq_linear_noalloc, fq_linear_noalloc_max_bytes,
                       fq_linear_workspace_bytes, fq_pack_weights, fq_prologue, fq_weight_bytes, last_error,
                       lib)
from .site import DeviceSite

__all__ = [
    "E2M3", "FqError", "abi_version", "fq_act_bytes", "fq_device_init", "fq_fold_gain", "fq_test_hook", "fq_geglu",
    "fq_gemm", "fq_gemm_heads", "fq_linear", "fq_linear_heads", "fq_linear_noalloc", "fq_linear_noalloc_max_bytes",
    "fq_linear_workspace_bytes",
    "fq_pack_weights", "fq_dequant_rows", "fq_prologue", "fq_weight_bytes", "last_error", "lib", "DeviceSite",
]
