"""Fused exact attention forward for MI355X (gfx950).

The computation lives in libfa.so (C ABI in include/fa.h, HIP kernels in
csrc/); ``binding`` exposes its entry points to Python with torch tensors for
device memory and streams.  libfa_debugsync.so is the race-check build of the
same sources (``debug_sync_build()`` routes the binding to it).  ``workloads`` draws the seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use.
"""
from .binding import (FA_FP8_V_HADAMARD, FA_QUANT_HADAMARD_QK, FA_QUANT_HADAMARD_V, FA_QUANT_POW2_SCALE_V, FaError,
                      attention, attention_bwd, attention_decode, attention_fp8, attention_fp8_ex, debug_sync_build, fa_bwd,
                      fa_bwd_workspace_bytes, fa_fwd, fa_fwd_decode, fa_fwd_decode_noalloc,
                      fa_fwd_decode_workspace_bytes, fa_fwd_fp8, fa_fwd_fp8_ex, fa_hadamard_fp8_quant, fa_lse_merge,
                      fa_mx_fp8_quant, fa_qkv_fp8_quant, fa_status_string, library_path, load, load_debug_sync,
                      lse_merge, quant_fp8, quant_mx_fp8, quant_qkv_fp8)

__all__ = ["FA_FP8_V_HADAMARD", "FA_QUANT_HADAMARD_QK", "FA_QUANT_HADAMARD_V", "FA_QUANT_POW2_SCALE_V", "FaError",
           "attention", "attention_bwd", "attention_decode", "attention_fp8", "attention_fp8_ex", "debug_sync_build", "fa_bwd",
           "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_decode", "fa_fwd_decode_noalloc",
           "fa_fwd_decode_workspace_bytes", "fa_fwd_fp8", "fa_fwd_fp8_ex", "fa_hadamard_fp8_quant", "fa_lse_merge",
           "fa_mx_fp8_quant", "fa_qkv_fp8_quant", "fa_status_string", "library_path", "load", "load_debug_sync", "lse_merge",
           "quant_fp8", "quant_mx_fp8", "quant_qkv_fp8"]
