"""Thin Python binding of libfa.so (include/fa.h), argument marshalling only.

Every function here checks the torch tensors it is given, passes their device
pointers, sizes and the current HIP stream to the C entry point of the same
name, and raises on a negative status.  No step of the computation runs in
Python or in torch: torch only allocates device memory and supplies the
stream.  If libfa.so is missing or cannot be loaded the functions raise; there
is no fallback implementation.  Inside ``with debug_sync_build():`` the same
functions call libfa_debugsync.so instead, the race-check build of the same
sources (every LDS buffer hand-off fully serialised), whose results must equal
libfa.so's bit for bit.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa.so")
_DEBUG_SYNC_PATH = os.path.join(_PKG, "libfa_debugsync.so")
_libs = {}                 # path -> loaded library
_active = _LIB_PATH        # the library the wrappers call

FA_F32, FA_BF16, FA_FP8_E4M3 = 0, 1, 2
FA_OK = 0
STATUS_NAMES = {0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_DTYPE",
                -4: "FA_ERR_UNSUPPORTED", -5: "FA_ERR_LAUNCH", -6: "FA_ERR_ARG", -7: "FA_ERR_SCRATCH"}
FA_DECODE_SCRATCH_BYTES = 16 * 1024 * 1024
EXPORTED = ("fa_fwd", "fa_fwd_fp8", "fa_fwd_fp8_ex", "fa_hadamard_fp8_quant", "fa_mx_fp8_quant", "fa_qkv_fp8_quant", "fa_fwd_decode_workspace_bytes",
            "fa_fwd_decode", "fa_fwd_decode_noalloc",
            "fa_lse_merge", "fa_bwd_workspace_bytes", "fa_bwd", "fa_status_string")
BLOCK = 128   # tokens per FP8 scaling block


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}: {fa_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfa.so once (after torch, so both share torch's HIP runtime)."""
    return _open(_LIB_PATH)


def load_debug_sync() -> ctypes.CDLL:
    """Load the race-check build libfa_debugsync.so once."""
    return _open(_DEBUG_SYNC_PATH)


@contextlib.contextmanager
def debug_sync_build():
    """Route every wrapper of this module to libfa_debugsync.so inside the block.

    The switch is process-wide (not per thread): calls made from other threads
    while the block is open go to the debug-sync build as well."""
    global _active
    lib = load_debug_sync()
    prev, _active = _active, _DEBUG_SYNC_PATH
    try:
        yield lib
    finally:
        _active = prev


def _cur() -> ctypes.CDLL:
    return _open(_active)


def _open(path: str) -> ctypes.CDLL:
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m io_aware_exact_16_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, I, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_fwd_fp8.restype = I
    lib.fa_hadamard_fp8_quant.argtypes = [P, I, P, P, I, I, I, I, I, P]
    lib.fa_hadamard_fp8_quant.restype = I
    lib.fa_mx_fp8_quant.argtypes = [P, I, P, P, I, I, I, I, I, P]
    lib.fa_mx_fp8_quant.restype = I
    lib.fa_fwd_fp8_ex.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P]
    lib.fa_fwd_fp8_ex.restype = I
    lib.fa_qkv_fp8_quant.argtypes = [P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.fa_qkv_fp8_quant.restype = I
    lib.fa_fwd_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_fwd_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, ctypes.c_size_t, P]
    lib.fa_fwd_decode.restype = I
    lib.fa_fwd_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_fwd_decode_noalloc.restype = I
    lib.fa_lse_merge.argtypes = [P, P, I, I, I, I, I, P, I, P, P]
    lib.fa_lse_merge.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, ctypes.c_size_t, P]
    lib.fa_bwd.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    _libs[path] = lib
    return lib


def fa_status_string(status: int) -> str:
    return _cur().fa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn, status):
    if status != FA_OK:
        raise FaError(fn, status)


def _dev4(name, t, dtype, shape=None):
    if not (t.is_cuda and t.is_contiguous() and t.dtype == dtype and t.dim() == 4):
        raise ValueError(f"{name}: need a contiguous 4-d {dtype} CUDA tensor, got {t.dtype} {tuple(t.shape)}"
                         f" cuda={t.is_cuda} contiguous={t.is_contiguous()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


# ---------------------------------------------------------------------------
# the C entry points, one to one
def fa_fwd(q, k, v, o, lse, scale: float, causal: bool) -> None:
    """O, LSE <- attention(q, k, v); q/k/v/o [B,H,N,d] fp32 or bf16, lse [B,H,N] fp32."""
    dtype = q.dtype
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(dtype)
    if code is None:
        raise ValueError(f"fa_fwd: unsupported dtype {dtype}")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _dev4(name, t, dtype, (B, H, N, d))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N)):
        raise ValueError("fa_fwd: lse must be a contiguous float32 CUDA tensor [B,H,N]")
    st = _cur().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                       code, _stream(q))
    _check("fa_fwd", st)


def fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, scale: float, causal: bool) -> None:
    """O (bf16), LSE <- attention on per-block-scaled E4M3 operands (uint8 tensors)."""
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _dev4(name, t, torch.uint8, (B, H, N, d))
    _dev4("o", o, torch.bfloat16, (B, H, N, d))
    nb = -(-N // BLOCK)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and tuple(t.shape) == (B, H, nb)):
            raise ValueError(f"fa_fwd_fp8: {name} must be a contiguous float32 CUDA tensor [B,H,{nb}]")
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N)):
        raise ValueError("fa_fwd_fp8: lse must be a contiguous float32 CUDA tensor [B,H,N]")
    st = _cur().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(o),
                           _ptr(lse), B, H, N, d, float(scale), int(bool(causal)), _stream(q8))
    _check("fa_fwd_fp8", st)


FA_FP8_V_HADAMARD = 1


def fa_fwd_fp8_ex(q8, k8, v8, q_scale, k_scale, v_scale, q_mx, k_mx, o, lse, scale: float, causal: bool,
                  flags: int) -> None:
    """fa_fwd_fp8 with MX-style E8M0 scales for Q and K (uint8 [B,H,N,4], both or neither
    None) and ``flags`` (FA_FP8_V_HADAMARD: v8 holds the codes of V H / sqrt(128))."""
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _dev4(name, t, torch.uint8, (B, H, N, d))
    _dev4("o", o, torch.bfloat16, (B, H, N, d))
    nb = -(-N // BLOCK)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and tuple(t.shape) == (B, H, nb)):
            raise ValueError(f"fa_fwd_fp8_ex: {name} must be a contiguous float32 CUDA tensor [B,H,{nb}]")
    for name, t in (("q_mx", q_mx), ("k_mx", k_mx)):
        if t is not None:
            _dev4(name, t, torch.uint8, (B, H, N, d // 32))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N)):
        raise ValueError("fa_fwd_fp8_ex: lse must be a contiguous float32 CUDA tensor [B,H,N]")
    st = _cur().fa_fwd_fp8_ex(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(q_mx),
                              _ptr(k_mx), _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)), int(flags),
                              _stream(q8))
    _check("fa_fwd_fp8_ex", st)


def fa_mx_fp8_quant(x, x8, e8m0, hadamard: bool) -> None:
    """x8 (uint8 E4M3) and e8m0 (uint8 [B,H,N,4]) <- MX-style quantisation of x (bf16 or
    fp32, [B,H,N,128]): one power-of-two scale per 32 coordinates of a row, after the
    normalised Hadamard transform when ``hadamard``."""
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(x.dtype)
    if code is None:
        raise ValueError(f"fa_mx_fp8_quant: unsupported dtype {x.dtype}")
    B, H, N, d = x.shape
    _dev4("x", x, x.dtype)
    _dev4("x8", x8, torch.uint8, (B, H, N, d))
    _dev4("e8m0", e8m0, torch.uint8, (B, H, N, d // 32))
    st = _cur().fa_mx_fp8_quant(_ptr(x), code, _ptr(x8), _ptr(e8m0), B, H, N, d, int(bool(hadamard)), _stream(x))
    _check("fa_mx_fp8_quant", st)


def fa_hadamard_fp8_quant(x, x8, scales, hadamard: bool) -> None:
    """x8 (uint8 E4M3), scales [B,H,ceil(N/128)] <- per-block quantisation of x
    (bf16 or fp32), after the normalised Hadamard transform when ``hadamard``."""
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(x.dtype)
    if code is None:
        raise ValueError(f"fa_hadamard_fp8_quant: unsupported dtype {x.dtype}")
    B, H, N, d = x.shape
    _dev4("x", x, x.dtype)
    _dev4("x8", x8, torch.uint8, (B, H, N, d))
    nb = -(-N // BLOCK)
    if not (scales.is_cuda and scales.is_contiguous() and scales.dtype == torch.float32
            and tuple(scales.shape) == (B, H, nb)):
        raise ValueError(f"fa_hadamard_fp8_quant: scales must be a contiguous float32 CUDA tensor [B,H,{nb}]")
    st = _cur().fa_hadamard_fp8_quant(_ptr(x), code, _ptr(x8), _ptr(scales), B, H, N, d, int(bool(hadamard)),
                                      _stream(x))
    _check("fa_hadamard_fp8_quant", st)


FA_QUANT_HADAMARD_QK, FA_QUANT_HADAMARD_V, FA_QUANT_POW2_SCALE_V = 1, 2, 4


def fa_qkv_fp8_quant(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, flags: int) -> None:
    """q8, k8, v8 (uint8 E4M3) and their block scales <- per-block quantisation of q, k, v
    (bf16 or fp32, [B,H,N,128]) in one launch; ``flags`` is an OR of FA_QUANT_HADAMARD_QK,
    FA_QUANT_HADAMARD_V and FA_QUANT_POW2_SCALE_V."""
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(q.dtype)
    if code is None:
        raise ValueError(f"fa_qkv_fp8_quant: unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev4(name, t, q.dtype, (B, H, N, d))
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _dev4(name, t, torch.uint8, (B, H, N, d))
    nb = -(-N // BLOCK)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and tuple(t.shape) == (B, H, nb)):
            raise ValueError(f"fa_qkv_fp8_quant: {name} must be a contiguous float32 CUDA tensor [B,H,{nb}]")
    st = _cur().fa_qkv_fp8_quant(_ptr(q), _ptr(k), _ptr(v), code, _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale),
                                 _ptr(k_scale), _ptr(v_scale), B, H, N, d, int(flags), _stream(q))
    _check("fa_qkv_fp8_quant", st)


def fa_fwd_decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    """Device workspace (bytes) fa_fwd_decode needs; 0 for invalid sizes.  No GPU needed."""
    return int(_cur().fa_fwd_decode_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d)))


def fa_fwd_decode(q, k, v, o, lse, scale: float, causal: bool, workspace) -> None:
    """O, LSE <- attention of q [B,H,Nq,d] against k, v [B,H,Nk,d] (bf16), split over the keys.
    Causal: the queries are the last Nq of the Nk tokens.  ``workspace``: a CUDA tensor of
    at least fa_fwd_decode_workspace_bytes(...) bytes."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _dev4("q", q, torch.bfloat16)
    _dev4("k", k, torch.bfloat16, (B, H, Nk, d))
    _dev4("v", v, torch.bfloat16, (B, H, Nk, d))
    _dev4("o", o, torch.bfloat16, (B, H, Nq, d))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, Nq)):
        raise ValueError("fa_fwd_decode: lse must be a contiguous float32 CUDA tensor [B,H,Nq]")
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("fa_fwd_decode: workspace must be a contiguous CUDA tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = _cur().fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                              int(bool(causal)), _ptr(workspace), nbytes, _stream(q))
    _check("fa_fwd_decode", st)


def fa_fwd_decode_noalloc(q, k, v, o, lse, scale: float, causal: bool) -> None:
    """fa_fwd_decode with the partial results in the library's static device scratch
    (FA_DECODE_SCRATCH_BYTES per GPU): allocates nothing; calls that overlap on one GPU race."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _dev4("q", q, torch.bfloat16)
    _dev4("k", k, torch.bfloat16, (B, H, Nk, d))
    _dev4("v", v, torch.bfloat16, (B, H, Nk, d))
    _dev4("o", o, torch.bfloat16, (B, H, Nq, d))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, Nq)):
        raise ValueError("fa_fwd_decode_noalloc: lse must be a contiguous float32 CUDA tensor [B,H,Nq]")
    st = _cur().fa_fwd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                                      int(bool(causal)), _stream(q))
    _check("fa_fwd_decode_noalloc", st)


def fa_lse_merge(o_parts, lse_parts, o, lse) -> None:
    """O, LSE <- merge of P partial attentions: o_parts [P,B,H,N,d] and lse_parts [P,B,H,N]
    (float32); o [B,H,N,d] float32 or bf16, lse [B,H,N] float32."""
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(o.dtype)
    if code is None:
        raise ValueError(f"fa_lse_merge: unsupported output dtype {o.dtype}")
    if not (o_parts.is_cuda and o_parts.is_contiguous() and o_parts.dtype == torch.float32 and o_parts.dim() == 5):
        raise ValueError("fa_lse_merge: o_parts must be a contiguous float32 CUDA tensor [P,B,H,N,d]")
    P, B, H, N, d = o_parts.shape
    if not (lse_parts.is_cuda and lse_parts.is_contiguous() and lse_parts.dtype == torch.float32
            and tuple(lse_parts.shape) == (P, B, H, N)):
        raise ValueError("fa_lse_merge: lse_parts must be a contiguous float32 CUDA tensor [P,B,H,N]")
    _dev4("o", o, o.dtype, (B, H, N, d))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N)):
        raise ValueError("fa_lse_merge: lse must be a contiguous float32 CUDA tensor [B,H,N]")
    st = _cur().fa_lse_merge(_ptr(o_parts), _ptr(lse_parts), P, B, H, N, d, _ptr(o), code, _ptr(lse),
                             _stream(o_parts))
    _check("fa_lse_merge", st)


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    """Device workspace (bytes) fa_bwd needs; 0 for invalid sizes.  No GPU needed."""
    return int(_cur().fa_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale: float, causal: bool, workspace) -> None:
    """dQ, dK, dV <- gradients of sum(dout * O) for O, LSE = attention(q, k, v); all
    [B,H,N,d] bf16 except lse [B,H,N] float32.  ``workspace``: a CUDA tensor of at
    least fa_bwd_workspace_bytes(...) bytes."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _dev4(name, t, torch.bfloat16, (B, H, N, d))
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N)):
        raise ValueError("fa_bwd: lse must be a contiguous float32 CUDA tensor [B,H,N]")
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("fa_bwd: workspace must be a contiguous CUDA tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = _cur().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                       B, H, N, d, float(scale), int(bool(causal)), FA_BF16, _ptr(workspace), nbytes, _stream(q))
    _check("fa_bwd", st)


# ---------------------------------------------------------------------------
# allocating conveniences (torch allocates the outputs, the library computes)
def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Return (o, lse) for q, k, v [B,H,N,d] (bf16 or fp32, on the GPU)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def quant_fp8(x, hadamard: bool = True):
    """Return (x8, scales): E4M3 codes as uint8 [B,H,N,d] and float32 block scales."""
    B, H, N, d = x.shape
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, -(-N // BLOCK)), dtype=torch.float32, device=x.device)
    fa_hadamard_fp8_quant(x, x8, scales, hadamard)
    return x8, scales


def quant_qkv_fp8(q, k, v, hadamard_qk: bool = True, hadamard_v: bool = False, pow2_v: bool = True):
    """Return ((q8, qs), (k8, ks), (v8, vs)) from one fa_qkv_fp8_quant launch (by default
    the FP8 attention path: Q and K transformed, V with a power-of-two block scale)."""
    B, H, N, d = q.shape
    xs = [torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device) for _ in range(3)]
    ss = [torch.empty((B, H, -(-N // BLOCK)), dtype=torch.float32, device=q.device) for _ in range(3)]
    flags = ((FA_QUANT_HADAMARD_QK if hadamard_qk else 0) | (FA_QUANT_HADAMARD_V if hadamard_v else 0)
             | (FA_QUANT_POW2_SCALE_V if pow2_v else 0))
    fa_qkv_fp8_quant(q, k, v, *xs, *ss, flags)
    return tuple(zip(xs, ss))


def attention_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None):
    """Return (o bf16, lse fp32) for E4M3 operands and their block scales."""
    if scale is None:
        scale = 1.0 / math.sqrt(q8.shape[-1])
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, scale, causal)
    return o, lse


def quant_mx_fp8(x, hadamard: bool = True):
    """Return (x8, e8m0) from fa_mx_fp8_quant."""
    B, H, N, d = x.shape
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    e8 = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device=x.device)
    fa_mx_fp8_quant(x, x8, e8, hadamard)
    return x8, e8


def attention_fp8_ex(q8, k8, v8, q_scale, k_scale, v_scale, q_mx=None, k_mx=None, causal: bool = False,
                     scale: float | None = None, v_hadamard: bool = False):
    """Return (o bf16, lse fp32) from fa_fwd_fp8_ex."""
    if scale is None:
        scale = 1.0 / math.sqrt(q8.shape[-1])
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    fa_fwd_fp8_ex(q8, k8, v8, q_scale, k_scale, v_scale, q_mx, k_mx, o, lse, scale, causal,
                  FA_FP8_V_HADAMARD if v_hadamard else 0)
    return o, lse


def attention_decode(q, k, v, causal: bool = False, scale: float | None = None):
    """Return (o bf16, lse fp32) for q [B,H,Nq,d] against k, v [B,H,Nk,d] (bf16, on the GPU);
    the workspace is a torch allocation."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    B, H, Nq, d = q.shape
    nbytes = fa_fwd_decode_workspace_bytes(B, H, Nq, k.shape[2], d)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_decode(q, k, v, o, lse, scale, causal, ws)
    return o, lse


def lse_merge(o_parts, lse_parts, out_dtype=torch.float32):
    """Return (o, lse) merging partial attentions o_parts [P,B,H,N,d], lse_parts [P,B,H,N]."""
    o = torch.empty(o_parts.shape[1:], dtype=out_dtype, device=o_parts.device)
    lse = torch.empty(o_parts.shape[1:4], dtype=torch.float32, device=o_parts.device)
    fa_lse_merge(o_parts, lse_parts, o, lse)
    return o, lse


def attention_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None):
    """Return (dq, dk, dv) bf16 for the forward (o, lse) = attention(q, k, v, causal, scale)
    and the upstream gradient dout; the workspace is a torch allocation."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    B, H, N, d = q.shape
    ws = torch.empty(max(fa_bwd_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale, causal, ws)
    return dq, dk, dv
