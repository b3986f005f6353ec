"""The C-ABI library loads and exports every entry point include/fa.h declares,
and argument checking returns the documented status before any HIP call.
CPU only: no kernel is launched here."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "fa.h")
# FA_ABI_LIB: another build of the same library to check (the host-sanitizer build)
LIB = os.environ.get("FA_ABI_LIB") or os.path.join(ROOT, "io_aware_exact_16_amd", "libfa.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_decode",
                                    "fa_fwd_decode_noalloc", "fa_fwd_decode_workspace_bytes", "fa_fwd_fp8",
                                    "fa_fwd_fp8_ex", "fa_hadamard_fp8_quant", "fa_lse_merge", "fa_mx_fp8_quant",
                                    "fa_qkv_fp8_quant", "fa_status_string"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfa.so is not built (run `python -m io_aware_exact_16_amd.build`)")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_debug_sync_build_exports_every_declared_symbol():
    # the race-check twin (the same sources built with FA_DEBUG_SYNC) is a drop-in replacement
    path = os.path.join(ROOT, "io_aware_exact_16_amd", "libfa_debugsync.so")
    if not os.path.exists(path):
        pytest.fail("libfa_debugsync.so is not built (run `python -m io_aware_exact_16_amd.build`)")
    dl = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(dl, name), name
    with open(path, "rb") as f, open(os.path.join(ROOT, "io_aware_exact_16_amd", "libfa.so"), "rb") as g:
        assert f.read() != g.read(), "the debug-sync build is identical to libfa.so"


def test_binding_names_match_header():
    import io_aware_exact_16_amd as fa
    for name in declared_functions():
        assert callable(getattr(fa, name)), name


def test_status_strings(lib):
    lib.fa_status_string.restype = ctypes.c_char_p
    seen = set()
    for code in range(0, -8, -1):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert lib.fa_status_string(42).decode() == "unknown status"


# Validation cases.  Each is constructed to fail a check that runs before any
# HIP call; the non-NULL "pointers" are never dereferenced.  They are only run
# where no GPU is visible, so a validation bug can never reach a real device.
FAKE = ctypes.c_void_p(0x1000)
FAKE2 = ctypes.c_void_p(0x2000)
FAKE3 = ctypes.c_void_p(0x3000)
FAKE4 = ctypes.c_void_p(0x4000)
FAKE5 = ctypes.c_void_p(0x5000)
NULL = ctypes.c_void_p(None)

FWD_CASES = [
    # (q, k, v, o, lse, B, H, N, d, scale, causal, dtype) -> status
    ((NULL, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, 0.1, 0, 1), -1),
    ((FAKE, FAKE2, FAKE3, FAKE4, NULL, 1, 1, 8, 64, 0.1, 0, 1), -1),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, 0.1, 0, 7), -3),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, 0.1, 0, 2), -3),     # FP8 goes to fa_fwd_fp8
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 96, 0.1, 0, 1), -4),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 256, 0.1, 0, 0), -4),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 0, 1, 8, 64, 0.1, 0, 1), -2),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, -3, 8, 64, 0.1, 0, 1), -2),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 0, 64, 0.1, 0, 1), -2),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 65536, 65536, 65536, 128, 0.1, 0, 1), -2),   # grid overflow
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, float("nan"), 0, 1), -6),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, float("inf"), 0, 1), -6),
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 64, 0.1, 2, 1), -6),
    ((FAKE, FAKE2, FAKE3, FAKE, FAKE5, 1, 1, 8, 64, 0.1, 0, 1), -6),         # o aliases q
    ((FAKE, FAKE2, FAKE3, FAKE4, FAKE4, 1, 1, 8, 64, 0.1, 0, 1), -6),        # lse aliases o
]


def _sig(lib):
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, I, P]
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_hadamard_fp8_quant.argtypes = [P, I, P, P, I, I, I, I, I, P]
    lib.fa_qkv_fp8_quant.argtypes = [P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.fa_mx_fp8_quant.argtypes = [P, I, P, P, I, I, I, I, I, P]
    lib.fa_fwd_fp8_ex.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P]
    lib.fa_fwd_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_fwd_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, ctypes.c_size_t, P]
    lib.fa_fwd_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_lse_merge.argtypes = [P, P, I, I, I, I, I, P, I, P, P]
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, ctypes.c_size_t, P]


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
@pytest.mark.parametrize("args,status", FWD_CASES)
def test_fa_fwd_validation(lib, args, status):
    _sig(lib)
    assert lib.fa_fwd(*args, None) == status


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_fa_fwd_fp8_validation(lib):
    _sig(lib)
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(8)]
    assert lib.fa_fwd_fp8(*p[:7], NULL, 1, 1, 8, 128, 0.1, 0, None) == -1
    assert lib.fa_fwd_fp8(*p, 1, 1, 8, 64, 0.1, 0, None) == -4
    assert lib.fa_fwd_fp8(*p, 1, 0, 8, 128, 0.1, 0, None) == -2
    assert lib.fa_fwd_fp8(*p, 1, 1, 8, 128, float("nan"), 0, None) == -6
    assert lib.fa_fwd_fp8(*p, 1, 1, 8, 128, 0.1, 5, None) == -6
    q = list(p)
    q[6] = q[0]                                                     # o aliases q8
    assert lib.fa_fwd_fp8(*q, 1, 1, 8, 128, 0.1, 0, None) == -6


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_quant_validation(lib):
    _sig(lib)
    assert lib.fa_hadamard_fp8_quant(NULL, 1, FAKE2, FAKE3, 1, 1, 8, 128, 1, None) == -1
    assert lib.fa_hadamard_fp8_quant(FAKE, 2, FAKE2, FAKE3, 1, 1, 8, 128, 1, None) == -3
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 8, 64, 1, None) == -4   # Hadamard needs d=128
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 8, 96, 0, None) == -4
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 0, 128, 1, None) == -2
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 8, 128, 3, None) == -6
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE, FAKE3, 1, 1, 8, 128, 1, None) == -6
    # one head of the input is addressed with 32-bit byte offsets: N d sizeof(x) < 2^32
    assert lib.fa_hadamard_fp8_quant(FAKE, 0, FAKE2, FAKE3, 1, 1, 1 << 23, 128, 1, None) == -2   # fp32
    assert lib.fa_hadamard_fp8_quant(FAKE, 0, FAKE2, FAKE3, 1, 1, 1 << 23, 128, 0, None) == -2
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 1 << 24, 128, 1, None) == -2   # bf16
    assert lib.fa_hadamard_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 1 << 25, 64, 0, None) == -2


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_qkv_quant_validation(lib):
    _sig(lib)
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(9)]
    f = lambda ptrs, dt=1, B=1, H=1, N=8, d=128, flags=5: lib.fa_qkv_fp8_quant(
        ptrs[0], ptrs[1], ptrs[2], dt, *ptrs[3:], B, H, N, d, flags, None)
    assert f([NULL] + p[1:]) == -1
    assert f(p[:8] + [NULL]) == -1
    assert f(p, dt=2) == -3
    assert f(p, flags=8) == -6 and f(p, flags=-1) == -6
    assert f(p, d=64) == -4
    assert f(p, N=0) == -2 and f(p, B=0) == -2
    assert f(p, dt=0, N=1 << 23) == -2 and f(p, N=1 << 24) == -2      # 32-bit offsets per head
    q = list(p)
    q[4] = q[1]                                                       # k8 aliases k
    assert f(q) == -6
    q = list(p)
    q[8] = q[6]                                                       # v_scale aliases q_scale
    assert f(q) == -6


def test_decode_workspace_bytes(lib):
    """Host-only size query: a whole number of key chunks of at least 256 keys each
    (fewer only when Nk < 256), and 0 for invalid sizes."""
    _sig(lib)
    ws = lib.fa_fwd_decode_workspace_bytes
    for bad in [(0, 1, 1, 8, 128), (1, 1, 0, 8, 128), (1, 1, 1, 0, 128), (1, 1, 1, 8, 96)]:
        assert ws(*bad) == 0
    for (B, H, Nq, Nk, d) in [(1, 1, 1, 1, 128), (1, 1, 1, 200, 64), (4, 32, 1, 32768, 128), (2, 8, 40, 5000, 128),
                              (1, 32, 7, 131072, 64), (64, 64, 33, 4096, 128)]:
        n = ws(B, H, Nq, Nk, d)
        per_split = B * H * Nq * (d + 1) * 4
        assert n > 0 and n % per_split == 0, (B, H, Nq, Nk, d, n)
        S = n // per_split
        assert 1 <= S <= max(1, -(-Nk // 256)), (B, H, Nq, Nk, d, S)
        if B * H * (-(-Nq // 32)) >= 2048:
            assert S == 1
    assert ws(4, 32, 1, 32768, 128) == 16 * 4 * 32 * 129 * 4     # 16 chunks of 2048 keys


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_decode_and_merge_validation(lib):
    _sig(lib)
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(6)]
    big = 1 << 30
    dec = lib.fa_fwd_decode
    assert dec(*p[:5], 1, 1, 1, 64, 128, 0.1, 1, NULL, big, None) == -1              # no workspace
    assert dec(*p[:5], 1, 1, 1, 64, 96, 0.1, 1, p[5], big, None) == -4
    assert dec(*p[:5], 1, 1, 65, 64, 128, 0.1, 1, p[5], big, None) == -2             # causal needs Nq <= Nk
    assert dec(*p[:5], 1, 1, 0, 64, 128, 0.1, 0, p[5], big, None) == -2
    assert dec(*p[:5], 1, 1, 1, 64, 128, float("nan"), 0, p[5], big, None) == -6
    assert dec(*p[:5], 1, 1, 1, 64, 128, 0.1, 3, p[5], big, None) == -6
    assert dec(*p[:5], 1, 1, 1, 64, 128, 0.1, 1, p[5], 16, None) == -6               # workspace too small
    assert dec(*p[:5], 1, 1, 1, 64, 128, 0.1, 1, p[0], big, None) == -6              # workspace aliases q
    assert dec(p[0], p[1], p[2], p[0], p[4], 1, 1, 1, 64, 128, 0.1, 1, p[5], big, None) == -6   # o aliases q
    mrg = lib.fa_lse_merge
    assert mrg(NULL, p[1], 2, 1, 1, 8, 128, p[2], 0, p[3], None) == -1
    assert mrg(p[0], p[1], 2, 1, 1, 8, 128, p[2], 2, p[3], None) == -3              # FP8 output: no
    assert mrg(p[0], p[1], 2, 1, 1, 8, 96, p[2], 0, p[3], None) == -4
    assert mrg(p[0], p[1], 0, 1, 1, 8, 128, p[2], 0, p[3], None) == -2              # no part
    assert mrg(p[0], p[1], 2, 1, 1, 8, 128, p[0], 0, p[3], None) == -6              # o aliases o_parts
    assert mrg(p[0], p[1], 2, 1, 1, 8, 128, p[2], 1, p[2], None) == -6              # lse aliases o


def test_bwd_workspace_bytes(lib):
    """Host-only size query: Delta and LSE log2(e), float32 [B,H,N] each, each part
    256-byte aligned."""
    _sig(lib)
    ws = lib.fa_bwd_workspace_bytes
    for bad in [(0, 1, 8, 128), (1, 0, 8, 128), (1, 1, 0, 128), (1, 1, 8, 96)]:
        assert ws(*bad) == 0
    up = lambda x: -(-x // 256) * 256
    for (B, H, N, d) in [(1, 1, 1, 128), (2, 16, 8192, 128), (3, 5, 1000, 64)]:
        assert ws(B, H, N, d) == 2 * up(B * H * N * 4)


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_bwd_validation(lib):
    _sig(lib)
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(10)]
    big = 1 << 30
    bwd = lib.fa_bwd

    def call(ptrs=None, B=1, H=1, N=64, d=128, scale=0.1, causal=1, dtype=1, nbytes=big):
        ptrs = p if ptrs is None else ptrs
        return bwd(*ptrs[:9], B, H, N, d, scale, causal, dtype, ptrs[9], nbytes, None)

    assert call(ptrs=p[:9] + [NULL]) == -1                      # no workspace
    assert call(ptrs=[NULL] + p[1:]) == -1
    assert call(dtype=0) == -3                                  # bf16 only
    assert call(d=96) == -4
    assert call(N=0) == -2
    assert call(scale=float("inf")) == -6
    assert call(causal=2) == -6
    assert call(nbytes=16) == -6                                # workspace too small
    q = list(p)
    q[6] = q[0]                                                 # dq aliases q
    assert call(ptrs=q) == -6
    q = list(p)
    q[8] = q[7]                                                 # dv aliases dk
    assert call(ptrs=q) == -6
    q = list(p)
    q[9] = q[4]                                                 # workspace aliases lse
    assert call(ptrs=q) == -6


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_decode_noalloc_validation(lib):
    """The same checks as fa_fwd_decode, and sizes whose partial results exceed the
    static scratch return FA_ERR_SCRATCH before any HIP call."""
    _sig(lib)
    f = lambda ptrs, B=1, H=1, Nq=1, Nk=1024, d=128, scale=0.1, causal=1: lib.fa_fwd_decode_noalloc(
        *ptrs, B, H, Nq, Nk, d, scale, causal, None)
    p = [FAKE, FAKE2, FAKE3, FAKE4, FAKE5]
    assert f([NULL] + p[1:]) == -1
    assert f(p, d=96) == -4
    assert f(p, Nq=2000, Nk=1000) == -2                 # causal needs Nq <= Nk
    assert f(p, scale=float("nan")) == -6
    assert f(p[:3] + [FAKE] + p[4:]) == -6             # o aliases q
    need = lib.fa_fwd_decode_workspace_bytes(4, 32, 64, 8192, 128)
    assert need > 16 * 1024 * 1024
    assert f(p, B=4, H=32, Nq=64, Nk=8192) == -7
    lib.fa_status_string.restype = ctypes.c_char_p
    assert b"scratch" in lib.fa_status_string(-7)


@pytest.mark.skipif(gpu_available(), reason="fake-pointer validation runs only where no GPU is visible")
def test_fp8_variant_validation(lib):
    _sig(lib)
    assert lib.fa_mx_fp8_quant(NULL, 1, FAKE2, FAKE3, 1, 1, 8, 128, 1, None) == -1
    assert lib.fa_mx_fp8_quant(FAKE, 2, FAKE2, FAKE3, 1, 1, 8, 128, 1, None) == -3
    assert lib.fa_mx_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 8, 64, 0, None) == -4
    assert lib.fa_mx_fp8_quant(FAKE, 1, FAKE2, FAKE3, 1, 1, 8, 128, 2, None) == -6
    assert lib.fa_mx_fp8_quant(FAKE, 1, FAKE, FAKE3, 1, 1, 8, 128, 1, None) == -6
    assert lib.fa_mx_fp8_quant(FAKE, 0, FAKE2, FAKE3, 1, 1, 1 << 23, 128, 1, None) == -2
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(10)]
    f = lambda ptrs, d=128, flags=0: lib.fa_fwd_fp8_ex(*ptrs, 1, 1, 8, d, 0.1, 1, flags, None)
    assert f(p[:6] + [NULL] + p[7:]) == -6                           # q_mx without k_mx
    assert f(p[:7] + [NULL] + p[8:]) == -6                           # k_mx without q_mx
    assert f(p, flags=2) == -6
    assert f(p, d=64) == -4
    q = list(p)
    q[8] = q[6]                                                       # o aliases q_mx
    assert f(q) == -6
    assert f([NULL] + p[1:]) == -1
