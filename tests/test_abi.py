"""The C-ABI library loads and exports every entry point include/fa.h declares,
and argument checking returns the documented status before any HIP call.
CPU only: no kernel is launched here."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "io_aware_exact_16_amd", "libfa.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_fwd", "fa_fwd_fp8", "fa_hadamard_fp8_quant", "fa_status_string"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfa.so is not built (run `python -m io_aware_exact_16_amd.build`)")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_header():
    import io_aware_exact_16_amd as fa
    for name in declared_functions():
        assert callable(getattr(fa, name)), name


def test_status_strings(lib):
    lib.fa_status_string.restype = ctypes.c_char_p
    seen = set()
    for code in range(0, -7, -1):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
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
