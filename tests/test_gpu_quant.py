"""GPU parity of the Hadamard + per-block E4M3 quantiser: codes bit-exact and
scales equal to the oracle's (both take the rounding decision on the same
float32 quotient; the transform itself is exact)."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import f64, log

pytestmark = pytest.mark.gpu


def _quant(x, hadamard):
    xd = x.to("cuda:0").contiguous()
    x8, s = fa.quant_fp8(xd, hadamard=hadamard)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), s.cpu().numpy()


def _exact(x, hadamard):
    codes, scales = _quant(x, hadamard)
    rc, rs = oracle.quantize_blocks(f64(x), hadamard)
    mism = int((codes != rc).sum())
    assert mism == 0, f"{mism} codes differ from the oracle"
    np.testing.assert_array_equal(scales, rs)


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("N", [1, 100, 128, 300, 1000])
def test_bf16_codes_exact(gpu, N, hadamard):
    q, _, _ = make_qkv(custom(2, 3, N, 128, True, "fp8", seed=N + 1, outlier_frac=0.001))
    _exact(q, hadamard)


@pytest.mark.parametrize("hadamard", [False, True])
def test_fp32_input_codes_exact(gpu, hadamard):
    g = torch.Generator().manual_seed(21)
    x = torch.randn(1, 2, 260, 128, generator=g)
    _exact(x, hadamard)


def test_d64_without_hadamard(gpu):
    q, _, _ = make_qkv(custom(1, 4, 333, 64, False, "bf16", seed=22))
    _exact(q, False)


@pytest.mark.parametrize("hadamard", [False, True])
def test_fp8_workload_full_size(gpu, hadamard):
    w = WORKLOADS["fp8_causal_8k"]
    q, k, v = make_qkv(w)
    for name, x, had in (("q", q, hadamard), ("k", k, hadamard), ("v", v, False)):
        log(f"[{w.name}] quantise {name} hadamard={had}")
        _exact(x, had)


def test_transform_of_basis_rows_is_hadamard_sign_pattern(gpu):
    # token i = e_i: y_u row i is row i of the +-1 matrix, so every code is +-448
    x = torch.eye(128).reshape(1, 1, 128, 128).to(torch.bfloat16)
    codes, scales = _quant(x, True)
    h = oracle.sylvester_hadamard(128)
    np.testing.assert_array_equal(codes[0, 0], np.where(h > 0, 0x7E, 0xFE).astype(np.uint8))
    assert scales[0, 0, 0] == np.float32(1.0 / (448.0 * np.sqrt(128.0)))


def test_zero_block_has_unit_scale(gpu):
    x = torch.zeros(1, 1, 200, 128, dtype=torch.bfloat16)
    x[0, 0, 150:] = 1.0
    codes, scales = _quant(x, True)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, :128] == 0)
    _exact(x, True)


def test_deterministic(gpu):
    q, _, _ = make_qkv(custom(2, 2, 1000, 128, True, "fp8", seed=23, outlier_frac=0.001))
    a = _quant(q, True)
    b = _quant(q, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
