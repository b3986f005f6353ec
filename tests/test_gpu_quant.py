"""GPU parity of the Hadamard + per-block E4M3 quantiser against the float64
definition code = E4M3(y / s), s = amax / 448.  The kernel decides in float32,
so a code is accepted when it is a valid rounding of the exact quotient within
the kernel's stated float32 margin (check_fp8_codes); the number of codes that
differ from the oracle's is reported and bounded."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import check_fp8_codes, f64, log

pytestmark = pytest.mark.gpu


def _quant(x, hadamard):
    xd = x.to("cuda:0").contiguous()
    x8, s = fa.quant_fp8(xd, hadamard=hadamard)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), s.cpu().numpy()


def _valid(x, hadamard, tag=""):
    codes, scales = _quant(x, hadamard)
    ndiff = check_fp8_codes(x, codes, scales, hadamard)
    log(f"  {tag} hadamard={hadamard}: {ndiff} of {codes.size} codes differ from the oracle "
        f"({100.0 * ndiff / max(codes.size, 1):.4f} %), all within the float32 margin")
    assert ndiff <= 1e-3 * codes.size + 1
    return ndiff


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("N", [1, 100, 128, 300, 1000])
def test_bf16_codes_valid(gpu, N, hadamard):
    q, _, _ = make_qkv(custom(2, 3, N, 128, True, "fp8", seed=N + 1, outlier_frac=0.001))
    _valid(q, hadamard, f"N={N}")


@pytest.mark.parametrize("hadamard", [False, True])
def test_fp32_input_codes_valid(gpu, hadamard):
    g = torch.Generator().manual_seed(21)
    x = torch.randn(1, 2, 260, 128, generator=g)
    _valid(x, hadamard, "fp32")


@pytest.mark.parametrize("hadamard", [False, True])
def test_fp32_input_wide_exponent_spread(gpu, hadamard):
    # rows mixing magnitudes 2^-30 .. 2^10: float32 sums are no longer exact
    g = torch.Generator().manual_seed(22)
    x = torch.randn(1, 2, 256, 128, generator=g) * torch.exp2(torch.randint(-30, 11, (1, 2, 256, 128), generator=g))
    _valid(x, hadamard, "fp32 wide spread")


def test_d64_without_hadamard(gpu):
    q, _, _ = make_qkv(custom(1, 4, 333, 64, False, "bf16", seed=22))
    _valid(q, False, "d=64")


@pytest.mark.parametrize("hadamard", [False, True])
def test_fp8_workload_full_size(gpu, hadamard):
    w = WORKLOADS["fp8_causal_8k"]
    q, k, v = make_qkv(w)
    for name, x, had in (("q", q, hadamard), ("k", k, hadamard), ("v", v, False)):
        log(f"[{w.name}] quantise {name} hadamard={had}")
        _valid(x, had, f"{w.name} {name}")


def test_transform_of_basis_rows_is_hadamard_sign_pattern(gpu):
    # token i = e_i: y_u row i is row i of the +-1 matrix, so every code is +-448
    x = torch.eye(128).reshape(1, 1, 128, 128).to(torch.bfloat16)
    codes, scales = _quant(x, True)
    h = oracle.sylvester_hadamard(128)
    np.testing.assert_array_equal(codes[0, 0], np.where(h > 0, 0x7E, 0xFE).astype(np.uint8))
    assert scales[0, 0, 0] == np.float32(1.0 / (448.0 * np.sqrt(128.0)))


def test_exact_ties_with_hadamard(gpu):
    # x = 20 H[3] + 0.9375 H[70] scales coordinate 70 to exactly 21 (a tie between
    # 20 and 22, to the even code 20); float32 butterflies are exact on these values
    h = torch.from_numpy(oracle.sylvester_hadamard(128))
    x = torch.zeros(1, 1, 128, 128, dtype=torch.float32)
    x[0, 0, 0] = 20.0 * h[3] + 0.9375 * h[70]
    x[0, 0, 1] = -x[0, 0, 0]
    codes, _ = _quant(x, True)
    assert oracle.e4m3_decode(codes[0, 0, 0, 70]) == 20.0 and oracle.e4m3_decode(codes[0, 0, 1, 70]) == -20.0
    _valid(x, True, "ties")


def test_zero_block_has_unit_scale(gpu):
    x = torch.zeros(1, 1, 200, 128, dtype=torch.bfloat16)
    x[0, 0, 150:] = 1.0
    codes, scales = _quant(x, True)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, :128] & 0x7F == 0)
    _valid(x, True, "zero block")


def test_deterministic(gpu):
    q, _, _ = make_qkv(custom(2, 2, 1000, 128, True, "fp8", seed=23, outlier_frac=0.001))
    a = _quant(q, True)
    b = _quant(q, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N", [1, 300, 1000])
def test_qkv_in_one_launch_equals_three_calls(gpu, N, dtype):
    w = custom(2, 3, N, 128, True, "fp8", seed=N + 5, outlier_frac=0.001)
    q, k, v = (t.to(dtype).to("cuda:0").contiguous() for t in make_qkv(w))
    for had_qk, had_v in ((True, False), (False, False), (True, True)):
        fused = fa.quant_qkv_fp8(q, k, v, hadamard_qk=had_qk, hadamard_v=had_v, pow2_v=False)
        sep = (fa.quant_fp8(q, had_qk), fa.quant_fp8(k, had_qk), fa.quant_fp8(v, had_v))
        torch.cuda.synchronize()
        for (x8, s), (y8, t) in zip(fused, sep):
            assert torch.equal(x8, y8) and torch.equal(s, t)


@pytest.mark.parametrize("hadamard_v", [False, True])
@pytest.mark.parametrize("N", [1, 300, 1000, 8192])
def test_pow2_v_scales(gpu, N, hadamard_v):
    """V with power-of-two block scales: without the transform y / s = x 2^-E is
    exact, so the codes equal the oracle's bit for bit; with it, within the
    float32 margin.  Q and K in the same launch are unaffected."""
    w = custom(2, 2, N, 128, True, "fp8", seed=N + 9, outlier_frac=0.001)
    q, k, v = make_qkv(w)
    qd, kd, vd = (t.to("cuda:0").contiguous() for t in (q, k, v))
    (q8, qs), (k8, ks), (v8, vs) = fa.quant_qkv_fp8(qd, kd, vd, hadamard_qk=True, hadamard_v=hadamard_v, pow2_v=True)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_blocks(f64(v), hadamard_v, pow2=True)
    np.testing.assert_array_equal(vs.cpu().numpy(), rs)
    if hadamard_v:
        t, _ = oracle.quotients(f64(v), True, pow2=True)
        eps = 8 * 2.0 ** -24 * np.abs(f64(v)).sum(axis=3, keepdims=True) * 1.01 / (
            np.sqrt(128.0) * np.repeat(rs.astype(np.float64), 128, axis=2)[:, :, :N, None]) + 4 * 2.0 ** -24 * np.abs(t)
        val = oracle.e4m3_decode(v8.cpu().numpy())
        lo = oracle.e4m3_decode(oracle.e4m3_encode(t - eps))
        hi = oracle.e4m3_decode(oracle.e4m3_encode(t + eps))
        assert np.all((val >= lo) & (val <= hi))
    else:
        np.testing.assert_array_equal(v8.cpu().numpy(), rc)
    for x8, s, x in ((q8, qs, q), (k8, ks, k)):
        assert check_fp8_codes(x, x8.cpu().numpy(), s.cpu().numpy(), True) <= 1e-3 * x8.numel() + 1


@pytest.mark.parametrize("hadamard", [False, True])
def test_nan_element(gpu, hadamard):
    """A NaN element is ignored by its block's scale (the largest magnitude) and turns into NaN codes: its own
    code, or with the transform every code of its token's row.  Every other code and every scale equal those of
    the same input with that element's whole row replaced by zeros, as long as that row does not hold the block's
    largest magnitude (a zero row and a NaN row both leave the maximum to the other rows)."""
    x = make_qkv(custom(1, 2, 300, 128, False, "bf16", seed=31))[0]
    r, c = 70, 9                                   # block 0 of head 0; a row that does not hold the block maximum
    xz = x.clone()
    xz[0, 0, r, :] = 0.0
    xn = xz.clone()
    xn[0, 0, r, c] = float("nan")
    codes = []
    for t in (xz, xn):
        c8, s = fa.quant_fp8(t.to("cuda"), hadamard=hadamard)
        torch.cuda.synchronize()
        codes.append((c8.cpu().numpy(), s.cpu().numpy()))
    (cz, sz), (cn, sn) = codes
    assert np.isfinite(sn).all() and np.array_equal(sn, sz)
    is_nan = (cn & 0x7F) == 0x7F                   # E4M3 NaN: exponent and mantissa all ones
    want = np.zeros(cn.shape, bool)
    if hadamard:
        want[0, 0, r, :] = True
    else:
        want[0, 0, r, c] = True
    assert np.array_equal(is_nan, want)
    assert np.array_equal(cn[~want], cz[~want])
