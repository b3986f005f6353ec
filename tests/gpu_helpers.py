"""Helpers shared by the GPU parity tests: run the HIP path, compare with the oracle."""
import sys

import numpy as np
import torch

import io_aware_exact_16_amd as fa
import oracle

# Tolerances.  bf16: max |O - O_ref| <= 2e-2 and |LSE - LSE_ref| <= 1e-3 * max(1, |LSE_ref|)
# against the unrounded float64 oracle on the same (bf16-rounded) inputs.
# f32: 1e-4 on O and 1e-5 * max(1, |LSE_ref|) on LSE (float32 arithmetic throughout).
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-4, 1e-5)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return tuple(t.to("cuda:0").contiguous() for t in ts)


def f64(t):
    return t.detach().to("cpu").double().numpy()


def run_attention(q, k, v, causal, scale):
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


def compare(o, lse, o_ref, lse_ref, kind):
    tol_o, tol_l = TOL[kind]
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    err_l = float((np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()) if lse.size else 0.0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert err_o <= tol_o, f"max |dO| = {err_o:.3g} > {tol_o}"
    assert err_l <= tol_l, f"max |dLSE|/max(1,|LSE|) = {err_l:.3g} > {tol_l}"
    return err_o, err_l


def sample_rows(N, n, seed):
    """n query rows of 0..N-1 including the first and last ones (and tile edges)."""
    r = np.random.default_rng(seed)
    fixed = [0, 1, N - 1] + [x for x in (63, 64, 127, 128, 129, 4095, 4096, N // 2) if x < N]
    rest = r.choice(N, size=min(N, n), replace=False)
    return np.unique(np.concatenate([fixed, rest]).astype(np.int64))


def compare_sampled(q, k, v, o, lse, causal, scale, kind, heads, rows):
    """Compare selected (b, h) heads and rows of a full-size result with the oracle."""
    qn, kn, vn = f64(q), f64(k), f64(v)
    worst = (0.0, 0.0)
    for (b, h) in heads:
        o_ref, lse_ref = oracle.attention(qn[b:b + 1, h:h + 1, rows], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1],
                                          scale, causal, q_index=rows)
        e = compare(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], o_ref, lse_ref, kind)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    return worst


# ---------------------------------------------------------------------------
# FP8 quantiser codes against the float64 definition
U32 = 2.0 ** -24     # unit roundoff of float32


def fp8_code_margins(x, hadamard):
    """The quantiser's float32 error bound, per element, in units of the quotient
    y / s: the transform is formed with float32 butterflies (log2 d stages, each
    adding at most U32 times the row's l1 norm), the block maximum from those
    values, and the quotient by one float32 multiply of float32 operands.
    Returns (oracle quotients t, block maxima A, margins eps)."""
    xn = np.asarray(x, dtype=np.float64)
    B, H, N, d = xn.shape
    t, A = oracle.quotients(xn, hadamard)
    stages = int(np.log2(d)) if hadamard else 0
    e_row = stages * U32 * np.abs(xn).sum(axis=3) * 1.01            # [B,H,N] transform error bound
    nb = A.shape[2]
    e_blk = np.zeros_like(A)
    for j in range(nb):
        e_blk[:, :, j] = e_row[:, :, 128 * j:128 * (j + 1)].max(axis=2)
    Ar = np.repeat(A, 128, axis=2)[:, :, :N]
    er = np.repeat(e_blk, 128, axis=2)[:, :, :N]
    with np.errstate(divide="ignore", invalid="ignore"):
        eps = np.where(Ar[..., None] > 0,
                       (448.0 * e_row[..., None] + np.abs(t) * er[..., None]) / Ar[..., None] + 4 * U32 * np.abs(t),
                       0.0)
    return t, A, eps


def check_fp8_codes(x, codes, scales, hadamard):
    """Every code must be a valid rounding of the float64 quotient within the
    kernel's float32 margin: its value lies between the E4M3 roundings of t - eps
    and t + eps (so either neighbour of a rounding boundary is accepted, and +0
    and -0 compare equal).  Scales agree with the float64 definition to the
    same margin.  Returns the number of codes whose value differs from the
    oracle's code."""
    xn = f64(x)
    t, A, eps = fp8_code_margins(xn, hadamard)
    rc, rs = oracle.quantize_blocks(xn, hadamard)
    val = oracle.e4m3_decode(codes)
    lo = oracle.e4m3_decode(oracle.e4m3_encode(t - eps))
    hi = oracle.e4m3_decode(oracle.e4m3_encode(t + eps))
    ok = (val >= lo) & (val <= hi)
    bad = int((~ok).sum())
    assert bad == 0, f"{bad} codes outside the valid rounding interval"
    ndiff = int((val != oracle.e4m3_decode(rc)).sum())
    nb = A.shape[2]
    e_blk = np.zeros_like(A)
    if hadamard:
        e_row = int(np.log2(xn.shape[3])) * U32 * np.abs(xn).sum(axis=3) * 1.01
        for j in range(nb):
            e_blk[:, :, j] = e_row[:, :, 128 * j:128 * (j + 1)].max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(A > 0, e_blk / A, 0.0) + 2 * U32
    sg, so = scales.astype(np.float64), rs.astype(np.float64)
    assert np.all(np.abs(sg - so) <= rel * so), "block scales differ from amax / 448 beyond the float32 margin"
    assert np.all(sg[A == 0] == 1.0)
    return ndiff
