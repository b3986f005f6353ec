"""GPU parity of the two FP8 variants of incoherent processing ("FlashAttention-3
(PT)", "Inovacoes tecnicas", item 3, taken further): MX-style E8M0 scales per 32
coordinates of Q and K applied by the matrix instruction (fa_mx_fp8_quant +
fa_fwd_fp8_ex), and the Hadamard transform of V undone on O
(FA_QUANT_HADAMARD_V + FA_FP8_V_HADAMARD).  Quantiser codes against the oracle's
definition; attention against float64 attention on the GPU's own codes (and the
oracle's emulation of P's rounding); the variants' error on the 8k workloads
against the bf16 sources, for the record."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import U32, f64, log, sample_rows

pytestmark = pytest.mark.gpu


def rel_rmse(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("N", [1, 100, 300])
def test_mx_quantiser(gpu, N, hadamard):
    w = custom(2, 3, N, 128, True, "fp8", seed=N + 41, outlier_frac=0.001)
    x, _, _ = make_qkv(w)
    x8, e8 = fa.quant_mx_fp8(x.to("cuda:0"), hadamard)
    torch.cuda.synchronize()
    x8, e8 = x8.cpu().numpy(), e8.cpu().numpy()
    rc, re = oracle.quantize_mx(f64(x), hadamard)
    if not hadamard:      # y / X = x 2^-E is exact: the codes are the oracle's bit for bit (up to the sign of zero)
        np.testing.assert_array_equal(e8, re)
        np.testing.assert_array_equal(oracle.e4m3_decode(x8), oracle.e4m3_decode(rc))
        return
    # with the transform the group maxima come from float32 butterflies: a group whose exponent
    # differs must sit at a power-of-two boundary within that error; the codes of the others must
    # be valid roundings within the float32 margin
    xn = f64(x)
    y = xn @ oracle.orthonormal_hadamard(128)
    e_row = 7 * U32 * np.abs(xn).sum(axis=3) * 1.01 / np.sqrt(128.0)          # transform error, in y units
    g_amax = np.abs(y.reshape(*y.shape[:3], 4, 32)).max(axis=-1)
    diff = e8 != re
    if diff.any():
        ratio = g_amax[diff] / 448.0
        dist = np.abs(ratio / np.exp2(np.round(np.log2(ratio))) - 1.0)
        assert np.all(dist <= 4 * e_row[diff.any(axis=-1)].max() / g_amax[diff].min() + 1e-6)
    ok_rows = ~diff.any(axis=-1)
    X = np.repeat(np.ldexp(1.0, re.astype(np.int64) - 127), 32, axis=-1)
    t = y / X
    eps = e_row[..., None] / X * 1.01 + 4 * U32 * np.abs(t)
    val = oracle.e4m3_decode(x8)
    lo = oracle.e4m3_decode(oracle.e4m3_encode(np.clip(t - eps, -448, 448)))
    hi = oracle.e4m3_decode(oracle.e4m3_encode(np.clip(t + eps, -448, 448)))
    good = (val >= lo) & (val <= hi)
    assert np.all(good[ok_rows])
    log(f"  N={N}: {int((val != oracle.e4m3_decode(rc)).sum())} codes and {int(diff.sum())} exponents differ "
        f"from the oracle, all within the float32 margin")


def _variant_run(q, k, v, causal, scale, mx, vhad):
    """Q and K through the transform (MX: per-32 scales; else per-block), V with a
    power-of-two block scale (with its own transform for the V variant)."""
    qd, kd, vd = (t.to("cuda:0").contiguous() for t in (q, k, v))
    flags = fa.FA_QUANT_HADAMARD_QK | fa.FA_QUANT_POW2_SCALE_V | (fa.FA_QUANT_HADAMARD_V if vhad else 0)
    (q8, qs), (k8, ks), (v8, vs) = fa.quant_qkv_fp8(qd, kd, vd, hadamard_qk=True, hadamard_v=vhad, pow2_v=True)
    qe = ke = None
    if mx:
        q8, qe = fa.quant_mx_fp8(qd, True)
        k8, ke = fa.quant_mx_fp8(kd, True)
        qs, ks = torch.ones_like(qs), torch.ones_like(ks)
    o, lse = fa.attention_fp8_ex(q8, k8, v8, qs, ks, vs, qe, ke, causal=causal, scale=scale, v_hadamard=vhad)
    torch.cuda.synchronize()
    ops = [x.cpu().numpy() if x is not None else None for x in (q8, k8, v8, qs, ks, vs, qe, ke)]
    return f64(o), f64(lse), ops


@pytest.mark.parametrize("mx,vhad", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 300, 1000])
def test_variant_kernel_vs_dequantised_oracle(gpu, N, causal, mx, vhad):
    w = custom(1, 2, N, 128, causal, "fp8", seed=N * 5 + 3, outlier_frac=0.001)
    q, k, v = make_qkv(w)
    o, lse, (q8, k8, v8, qs, ks, vs, qe, ke) = _variant_run(q, k, v, causal, w.scale, mx, vhad)
    kw = dict(q_mx=qe, k_mx=ke, v_hadamard=vhad)
    o_ref, lse_ref = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, w.scale, causal, quantize_p=False, **kw)
    o_emu, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, w.scale, causal, quantize_p=True, **kw)
    e_ref, e_emu = rel_rmse(o, o_ref), rel_rmse(o, o_emu)
    e_lse = float((np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max())
    log(f"  N={N} causal={causal} mx={mx} v_hadamard={vhad}: rel RMSE vs fp64 {e_ref:.4f}, vs P-emulation "
        f"{e_emu:.4f}, LSE {e_lse:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert e_ref <= 3e-2 and e_emu <= 1.5e-2 and e_lse <= 1e-3


@pytest.mark.parametrize("name", ["fp8_causal_8k", "fp8_channels_8k"])
def test_variants_on_the_8k_workloads(gpu, name):
    """Error of each variant against float64 attention on the bf16 sources, sampled rows of
    four heads (the same rows for every arm): recorded, with a regression bound of 8e-2
    (0.3 for the plain arm on channel outliers)."""
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    rows = sample_rows(w.N, 256, 45)
    heads = [(0, 0), (0, 7), (1, 3), (1, 15)]
    qn, kn, vn = f64(q), f64(k), f64(v)
    refs = {hd: oracle.attention(qn[hd[0]:hd[0] + 1, hd[1]:hd[1] + 1, rows], kn[hd[0]:hd[0] + 1, hd[1]:hd[1] + 1],
                                 vn[hd[0]:hd[0] + 1, hd[1]:hd[1] + 1], w.scale, w.causal, q_index=rows)[0]
            for hd in heads}
    errs = {}
    for mx, vhad in ((False, False), (True, False), (False, True), (True, True)):
        o, _, _ = _variant_run(q, k, v, w.causal, w.scale, mx, vhad)
        num = sum(float(((o[b:b + 1, h:h + 1, rows] - refs[(b, h)]) ** 2).sum()) for (b, h) in heads)
        den = sum(float((refs[(b, h)] ** 2).sum()) for (b, h) in heads)
        errs[(mx, vhad)] = (num / den) ** 0.5
    log(f"[{name}] rel RMSE vs the bf16 sources (Hadamard on Q and K in every arm): block scales "
        f"{errs[(False, False)]:.4f}, MX {errs[(True, False)]:.4f}, Hadamard on V {errs[(False, True)]:.4f}, "
        f"both {errs[(True, True)]:.4f}")
    for e in errs.values():
        assert e <= 8e-2
