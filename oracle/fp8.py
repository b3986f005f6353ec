"""Plain fp64 emulation of the FP8 path with incoherent processing.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module; the product path
never calls it.  It shares no code with the GPU path (no table, constant or
helper is common to both).

What the pages fix ("FlashAttention-3 (PT)", section "Inovacoes tecnicas",
item 3, low precision FP8 with incoherent processing; same list in the (SV)
and (IT) versions):
  1. before attention, Q and K are multiplied by a random orthogonal matrix,
     for example a Hadamard matrix;
  2. that spreads outlier coordinates over all coordinates;
  3. then Q and K are quantised to FP8, with less error;
  4. since the matrix is orthogonal it cancels in Q K^T, so the attention
     result is unchanged.

Readings where the pages are silent:
  - the matrix is the Sylvester Hadamard matrix of order d (d = 128), natural
    order, divided by sqrt(d) so it is orthogonal; the same matrix for every
    head, applied over the head dimension (row vector x -> x H);
  - FP8 is the OCP E4M3 "fn" format: 1 sign, 4 exponent (bias 7) and 3
    mantissa bits, no infinities, one NaN pattern per sign (S.1111.111),
    largest finite 448, subnormals m * 2^-9; conversion rounds to nearest,
    ties to even, and clamps magnitudes above 448 to 448;
  - scaling is per block: one scale per (batch, head, block of 128 tokens),
    over all d coordinates; s = amax / 448, or s = 1 when the block is all
    zero; the last block covers the remaining rows only; code = E4M3(y / s);
    the scale is stored as float32 (s rounded once from float64) and
    dequantisation is code * s;
  - the rounding decision is the definition itself, taken as exactly as
    float64 allows: with y_u = x H (the +-1 matrix; exact in float64 for bf16
    inputs) and A = max |y_u| over the block, the 1/sqrt(d) of the orthonormal
    matrix cancels and y / s is the real number 448 y_u / A, formed by one
    float64 division of exact operands (so an exact E4M3 tie, for example
    y_u = 0.9375 in a block whose maximum is 20, which scales to exactly 21,
    stays a tie and goes to the even code); the quantiser kernel decides in its
    own float32 arithmetic, so near a rounding boundary either neighbour is a
    valid code, and the tests check that against the float64 quotient this
    module returns (quotients());
  - variants (beyond the pages' pair of arms): MX-style scales, one power of
    two per 32 consecutive coordinates of a token (the OCP microscaling
    layout; the exponent is ceil(log2(amax / 448)) so that nothing clips),
    which the FP8 matrix instruction applies per lane; and the Hadamard transform of V with
    its inverse applied to O, which the orthogonality of the matrix allows
    (O = P V = (P V H) H^T);
  - V is quantised per block without the Hadamard matrix, with a power-of-two
    scale s = 2^ceil(log2(amax / 448)) (the E8M0 form, which the FP8 matrix
    instruction applies exactly; E4M3 is a floating format, so V's own
    rounding error does not change), so that the V scale never has to ride
    in P's E4M3 mantissa (see below);
  - inside attention P is quantised too (both products run on FP8 matrix
    cores), jointly with the V scale of its key's block relative to the
    largest V scale of the head: write s_v(j) / max_blocks s_v = 2^E_j r_j with
    E_j = ceil(log2 of that ratio), so 1/2 < r_j <= 1 (r = 1 in the block with
    the largest scale); P_j is stored as E4M3(256 p_j r_j) and stands for
    E4M3(256 p_j r_j) / (256 r_j) (the power of two 2^E_j is exact and travels
    separately); p = exp(S - m) relative to the row maximum, so 256 p r <= 256
    stays inside E4M3 range, the largest weight of the largest-scale block is
    exact, and the factor 256 keeps small p away from the subnormals whatever
    the other blocks' magnitudes; the row sum l uses the unquantised p.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def sylvester_hadamard(n: int) -> np.ndarray:
    """The +-1 Hadamard matrix of order n (a power of two) by Sylvester's
    doubling H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def orthonormal_hadamard(n: int) -> np.ndarray:
    return sylvester_hadamard(n) / np.sqrt(n)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte, read from the bit layout s.eeee.mmm."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Magnitudes of the 127 non-negative finite codes 0x00..0x7E; they increase
# strictly with the code, so the nearest value can be found by bisection.
_MAGS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest E4M3 code, ties to the even code,
    magnitudes above 448 clamped to 448, NaN to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left").clip(0, 0x7E)       # first magnitude >= a
    lo = (hi - 1).clip(0, 0x7E)
    d_hi = _MAGS[hi] - a
    d_lo = a - _MAGS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quotients(x, hadamard: bool, block: int = BLOCK, pow2: bool = False):
    """The per-block quantisation quotients y / s of a [B, H, N, d] tensor, in
    float64, and the block maxima A = max |y_u| (y_u = x H with the +-1 matrix,
    or x without the transform).  With ``pow2`` the scale is the power of two
    s = 2^ceil(log2(amax / 448)) instead of amax / 448.  Returns (t [B,H,N,d],
    A [B,H,ceil(N/block)]); t is 0 in an all-zero block."""
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    yu = x @ sylvester_hadamard(d) if hadamard else x          # y = yu / sqrt(d)
    nb = -(-N // block)
    t = np.zeros((B, H, N, d))
    amax = np.empty((B, H, nb))
    for j in range(nb):
        blk = yu[:, :, j * block:(j + 1) * block, :]
        a = np.abs(blk).max(axis=(2, 3))
        amax[:, :, j] = a
        with np.errstate(divide="ignore", invalid="ignore"):
            if pow2:                                            # y / s, s a power of two: exact division
                y = blk / np.sqrt(float(d)) if hadamard else blk
                tj = y / pow2_scale(a / (E4M3_MAX * (np.sqrt(float(d)) if hadamard else 1.0)))[:, :, None, None]
            else:
                tj = (E4M3_MAX * blk) / a[:, :, None, None]     # y / s = 448 y_u / A, one rounding
        t[:, :, j * block:(j + 1) * block, :] = np.where(a[:, :, None, None] > 0, tj, 0.0)
    return t, amax


def pow2_scale(s):
    """2^ceil(log2 s) for positive s (1 where s is 0): the power-of-two block
    scale, the E8M0 form of a scale that the FP8 matrix instruction applies
    exactly."""
    s = np.asarray(s, dtype=np.float64)
    E, _ = pow2_split(np.where(s > 0, s, 1.0))
    return np.where(s > 0, np.ldexp(1.0, E), 1.0)


def quantize_blocks(x, hadamard: bool, block: int = BLOCK, pow2: bool = False):
    """Incoherent processing (optional) then per-block FP8 quantisation of a
    [B, H, N, d] tensor: code = E4M3(y / s), s = amax / 448 (1 for an all-zero
    block), or with ``pow2`` s = 2^ceil(log2(amax / 448)).  Returns (codes
    uint8 [B,H,N,d], scales float32 [B,H,ceil(N/block)])."""
    d = np.shape(x)[-1]
    t, amax_u = quotients(x, hadamard, block, pow2)
    norm = E4M3_MAX * np.sqrt(float(d)) if hadamard else E4M3_MAX   # s = amax_u / (448 sqrt(d))
    s = np.where(amax_u > 0, amax_u / norm, 1.0)
    if pow2:
        s = pow2_scale(s)
    return e4m3_encode(t), s.astype(np.float32)


def pow2_split(s):
    """s = 2^E r with E = ceil(log2 s) and 1/2 < r <= 1, for positive finite s.
    Returns (E int64, r float64); both exact."""
    s = np.asarray(s, dtype=np.float64)
    m, e = np.frexp(s)                          # s = m 2^e, 1/2 <= m < 1
    exact = m == 0.5                            # s is a power of two: E = log2 s, r = 1
    E = np.where(exact, e - 1, e).astype(np.int64)
    return E, np.where(exact, 1.0, m)


def quantize_mx(x, hadamard: bool, group: int = 32):
    """MX-style quantisation of a [B, H, N, d] tensor along d, after the optional
    Hadamard transform: every group of 32 consecutive coordinates of a token row
    shares a power-of-two scale X = 2^ceil(log2(amax / 448)), so the group's
    largest magnitude lands in (224, 448] and nothing is clipped (the OCP
    microscaling rule 2^(floor(log2 amax) - 8) would leave amax / X in
    [256, 512) and clip the top of that range to 448), stored as its E8M0 code
    E + 127 with E clamped to [-127, 127]; code = E4M3(y / X).  An all-zero
    group gets code 0 (2^-127) and zero elements.  Returns (codes uint8
    [B,H,N,d], e8m0 uint8 [B,H,N,d/32])."""
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    y = x @ orthonormal_hadamard(d) if hadamard else x
    g = y.reshape(B, H, N, d // group, group)
    amax = np.abs(g).max(axis=-1)
    E, _ = pow2_split(np.where(amax > 0, amax / E4M3_MAX, 1.0))      # ceil(log2(amax / 448))
    E = np.clip(np.where(amax > 0, E, -127), -127, 127)
    t = g / np.ldexp(1.0, E)[..., None]                                # exact: a power of two
    codes = e4m3_encode(np.clip(t, -E4M3_MAX, E4M3_MAX)).reshape(B, H, N, d)
    return codes, (E + 127).astype(np.uint8)


def dequantize_mx(codes, e8m0, group: int = 32) -> np.ndarray:
    """code * 2^(e8m0 - 127) over groups of 32 along the last axis, in float64."""
    vals = e4m3_decode(codes)
    sc = np.ldexp(1.0, np.asarray(e8m0, dtype=np.int64) - 127)
    return vals * np.repeat(sc, group, axis=-1)


def dequantize_blocks(codes, scales, block: int = BLOCK) -> np.ndarray:
    """code * (float32 scale of its block), in float64."""
    vals = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :vals.shape[2]]
    return vals * s[..., None]


def attention_fp8(q8, k8, v8, qs, ks, vs, scale: float, causal: bool, quantize_p: bool = True,
                  block: int = BLOCK, q_mx=None, k_mx=None, v_hadamard: bool = False):
    """Attention on dequantised FP8 operands, with P itself quantised as
    E4M3(256 p r)/(256 r) when ``quantize_p`` (r: the mantissa part in (1/2, 1]
    of the key's V-block scale over the head's largest, see pow2_split; l from
    the unquantised p).  ``q_mx`` / ``k_mx``: E8M0 codes [B,H,N,d/32] of MX
    scales that multiply Q's / K's elements on top of their block scales.
    ``v_hadamard``: V's codes hold V H / sqrt(d) (the Hadamard transform of V);
    the output is transformed back, O = (P V') H / sqrt(d) (the orthonormal
    Sylvester matrix is symmetric and its own inverse).  Returns (O, LSE) in
    float64."""
    q = dequantize_blocks(q8, qs, block)
    k = dequantize_blocks(k8, ks, block)
    v = dequantize_blocks(v8, vs, block)
    if q_mx is not None:
        q = q * np.repeat(np.ldexp(1.0, np.asarray(q_mx, dtype=np.int64) - 127), 32, axis=-1)
    if k_mx is not None:
        k = k * np.repeat(np.ldexp(1.0, np.asarray(k_mx, dtype=np.int64) - 127), 32, axis=-1)
    B, H, N, d = q.shape
    idx = np.arange(N)
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    vs64 = np.asarray(vs, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(idx[None, :] > idx[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            if quantize_p:
                r = np.repeat(pow2_split(vs64[b, h] / vs64[b, h].max())[1], block)[:N][None, :]
                pq = e4m3_decode(e4m3_encode(256.0 * p * r)) / (256.0 * r)
            else:
                pq = p
            o[b, h] = (pq @ v[b, h]) / l
            lse[b, h] = (m + np.log(l))[:, 0]
    if v_hadamard:
        o = o @ orthonormal_hadamard(v.shape[3])
    return o, lse
