"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived cases, closed forms and invariants of softmax attention,
brute-force scalar loops, and library routines computing the same definition.
CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _expr(s):
    return eval(s, {"__builtins__": {}}, {"ln": math.log, "exp": math.exp})


# ---------------------------------------------------------------------------
# hand-derived fixtures
@pytest.mark.parametrize("causal", [False, True])
def test_hand_derived_cases(causal):
    cases = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        if c.get("q_is_ln3"):
            q[:] = math.log(3.0)
        k, v = np.array(c["k"], dtype=np.float64), np.array(c["v"], dtype=np.float64)
        o, lse = attention(q[None, None], k[None, None], v[None, None], c["scale"], causal)
        exp = c["causal" if causal else "noncausal"]
        o_ref = np.array([[_expr(x) for x in row] for row in exp["o"]])
        lse_ref = np.array([_expr(x) for x in exp["lse"]])
        np.testing.assert_allclose(o[0, 0], o_ref, rtol=0, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=0, atol=1e-14, err_msg=c["name"])


# ---------------------------------------------------------------------------
# brute force: scalar loops with math.exp, no arrays
def _brute(q, k, v, scale, causal):
    N, d = len(q), len(q[0])
    O, L = [], []
    for i in range(N):
        s = []
        for j in range(N):
            if causal and j > i:
                continue
            s.append((j, scale * sum(q[i][t] * k[j][t] for t in range(d))))
        m = max(x for _, x in s)
        w = [(j, math.exp(x - m)) for j, x in s]
        l = sum(x for _, x in w)
        O.append([sum(x * v[j][t] for j, x in w) / l for t in range(len(v[0]))])
        L.append(m + math.log(l))
    return O, L


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 4), (7, 2), (8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(N, d, causal):
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    scale = 0.7
    o, lse = attention(q[None, None], k[None, None], v[None, None], scale, causal)
    O, L = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o[0, 0], np.array(O), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(L), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms named for the path
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    # with V = identity, O is the probability matrix itself
    N, d = 37, 16
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    o, _ = attention(q[None, None], k[None, None], np.eye(N)[None, None], 0.3, causal)
    p = o[0, 0]
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(N, 1)] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    N, d = 29, 8
    q, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    k = np.tile(rng.standard_normal((1, d)), (N, 1))
    scale = 0.5
    o, lse = attention(q[None, None], k[None, None], v[None, None], scale, causal)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.tile(v.mean(axis=0), (N, 1))
    np.testing.assert_allclose(o[0, 0], mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], scale * q @ k[0] + np.log(cnt), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_single_token_returns_v(causal):
    q, k, v = (rng.standard_normal((3, 2, 1, 64)) for _ in range(3))
    o, lse = attention(q, k, v, 0.125, causal)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.125 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-14)


def test_causal_first_row_is_v0():
    q, k, v = (rng.standard_normal((2, 3, 50, 32)) for _ in range(3))
    o, lse = attention(q, k, v, 0.2, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.2 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-14)


def test_scale_zero_is_uniform():
    N, d = 40, 8
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    o, lse = attention(q, k, v, 0.0, False)
    np.testing.assert_allclose(o[0, 0], np.tile(v[0, 0].mean(axis=0), (N, 1)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(N), atol=1e-14)
    o, lse = attention(q, k, v, 0.0, True)
    np.testing.assert_allclose(o[0, 0], np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14)


def test_huge_scale_is_hardmax():
    N, d = 33, 16
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    o, lse = attention(q, k, v, 1e6, False)
    s = q[0, 0] @ k[0, 0].T
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o[0, 0], v[0, 0][s.argmax(axis=1)], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], 1e6 * s.max(axis=1), rtol=1e-15)


def test_permutation_equivariance():
    N, d = 45, 8
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    o, lse = attention(q, k, v, 0.4, False)
    pk, pq = rng.permutation(N), rng.permutation(N)
    o2, lse2 = attention(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.4, False)
    np.testing.assert_allclose(o2, o[:, :, pq], atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, pq], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # K <- K + 1 c^T adds scale*q_i.c to row i: O unchanged, LSE_i shifted by it
    N, d = 31, 8
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    c = rng.standard_normal(d)
    o, lse = attention(q, k, v, 0.6, causal)
    o2, lse2 = attention(q, k + c, v, 0.6, causal)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.6 * (q @ c), atol=1e-12)


def test_split_keys_merge_identity():
    # attention over two disjoint key sets, merged through their LSEs, equals
    # attention over all keys (the identity the online softmax accumulates by)
    N, d, a = 60, 16, 23
    q, k, v = (rng.standard_normal((2, 2, N, d)) for _ in range(3))
    o, lse = attention(q, k, v, 0.3, False)
    o1, l1 = attention(q, k[:, :, :a], v[:, :, :a], 0.3, False)
    o2, l2 = attention(q, k[:, :, a:], v[:, :, a:], 0.3, False)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    np.testing.assert_allclose((w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None], o, atol=1e-13)
    np.testing.assert_allclose(m + np.log(w1 + w2), lse, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_merge_of_key_chunks_is_full_attention(causal):
    # decode-shaped rows (the last Nq positions of Nk tokens) against key chunks of
    # uneven sizes; causal chunks see the keys at their absolute positions
    Nq, Nk, d = 5, 97, 16
    q, k, v = rng.standard_normal((1, 2, Nq, d)), rng.standard_normal((1, 2, Nk, d)), rng.standard_normal((1, 2, Nk, d))
    pos = oracle.decode_positions(Nq, Nk)
    assert list(pos) == list(range(Nk - Nq, Nk))
    o, lse = attention(q, k, v, 0.3, causal, q_index=pos)
    cuts = [0, 13, 40, 41, 90, Nk]
    parts = [attention(q, k[:, :, a:b], v[:, :, a:b], 0.3, causal, q_index=pos - a) for a, b in zip(cuts, cuts[1:])]
    om, lm = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, lse, atol=1e-13)


def test_lse_merge_special_cases():
    o1 = rng.standard_normal((2, 3, 8))
    l1 = rng.standard_normal((2, 3))
    om, lm = oracle.lse_merge(o1[None], l1[None])                     # one part: identity
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, l1, atol=1e-15)
    om, lm = oracle.lse_merge(np.stack([o1, o1]), np.stack([l1, l1]))  # two equal parts: LSE + ln 2
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, l1 + math.log(2.0), atol=1e-15)
    junk = np.full_like(o1, 1e30)                                      # a part that saw no key
    om, lm = oracle.lse_merge(np.stack([junk, o1]), np.stack([np.full_like(l1, -np.inf), l1]))
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, l1, atol=1e-15)
    om, lm = oracle.lse_merge(np.stack([junk]), np.stack([np.full_like(l1, -np.inf)]))  # nothing visible
    assert np.all(om == 0) and np.all(lm == -np.inf)
    # hand-derived: parts with LSE ln 1 and ln 3 weigh 1/4 and 3/4
    om, lm = oracle.lse_merge(np.array([[[2.0]], [[6.0]]]), np.array([[0.0], [math.log(3.0)]]))
    np.testing.assert_allclose(om, [[5.0]], atol=1e-15)
    np.testing.assert_allclose(lm, [math.log(4.0)], atol=1e-15)


def test_row_subset_matches_full():
    N, d = 300, 16
    q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    o, lse = attention(q, k, v, 0.25, True)
    rows = np.array([0, 1, 77, 128, 299])
    o2, lse2 = attention(q[:, :, rows], k, v, 0.25, True, q_index=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, :, rows], atol=1e-14)
    o3, _ = attention(q, k, v, 0.25, True, row_band=64)          # banding does not change a row
    np.testing.assert_allclose(o3, o, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 256, 511])
def test_matches_torch_sdpa_fp64(N, causal):
    d = 64
    q, k, v = (torch.randn(2, 3, N, d, dtype=torch.float64, generator=torch.Generator().manual_seed(N)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=0.125)
    o, _ = attention(q.numpy(), k.numpy(), v.numpy(), 0.125, causal)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    s = 0.125 * (q @ k.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    _, lse = attention(q.numpy(), k.numpy(), v.numpy(), 0.125, causal)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Gradients (oracle.attention_bwd): pinned to finite differences of the pinned
# forward, to torch autograd, and to identities of the softmax Jacobian.
def _loss(q, k, v, do, scale, causal):
    o, _ = attention(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_central_differences(causal):
    # every element of dQ, dK, dV against a central difference of L = sum(dO * O)
    N, d, h, scale = 5, 3, 1e-5, 0.7
    q, k, v, do = (rng.standard_normal((1, 2, N, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = x0 - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=1e-8, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 130])
def test_bwd_matches_torch_autograd_fp64(N, causal):
    d = 32
    gen = torch.Generator().manual_seed(100 + N)
    q, k, v, do = (torch.randn(2, 2, N, d, dtype=torch.float64, generator=gen) for _ in range(4))
    qt, kt, vt = (t.clone().requires_grad_(True) for t in (q, k, v))
    s = 0.3 * (qt @ kt.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    (torch.softmax(s, dim=-1) @ vt).backward(do)
    dq, dk, dv = oracle.attention_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), 0.3, causal, row_band=7)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_identities(causal):
    # rows of P sum to one: sum_j dV_j = sum_i dO_i; rows of dS sum to zero:
    # sum_j dK_j = 0; S is bilinear: <Q, dQ> = <K, dK> = sum_ij dS_ij S_ij
    N, d = 40, 16
    q, k, v, do = (rng.standard_normal((2, 3, N, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.45, causal)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose((q * dq).sum(axis=(2, 3)), (k * dk).sum(axis=(2, 3)), atol=1e-11)


def test_bwd_special_cases():
    d = 8
    q, k, v, do = (rng.standard_normal((1, 1, 1, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.9, False)      # one token: O = v
    np.testing.assert_allclose(dv, do, atol=1e-15)
    assert np.all(dq == 0) and np.all(dk == 0)
    N = 9                                                            # scale 0: P = 1/N
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.0, False)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape), atol=1e-15)
    assert np.all(dq == 0) and np.all(dk == 0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True)        # causal ends
    assert np.all(dq[0, 0, 0] == 0)                                  # query 0 sees key 0 only
    _, lse = attention(q, k, v, 0.5, True)
    p_last = math.exp(0.5 * float(q[0, 0, -1] @ k[0, 0, -1]) - lse[0, 0, -1])
    np.testing.assert_allclose(dv[0, 0, -1], p_last * do[0, 0, -1], atol=1e-14)   # key N-1: query N-1 only


# ---------------------------------------------------------------------------
# Hadamard
def test_hadamard_matches_textbook_order8():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "hadamard8.txt")) if not l.startswith("#") and l.strip()]
    np.testing.assert_array_equal(oracle.sylvester_hadamard(8), np.array(rows, dtype=np.float64))


@pytest.mark.parametrize("n", [1, 2, 64, 128])
def test_hadamard_orthogonal(n):
    h = oracle.sylvester_hadamard(n)
    assert set(np.unique(h)) <= {-1.0, 1.0}
    np.testing.assert_array_equal(h @ h.T, n * np.eye(n))
    hn = oracle.orthonormal_hadamard(n)
    np.testing.assert_allclose(hn @ hn.T, np.eye(n), atol=1e-15)


def test_incoherent_processing_leaves_qk_and_attention_unchanged():
    # the orthogonal matrix cancels in Q K^T (pages: incoherent processing, step 4)
    N, d = 1024, 128
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    for x in (q, k):
        m = rng.random(x.shape) < 0.001
        x[m] = 20.0 * np.sign(rng.standard_normal(m.sum()))
    hn = oracle.orthonormal_hadamard(d)
    s0 = q[0, 0] @ k[0, 0].T
    s1 = (q[0, 0] @ hn) @ (k[0, 0] @ hn).T
    assert np.abs(s1 - s0).max() <= 1e-11
    o0, l0 = attention(q, k, v, d ** -0.5, True)
    o1, l1 = attention(q @ hn, k @ hn, v, d ** -0.5, True)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, atol=1e-12)


# ---------------------------------------------------------------------------
# E4M3
def test_e4m3_decode_anchors():
    for line in open(os.path.join(GOLDEN, "e4m3_anchors.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = oracle.e4m3_decode(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert float(got) == float(val), code


def test_e4m3_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    # ties go to the even code; values above 448 clamp; half the smallest subnormal ties to zero
    assert oracle.e4m3_encode(1.0625) == 0x38
    assert oracle.e4m3_encode(1.1875) == 0x3A
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(3 * 2.0 ** -11) == 0x01
    assert oracle.e4m3_encode(-1.0625) == 0xB8


def test_e4m3_encode_matches_torch_cast():
    x = np.concatenate([rng.standard_normal(400_000) * 50,
                        rng.uniform(-448, 448, 300_000),
                        rng.standard_normal(300_000) * 1e-2])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# per-block quantisation
def test_quantize_blocks_properties():
    B, H, N, d = 2, 3, 300, 128                       # ragged last block (300 = 2*128 + 44)
    x = rng.standard_normal((B, H, N, d))
    x[0, 1, 128:256] = 0.0                              # an all-zero block
    for had in (False, True):
        codes, scales = oracle.quantize_blocks(x, had)
        assert codes.shape == x.shape and scales.shape == (B, H, 3)
        y = x @ oracle.orthonormal_hadamard(d) if had else x
        assert scales[0, 1, 1] == 1.0 and np.all(codes[0, 1, 128:256] & 0x7F == 0)
        deq = oracle.dequantize_blocks(codes, scales)
        for b in range(B):
            for h in range(H):
                for j in range(3):
                    blk = y[b, h, j * 128:(j + 1) * 128]
                    amax = np.abs(blk).max()
                    if amax == 0:
                        continue
                    s = amax / 448.0
                    assert abs(scales[b, h, j] - s) <= 2.0 ** -24 * s
                    # the amax element lands exactly on +-448
                    i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                    assert codes[b, h, j * 128 + i[0], i[1]] & 0x7F == 0x7E
                    # rounding error: half a step, relative 2^-4 for normals, 2^-10 s absolute below
                    err = np.abs(deq[b, h, j * 128:(j + 1) * 128] - blk)
                    bound = np.maximum(np.abs(blk) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
                    assert np.all(err <= bound)


def _e4m3_grid():
    """Every finite E4M3 value with its code, from the bit layout written out
    by hand: exponent field e (bias 7), mantissa field m; e = 0 is subnormal."""
    vals = []
    for sign in (0, 1):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue                                   # NaN
                mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
                vals.append((-mag if sign else mag, (sign << 7) | (e << 3) | m))
    return vals


def _nearest_e4m3_exact(t: Fraction) -> int:
    """Round an exact rational to E4M3 by exhaustive search: the nearest finite
    value, ties to the even code (mantissa bit 0), magnitudes beyond 448 to 448."""
    grid = _nearest_e4m3_exact.grid
    best = min(abs(v - t) for v, _ in grid)
    cands = [(v, c) for v, c in grid if abs(v - t) == best]
    if len(cands) > 1:
        cands = [(v, c) for v, c in cands if v != 0 or (c & 0x80) == ((t < 0) << 7)] or cands
        even = [(v, c) for v, c in cands if c & 1 == 0]
        cands = even or cands
    return cands[0][1]


_nearest_e4m3_exact.grid = _e4m3_grid()


@pytest.mark.parametrize("hadamard", [False, True])
def test_quantize_codes_are_exact_nearest_e4m3(hadamard):
    # bf16 inputs with +-20 outliers: for sampled elements the exact rational
    # y / s = 448 y_u / A (y_u = x H summed in exact rationals) is rounded to
    # E4M3 by exhaustive search over all finite codes; the oracle must agree.
    g = torch.Generator().manual_seed(3 + hadamard)
    x = torch.randn(1, 2, 256, 128, generator=g)
    m = torch.rand(x.shape, generator=g) < 0.001
    x[m] = 20.0 * (torch.randint(0, 2, x.shape, generator=g)[m] * 2.0 - 1.0)
    x = x.to(torch.bfloat16).double().numpy()
    codes, scales = oracle.quantize_blocks(x, hadamard)
    h = [[1 if bin(i & j).count("1") % 2 == 0 else -1 for j in range(128)] for i in range(128)]   # H[i][j]
    r = np.random.default_rng(7)
    for hh in range(2):
        for j in range(2):
            blk = x[0, hh, 128 * j:128 * (j + 1)]
            fr = [[Fraction(float(v)) for v in row] for row in blk]
            if hadamard:
                yu = [[sum(fr[t][k] * h[k][i] for k in range(128)) for i in range(128)] for t in range(128)]
            else:
                yu = fr
            A = max(abs(v) for row in yu for v in row)
            assert scales[0, hh, j] == np.float32(float(A) / (448.0 * (128 ** 0.5 if hadamard else 1.0)))
            for _ in range(300):
                t, i = int(r.integers(128)), int(r.integers(128))
                want = _nearest_e4m3_exact(448 * yu[t][i] / A)
                assert codes[0, hh, 128 * j + t, i] == want, (hh, j, t, i)


def test_quantize_pow2_scales():
    # power-of-two block scales: amax / 448 <= s < 2 amax / 448, s = 1 for a zero
    # block, and each code is the exact E4M3 rounding of x / s (exhaustive search
    # over all finite codes on exact rationals, for sampled elements)
    g = torch.Generator().manual_seed(17)
    x = torch.randn(1, 2, 300, 128, generator=g).to(torch.bfloat16).double().numpy()
    x[0, 1, 128:256] = 0.0
    codes, scales = oracle.quantize_blocks(x, False, pow2=True)
    r = np.random.default_rng(8)
    for hh in range(2):
        for j in range(3):
            blk = x[0, hh, 128 * j:128 * (j + 1)]
            amax = np.abs(blk).max()
            sc = float(scales[0, hh, j])
            if amax == 0:
                assert sc == 1.0 and np.all(codes[0, hh, 128 * j:128 * (j + 1)] & 0x7F == 0)
                continue
            assert math.frexp(sc)[0] == 0.5                            # a power of two
            assert amax / 448.0 <= sc < 2.0 * amax / 448.0
            for _ in range(200):
                t, i = int(r.integers(blk.shape[0])), int(r.integers(128))
                want = _nearest_e4m3_exact(Fraction(float(blk[t, i])) / Fraction(sc))
                assert codes[0, hh, 128 * j + t, i] == want


def test_quantize_mx_exact():
    # MX-style groups of 32 coordinates: X = 2^E with E the smallest integer such
    # that amax <= 448 2^E (found here by exact comparison), and every code the
    # exact E4M3 rounding of x / X (exhaustive search on exact rationals)
    g = torch.Generator().manual_seed(19)
    x = torch.randn(1, 2, 40, 128, generator=g)
    x[0, 0, 3, 5] = 20.0                                         # an outlier widens one group only
    x[0, 1, 7, :32] = 0.0                                        # an all-zero group
    x = x.to(torch.bfloat16).double().numpy()
    codes, e8 = oracle.quantize_mx(x, False)
    assert e8.shape == (1, 2, 40, 4) and e8.dtype == np.uint8
    assert e8[0, 1, 7, 0] == 0 and np.all(codes[0, 1, 7, :32] == 0)
    r = np.random.default_rng(9)
    for _ in range(600):
        hh, t, i = int(r.integers(2)), int(r.integers(40)), int(r.integers(128))
        grp = x[0, hh, t, 32 * (i // 32):32 * (i // 32) + 32]
        amax = Fraction(float(np.abs(grp).max()))
        if amax == 0:
            continue
        E = -200
        while amax > 448 * Fraction(2) ** E:
            E += 1
        assert int(e8[0, hh, t, i // 32]) == E + 127
        assert codes[0, hh, t, i] == _nearest_e4m3_exact(Fraction(float(x[0, hh, t, i])) / Fraction(2) ** E)
    deq = oracle.dequantize_mx(codes, e8)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * np.repeat(
        np.ldexp(1.0, e8.astype(np.int64) - 127), 32, axis=-1) + 1e-300)


def test_attention_fp8_variants_compose_pinned_parts():
    # MX scales on Q and K multiply their elements; V's Hadamard variant holds the
    # codes of V H / sqrt(d) and transforms the output back: with exact operands
    # both equal plain attention on the dequantised values
    shape = (1, 2, 150, 128)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    q8, qe = oracle.quantize_mx(q, True)
    k8, ke = oracle.quantize_mx(k, True)
    vh8, vhs = oracle.quantize_blocks(v, True)                   # codes of V H / sqrt(d)
    ones = np.ones((1, 2, 2), dtype=np.float32)
    o, lse = oracle.attention_fp8(q8, k8, vh8, ones, ones, vhs, 0.09, True, quantize_p=False, q_mx=qe, k_mx=ke,
                                  v_hadamard=True)
    qd, kd = oracle.dequantize_mx(q8, qe), oracle.dequantize_mx(k8, ke)
    vd = oracle.dequantize_blocks(vh8, vhs) @ oracle.orthonormal_hadamard(128)    # back to V's coordinates
    o_ref, lse_ref = attention(qd, kd, vd, 0.09, True)
    np.testing.assert_allclose(o, o_ref, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-11)
    # and both are close to attention on the unquantised inputs (FP8 rounding only)
    o_src, _ = attention(q, k, v, 0.09, True)
    assert np.linalg.norm(o - o_src) / np.linalg.norm(o_src) < 0.06


def test_quantize_exact_tie_with_hadamard_goes_to_even():
    # x = 20 H[3] + 0.9375 H[70] (rows of the +-1 matrix) gives y_u = x H =
    # 128 (20 e_3 + 0.9375 e_70): A = 2560 and coordinate 70 scales to exactly
    # 448 * 120 / 2560 = 21, halfway between the E4M3 values 20 and 22
    h = oracle.sylvester_hadamard(128)
    x = np.zeros((1, 1, 128, 128))
    x[0, 0, 0] = 20.0 * h[3] + 0.9375 * h[70]
    x[0, 0, 1] = -(20.0 * h[3]) - 0.9375 * h[70]
    codes, scales = oracle.quantize_blocks(x, True)
    assert oracle.e4m3_decode(codes[0, 0, 0, 70]) == 20.0 and oracle.e4m3_decode(codes[0, 0, 1, 70]) == -20.0
    assert codes[0, 0, 0, 3] == 0x7E and codes[0, 0, 1, 3] == 0xFE
    t, amax = oracle.quotients(x, True)
    assert t[0, 0, 0, 70] == 21.0 and amax[0, 0, 0] == 2560.0


def test_quotients_are_one_rounding_of_the_exact_ratio():
    x = rng.standard_normal((1, 1, 128, 128)).astype(np.float32).astype(np.float64)
    t, amax = oracle.quotients(x, False)
    A = max(abs(Fraction(float(v))) for v in x.ravel())
    for (i, j) in [(0, 0), (5, 17), (127, 127), (64, 3)]:
        exact = 448 * Fraction(float(x[0, 0, i, j])) / A
        assert abs(Fraction(float(t[0, 0, i, j])) - exact) <= abs(exact) * Fraction(2) ** -53


def test_pow2_split():
    s = np.array([1.0, 0.75, 3.0, 2.0 ** -140, 2.0 ** 20, 448.0, 1.0 / 448.0, 5.0e-39, 1e30])
    E, r = oracle.pow2_split(s)
    for si, ei, ri in zip(s, E, r):
        assert 0.5 < ri <= 1.0
        assert math.ldexp(float(ri), int(ei)) == float(si)
        assert ei == math.ceil(math.log2(float(si))) or (si == 5.0e-39)   # log2 of a subnormal may round


def test_quantize_exact_tie_goes_to_even():
    # a block with amax 20: x = 0.9375 scales to exactly 21, halfway between 20 and 22
    x = np.zeros((1, 1, 128, 64))
    x[0, 0, 0, 0], x[0, 0, 5, 7], x[0, 0, 9, 1] = 20.0, 0.9375, -0.9375
    codes, scales = oracle.quantize_blocks(x, False)
    assert oracle.e4m3_decode(codes[0, 0, 5, 7]) == 20.0 and oracle.e4m3_decode(codes[0, 0, 9, 1]) == -20.0
    assert codes[0, 0, 0, 0] == 0x7E and codes[0, 0, 1, 1] == 0x00
    assert scales[0, 0, 0] == np.float32(20.0 / 448.0)


def test_quantize_hadamard_scale_is_amax_of_orthonormal_transform():
    x = rng.standard_normal((1, 2, 130, 128))
    codes, scales = oracle.quantize_blocks(x, True)
    y = x @ oracle.orthonormal_hadamard(128)
    for j, sl in enumerate((slice(0, 128), slice(128, 130))):
        s = np.abs(y[:, :, sl]).max(axis=(2, 3)) / 448.0
        np.testing.assert_allclose(scales[:, :, j], s, rtol=2.0 ** -23)
    deq = oracle.dequantize_blocks(codes, scales)
    assert np.abs(deq - y).max() <= np.abs(y).max() * 2.0 ** -4


# ---------------------------------------------------------------------------
# FP8 attention emulation
def _exact_codes(shape):
    """Random E4M3 codes whose every 128-row block holds a +-448 element, so
    the block scale is exactly 1 and dequantisation returns the code values."""
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    c = np.where(c >= 0x78, c - 0x40, c).astype(np.uint8)     # keep magnitudes moderate
    c |= (rng.random(shape) < 0.5).astype(np.uint8) << 7
    for j in range(0, shape[2], 128):
        c[:, :, j, 0] = 0x7E
    return c


def test_attention_fp8_without_p_quant_is_plain_attention():
    shape = (1, 2, 200, 128)
    q8, k8, v8 = _exact_codes(shape), _exact_codes(shape), _exact_codes(shape)
    ones = np.ones((1, 2, 2), dtype=np.float32)
    o, lse = oracle.attention_fp8(q8, k8, v8, ones, ones, ones, 1e-3, True, quantize_p=False)
    o_ref, lse_ref = attention(oracle.e4m3_decode(q8), oracle.e4m3_decode(k8), oracle.e4m3_decode(v8), 1e-3, True)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_attention_fp8_p_quant_error_bound():
    # each quantised p is within 2^-4 relative (normal range of 256 p r) or
    # 2^-10 / (256 r) <= 2^-17 absolute (subnormals; r > 1/2), so
    # |O_q - O| <= (2^-4 + N 2^-17 / l) max|V| with l >= 1
    shape = (1, 1, 256, 128)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    v[:, :, 128:] *= 3.0                                   # unequal V-block scales
    q8, qs = oracle.quantize_blocks(q, False)
    k8, ks = oracle.quantize_blocks(k, False)
    v8, vs = oracle.quantize_blocks(v, False)
    o_q, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, 128 ** -0.5, False, quantize_p=True)
    o_n, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, 128 ** -0.5, False, quantize_p=False)
    vmax = np.abs(oracle.dequantize_blocks(v8, vs)).max()
    assert np.abs(o_q - o_n).max() <= (2.0 ** -4 + 256 * 2.0 ** -17) * vmax
    assert np.abs(o_q - o_n).max() > 0
    # in a head with a single V block r = 1: the largest weight of each row (p = 1)
    # is stored exactly
    o_q1, _ = oracle.attention_fp8(q8[:, :, :128], k8[:, :, :128], v8[:, :, :128], qs[:, :, :1], ks[:, :, :1],
                                   vs[:, :, :1], 128 ** -0.5, False, quantize_p=True)
    o_h, _ = oracle.attention_fp8(q8[:, :, :128], k8[:, :, :128], v8[:, :, :128], qs[:, :, :1], ks[:, :, :1],
                                  vs[:, :, :1] * 0.7, 128 ** -0.5, False, quantize_p=True)
    np.testing.assert_allclose(o_h, 0.7 * o_q1, rtol=1e-7, atol=1e-12)   # r depends on the ratio only (float32 scale)


def test_attention_fp8_p_quant_folds_v_block_scales():
    # with unequal V-block scales, P is quantised as E4M3(256 p r)/(256 r) with r
    # the block scale over the head's largest, over the next power of two up: one
    # row against a scalar loop
    shape = (1, 1, 256, 128)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    v[:, :, 128:] *= 3.0                                   # second V block has a larger scale
    q8, qs = oracle.quantize_blocks(q, False)
    k8, ks = oracle.quantize_blocks(k, False)
    v8, vs = oracle.quantize_blocks(v, False)
    o, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, 0.1, False, quantize_p=True)
    qd, kd, vd = (oracle.dequantize_blocks(x, y) for x, y in ((q8, qs), (k8, ks), (v8, vs)))
    i = 77
    srow = 0.1 * (kd[0, 0] @ qd[0, 0, i])
    p = np.exp(srow - srow.max())
    num = np.zeros(128)
    for j in range(256):
        ratio = float(vs[0, 0, j // 128]) / float(vs[0, 0].max())
        r = ratio / 2.0 ** math.ceil(math.log2(ratio))
        pq = float(oracle.e4m3_decode(oracle.e4m3_encode(256.0 * p[j] * r))) / (256.0 * r)
        num += pq * vd[0, 0, j]
    np.testing.assert_allclose(o[0, 0, i], num / p.sum(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("std", [1.0, 1e-2, 1e-3])
def test_attention_fp8_p_quant_with_a_zero_v_block(std):
    # an all-zero V block gets the unit scale; the other blocks' P must keep its
    # relative precision whatever V's magnitude (each block's fold is its own)
    shape = (1, 2, 384, 128)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    v = v * std
    v[:, :, 256:] = 0.0
    q8, qs = oracle.quantize_blocks(q, False)
    k8, ks = oracle.quantize_blocks(k, False)
    v8, vs = oracle.quantize_blocks(v, False)
    assert np.all(vs[:, :, 2] == 1.0)
    o_q, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, 128 ** -0.5, True, quantize_p=True)
    o_n, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, 128 ** -0.5, True, quantize_p=False)
    assert np.linalg.norm(o_q - o_n) / np.linalg.norm(o_n) <= 3e-2


def test_fp8_incoherent_processing_helps_on_channel_outliers():
    # outlier *channels* shared by Q and K (the channel-outlier workload's model,
    # at 1k tokens): the Hadamard transform spreads each outlier channel over all
    # 128 coordinates of a row, and the pages' ~2.6x lower error appears
    from io_aware_exact_16_amd.workloads import WORKLOADS, make_qkv
    w = WORKLOADS["fp8_channels_8k"].with_shape(B=1, H=2, N=1024)
    q, k, v = (t.double().numpy() for t in make_qkv(w))
    o_ref, _ = attention(q, k, v, w.scale, True)
    errs = {}
    for had in (False, True):
        q8, qs = oracle.quantize_blocks(q, had)
        k8, ks = oracle.quantize_blocks(k, had)
        v8, vs = oracle.quantize_blocks(v, False)
        o, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, w.scale, True)
        errs[had] = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    # the pages' claim is the ratio (~2.6x lower error); 8e-2 is a regression bound
    # (the 6e-2 bound is stated for the sparse-outlier workload, not this one)
    assert errs[True] <= 8e-2 and errs[False] >= 2.0 * errs[True], errs


def test_fp8_variants_study():
    # Two FP8 variants measured in emulation (neither is built on the GPU): a
    # Hadamard transform of V undone on O (O = (P (V H)) H, H symmetric and
    # orthonormal), and MX-style power-of-two scales per 32 channels of a token.
    # E4M3 is a floating format: per element its relative error does not depend
    # on the scale (away from subnormals), and an orthogonal transform of V keeps
    # the error energy of P V.  So neither variant lowers the error; the
    # Hadamard transform of Q and K does, by spreading the products of shared
    # outlier channels over all 128 terms of each dot product.
    from oracle.fp8 import e4m3_decode, e4m3_encode, orthonormal_hadamard
    N, d = 512, 128
    g = np.random.default_rng(2024)
    hm = orthonormal_hadamard(d)
    bf = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    q_blk = lambda x: oracle.dequantize_blocks(*oracle.quantize_blocks(x, False))

    def q_mx(x):
        xr = x.reshape(x.shape[:-1] + (d // 32, 32))
        amax = np.abs(xr).max(axis=-1, keepdims=True)
        sc = np.where(amax > 0, 2.0 ** np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 1.0)
        return (e4m3_decode(e4m3_encode(xr / sc)) * sc).reshape(x.shape)

    q, k, v = (g.standard_normal((1, 2, N, d)) for _ in range(3))
    ch = g.choice(d, 4, replace=False)
    v[..., ch] *= 8.0
    q, k, v = bf(q), bf(k), bf(v)
    ref, _ = attention(q, k, v, d ** -0.5, True)
    err = lambda o: np.linalg.norm(o - ref) / np.linalg.norm(ref)
    e_v = err(attention(q, k, q_blk(v), d ** -0.5, True)[0])
    e_hv = err(attention(q, k, q_blk(v @ hm), d ** -0.5, True)[0] @ hm)
    e_mx = err(attention(q, k, q_mx(v), d ** -0.5, True)[0])
    assert 0.9 * e_v <= e_hv and 0.9 * e_v <= e_mx, (e_v, e_hv, e_mx)      # no gain from either variant
    q[..., ch] *= 8.0
    k[..., ch] *= 8.0
    q, k = bf(q), bf(k)
    ref, _ = attention(q, k, v, d ** -0.5, True)
    e_qk = err(attention(q_blk(q), q_blk(k), v, d ** -0.5, True)[0])
    e_hqk = err(attention(q_blk(q @ hm), q_blk(k @ hm), v, d ** -0.5, True)[0])
    e_mxqk = err(attention(q_mx(q), q_mx(k), v, d ** -0.5, True)[0])
    assert e_qk >= 2.0 * e_hqk and e_mxqk >= 0.9 * e_qk, (e_qk, e_hqk, e_mxqk)


def test_fp8_incoherent_processing_helps_at_1k_tokens():
    # outlier inputs as in the FP8 workload, at a short sequence where the
    # Hadamard arm is expected to have the lower error
    N, d, H = 1024, 128, 4
    g = torch.Generator().manual_seed(99)
    q, k, v = (torch.randn(1, H, N, d, generator=g) for _ in range(3))
    for t in (q, k):
        m = torch.rand(t.shape, generator=g) < 0.001
        t[m] = 20.0 * (torch.randint(0, 2, t.shape, generator=g)[m] * 2.0 - 1.0)
    q, k, v = (t.to(torch.bfloat16).double().numpy() for t in (q, k, v))
    scale = d ** -0.5
    o_ref, _ = attention(q, k, v, scale, True)
    errs = {}
    for had in (False, True):
        q8, qs = oracle.quantize_blocks(q, had)
        k8, ks = oracle.quantize_blocks(k, had)
        v8, vs = oracle.quantize_blocks(v, False)
        o, _ = oracle.attention_fp8(q8, k8, v8, qs, ks, vs, scale, True)
        errs[had] = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    assert 0.02 < errs[True] < errs[False] < 0.1, errs
