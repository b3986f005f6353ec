"""GPU parity of the fused attention kernels (bf16 and fp32) against the fp64
oracle, on seeded inputs: edge shapes, every workload at full size (whole
output where the oracle is fast, sampled rows otherwise), the special cases the
method has, and the API contract (no allocation, determinism, streams)."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import TOL, compare, compare_sampled, f64, log, run_attention, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _check_full(w, kind):
    q, k, v = make_qkv(w)
    log(f"[{w.name}] B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    o, lse = run_attention(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention(f64(q), f64(k), f64(v), w.scale, w.causal)
    return compare(o, lse, o_ref, lse_ref, kind)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 1000])
def test_bf16_edge_shapes(gpu, N, d, causal):
    _check_full(custom(1, 2, N, d, causal, "bf16", seed=N * 7 + d), "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 5, 64, 100, 128, 300])
def test_f32_edge_shapes(gpu, N, d, causal):
    _check_full(custom(1, 2, N, d, causal, "f32", seed=N * 5 + d), "f32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_several_tiles_ragged(gpu, d, causal):
    # 3000 = 23 * 128 + 56: many query blocks and key tiles plus a ragged tail
    _check_full(custom(2, 3, 3000, d, causal, "bf16", seed=3000 + d), "bf16")


def test_workload_f32_tiny(gpu):
    _check_full(WORKLOADS["f32_tiny"], "f32")


def test_workload_bf16_causal_2k_full(gpu):
    e = _check_full(WORKLOADS["bf16_causal_2k"], "bf16")
    log(f"  max|dO|={e[0]:.3g} max rel dLSE={e[1]:.3g}")


@pytest.mark.parametrize("name", ["bf16_d64_4k", "bf16_causal_8k"])
def test_workload_whole_output(gpu, name):
    """Every head and every row of the non-causal d = 64 workload and of the 8k-token
    causal headline workload against the float64 oracle."""
    w = WORKLOADS[name]
    log(f"[{name}] whole output, {w.B * w.H} heads")
    e = _check_full(w, "bf16")
    log(f"  max|dO|={e[0]:.3g} max rel dLSE={e[1]:.3g}")


@pytest.mark.parametrize("name", ["bf16_causal_32k"])
def test_workload_sampled_rows(gpu, name):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    log(f"[{name}] B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} (sampled rows)")
    o, lse = run_attention(q, k, v, w.causal, w.scale)
    heads = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2)]
    e = compare_sampled(q, k, v, o, lse, w.causal, w.scale, "bf16", heads, sample_rows(w.N, 96, 11))
    # properties that hold for every row: finite, and |O| within the range of V
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.abs(o).max() <= np.abs(f64(v)).max() * (1 + 2 ** -7)
    log(f"  max|dO|={e[0]:.3g} max rel dLSE={e[1]:.3g}")


@pytest.mark.parametrize("B,H,N,scale_mult", [
    (2, 16, 8192, 1.0),    # 32 heads x 32 blocks of 256 rows: 4 items per persistent workgroup, heads grouped per XCD
    (3, 5, 5000, 1.0),     # 15 heads (not a multiple of 8): global item order; 5000 % 256 = 136: odd tile count
    (1, 8, 1024, -1.0),    # fewer items than compute units; negative scale
])
def test_causal_d128_every_work_item(gpu, B, H, N, scale_mult):
    """Causal d = 128 runs the persistent kernel: rows from every 256-row block of every head."""
    w = custom(B, H, N, 128, True, "bf16", seed=N + 31 * H + B)
    scale = w.scale * scale_mult
    q, k, v = make_qkv(w)
    log(f"[persistent] B={B} H={H} N={N} scale={scale:.4f}")
    o, lse = run_attention(q, k, v, True, scale)
    rows = np.unique(np.array([r for b0 in range(0, N, 256) for r in (b0, b0 + 37, b0 + 128, b0 + 255)] + [N - 1]))
    rows = rows[rows < N]
    heads = [(b, h) for b in range(B) for h in range(H)]
    e = compare_sampled(q, k, v, o, lse, True, scale, "bf16", heads, rows)
    log(f"  {len(heads)} heads x {len(rows)} rows: max|dO|={e[0]:.3g} max rel dLSE={e[1]:.3g}")


def test_long_context_allocates_nothing(gpu):
    w = WORKLOADS["bf16_causal_32k"]
    q, k, v = to_dev(*make_qkv(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)        # first call may load code objects
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes during the call"


# ---------------------------------------------------------------------------
# special cases of the method, through the GPU path
def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(gpu, causal):
    g = torch.Generator().manual_seed(5)
    N, d = 300, 128
    q = torch.randn(1, 2, N, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, 1, d, generator=g).expand(1, 2, N, d).contiguous().to(torch.bfloat16)
    v = torch.randn(1, 2, N, d, generator=g).to(torch.bfloat16)
    o, lse = run_attention(q, k, v, causal, d ** -0.5)
    vn = f64(v)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vn, axis=2) / cnt[:, None] if causal else np.broadcast_to(vn.mean(axis=2, keepdims=True), vn.shape)
    assert np.abs(o - mean).max() <= 2e-2
    ref_lse = d ** -0.5 * np.einsum("bhnd,bhd->bhn", f64(q), f64(k)[:, :, 0]) + np.log(cnt)
    assert (np.abs(lse - ref_lse) / np.maximum(1, np.abs(ref_lse))).max() <= 1e-3


@pytest.mark.parametrize("N,d,causal", [(1 << 22, 128, True), (1 << 21, 64, False)])
def test_identical_keys_at_large_sizes(gpu, N, d, causal):
    """One head of 4M (2M) tokens: every K, V and O tensor of the head is 1 GiB (256 MiB), so tile and row byte
    offsets reach the top of the 32-bit range the kernels address a head with.  With one key vector repeated,
    the closed form holds at any size: O_i is the mean of the values the row sees and LSE_i = scale q_i.k + ln(count);
    it is checked on sampled rows (reductions in float64 by torch on the device, not by the library)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(N + d)
    q = torch.randn(1, 1, N, d, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 1, 1, d, generator=g, device="cuda").to(torch.bfloat16).expand(1, 1, N, d).contiguous()
    v = torch.randn(1, 1, N, d, generator=g, device="cuda").to(torch.bfloat16)
    scale = d ** -0.5
    log(f"[large] N={N} d={d} causal={causal}: {q.numel() * 2 / 2**20:.0f} MiB per tensor")
    o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 63, 64, 255, 256, 65535, 65536, N // 2 - 1, N // 2, N - 257, N - 2, N - 1}
                  | set(torch.randint(0, N, (8,), generator=torch.Generator().manual_seed(N)).tolist()))
    vd = v[0, 0].double()
    k0 = k[0, 0, 0].double()
    full_mean = vd.mean(dim=0)
    err_o = err_l = 0.0
    for i in rows:
        cnt = i + 1 if causal else N
        mean = vd[:cnt].mean(dim=0) if causal else full_mean
        err_o = max(err_o, float((o[0, 0, i].double() - mean).abs().max()))
        ref_l = scale * float(q[0, 0, i].double() @ k0) + float(np.log(cnt))
        err_l = max(err_l, abs(float(lse[0, 0, i]) - ref_l) / max(1.0, abs(ref_l)))
    log(f"  {len(rows)} rows: max|dO|={err_o:.3g} max rel dLSE={err_l:.3g}")
    assert err_o <= 2e-2 and err_l <= 1e-3
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("d", [64, 128])
def test_single_token_returns_v(gpu, d):
    g = torch.Generator().manual_seed(6)
    q, k, v = (torch.randn(3, 4, 1, d, generator=g).to(torch.bfloat16) for _ in range(3))
    for causal in (False, True):
        o, lse = run_attention(q, k, v, causal, 0.3)
        np.testing.assert_array_equal(o, f64(v))
        np.testing.assert_allclose(lse, 0.3 * np.einsum("bhnd,bhnd->bhn", f64(q), f64(k)), rtol=1e-5, atol=1e-5)


def test_causal_first_row_is_v0(gpu):
    q, k, v = make_qkv(custom(2, 3, 777, 128, True, "bf16", seed=8))
    o, lse = run_attention(q, k, v, True, 128 ** -0.5)
    np.testing.assert_array_equal(o[:, :, 0], f64(v)[:, :, 0])


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0])
def test_unusual_scales(gpu, scale):
    # scale 0 is uniform attention; a negative scale flips the scores; a large one sharpens them
    for causal in (False, True):
        q, k, v = make_qkv(custom(1, 2, 333, 64, causal, "bf16", seed=9))
        o, lse = run_attention(q, k, v, causal, scale)
        o_ref, lse_ref = oracle.attention(f64(q), f64(k), f64(v), scale, causal)
        compare(o, lse, o_ref, lse_ref, "bf16")


def _jumping_keys(N, d, seed, gain):
    """Q, K, V ~ N(0,1) with the keys scaled up in steps along the sequence
    (x1 up to key 299, x4 up to 699, x gain after), so that the row maxima of
    the scaled scores jump between key tiles instead of settling early."""
    q, k, v = make_qkv(custom(1, 2, N, d, False, "bf16", seed=seed))
    g = torch.ones(N)
    g[300:700] = 4.0
    g[700:] = gain
    k = (k.float() * g[None, None, :, None]).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("gain", [16.0, 40.0])
def test_scores_jump_between_tiles(gpu, d, causal, gain):
    # The softmax keeps a reference maximum that it moves only when a tile's
    # p would leave its range.  Keys that grow along the sequence move it in
    # the middle of rows; with gain 40 the later scores exceed the early
    # reference by more than 2^128 in the exp2 domain, so p computed against
    # the old reference would overflow before the reference moves.
    q, k, v = _jumping_keys(1500, d, 21 + d, gain)
    scale = d ** -0.5
    o, lse = run_attention(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(f64(q), f64(k), f64(v), scale, causal)
    compare(o, lse, o_ref, lse_ref, "bf16")


def test_incoherent_inputs_match_oracle(gpu):
    # Q H and K H (normalised Hadamard) as inputs: same parity bar
    q, k, v = make_qkv(custom(1, 2, 1000, 128, True, "bf16", seed=10, outlier_frac=0.001))
    h = torch.from_numpy(oracle.orthonormal_hadamard(128)).float()
    qh, kh = (q.float() @ h).to(torch.bfloat16), (k.float() @ h).to(torch.bfloat16)
    o, lse = run_attention(qh, kh, v, True, 128 ** -0.5)
    o_ref, lse_ref = oracle.attention(f64(qh), f64(kh), f64(v), 128 ** -0.5, True)
    compare(o, lse, o_ref, lse_ref, "bf16")


# ---------------------------------------------------------------------------
# API contract
def test_deterministic(gpu):
    q, k, v = to_dev(*make_qkv(custom(2, 4, 2500, 128, True, "bf16", seed=12)))
    o1, l1 = fa.attention(q, k, v, causal=True)
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_runs_on_the_callers_stream(gpu):
    q, k, v = to_dev(*make_qkv(custom(1, 2, 1024, 128, False, "bf16", seed=13)))
    ref_o, ref_l = fa.attention(q, k, v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = fa.attention(q, k, v)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_error_status_with_device_tensors(gpu):
    q = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.attention(q, q.clone(), q.clone())
    assert e.value.status == -4
    q = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 16), 7.0, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(q, q, q, o, lse, float("nan"), False)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)      # outputs untouched on error


# ---------------------------------------------------------------------------
# NaN in the inputs is not an error: it reaches exactly the outputs that depend on it
@pytest.mark.parametrize("d,causal", [(128, True), (64, False), (128, False)])
def test_nan_reaches_only_dependent_outputs(gpu, d, causal):
    N, jk, jq, jv, cv = 300, 150, 77, 200, 5
    w = custom(1, 2, N, d, causal, "bf16", seed=400 + d)
    q, k, v = make_qkv(w)
    nan = float("nan")
    q[0, 0, jq, 3] = nan          # one element of query row jq, head 0
    k[0, 1, jk, 7] = nan          # one element of key jk, head 1
    v[0, 0, jv, cv] = nan         # one element of value jv, column cv, head 0
    o, lse = run_attention(q, k, v, causal, w.scale)
    qc, kc, vc = q.clone(), k.clone(), v.clone()
    qc[0, 0, jq, 3] = 0.0
    kc[0, 1, jk, 7] = 0.0
    vc[0, 0, jv, cv] = 0.0
    o_ref, lse_ref = oracle.attention(f64(qc), f64(kc), f64(vc), w.scale, causal)
    rows = np.arange(N)
    # rows that see value jv, and (causal) the rows of its 64-key tile that the mask hides from it: their
    # zero weight times the NaN in the matrix product
    sees = (rows >= 64 * (jv // 64)) if causal else np.ones(N, bool)
    sees_k = (rows >= jk) if causal else np.ones(N, bool)               # rows that see key jk
    nan_o = np.zeros(o.shape, bool)
    nan_l = np.zeros(lse.shape, bool)
    nan_o[0, 0, jq, :] = True                                           # a NaN query: its whole row
    nan_l[0, 0, jq] = True
    nan_o[0, 0, sees, cv] = True                                        # a NaN value: its column, in rows that see it
    nan_o[0, 1, sees_k, :] = True                                       # a NaN key: whole rows that see it
    nan_l[0, 1, sees_k] = True
    assert np.isnan(o[nan_o]).all() and np.isnan(lse[nan_l]).all()
    assert np.isfinite(o[~nan_o]).all() and np.isfinite(lse[~nan_l]).all()
    assert np.abs(o[~nan_o] - o_ref[~nan_o]).max() <= TOL["bf16"][0]
    assert (np.abs(lse[~nan_l] - lse_ref[~nan_l]) / np.maximum(1, np.abs(lse_ref[~nan_l]))).max() <= TOL["bf16"][1]
