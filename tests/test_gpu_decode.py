"""GPU parity of the split-KV decode forward and of the LSE merge against the
fp64 oracle (oracle.attention with decode-step query positions, and
oracle.lse_merge), on seeded inputs: query counts below, at and above one
32-query group, key counts that end inside a tile, at a tile edge and span
many key chunks, both head dimensions, causal and not, and the full-size
decode workload on sampled heads."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import TOL, f64, log, to_dev

pytestmark = pytest.mark.gpu


def _decode_check(B, H, Nq, Nk, d, causal, seed, heads=None, scale=None):
    w = custom(B, H, Nk, d, causal, "bf16", seed=seed, n_q=Nq)
    scale = w.scale if scale is None else scale
    q, k, v = make_qkv(w)
    log(f"[decode] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} scale={scale:.4f}")
    o, lse = fa.attention_decode(*to_dev(q, k, v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    pos = oracle.decode_positions(Nq, Nk)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    qn, kn, vn = f64(q), f64(k), f64(v)
    worst = (0.0, 0.0)
    tol_o, tol_l = TOL["bf16"]
    for (b, h) in heads:
        ro, rl = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], scale, causal,
                                  q_index=pos)
        eo = float(np.abs(o[b:b + 1, h:h + 1] - ro).max())
        el = float((np.abs(lse[b:b + 1, h:h + 1] - rl) / np.maximum(1.0, np.abs(rl))).max())
        worst = (max(worst[0], eo), max(worst[1], el))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert worst[0] <= tol_o and worst[1] <= tol_l, worst
    log(f"  max|dO|={worst[0]:.3g} max rel dLSE={worst[1]:.3g}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 63), (1, 64), (1, 65), (5, 1000), (32, 4096), (33, 3000),
                                   (100, 777), (7, 20000)])
def test_decode_matches_oracle(gpu, Nq, Nk, d, causal):
    _decode_check(2, 3, Nq, Nk, d, causal, seed=Nq * 31 + Nk + d)


def test_decode_long_keys(gpu):
    _decode_check(1, 4, 1, 32768, 128, True, seed=77)


def test_decode_scores_jump_between_tiles(gpu):
    # keys scaled up in steps along the sequence: the reference maximum of each
    # split-KV chunk moves mid-chunk, and by more than 2^128 (exp2 domain) at
    # the last step
    w = custom(1, 2, 3000, 128, True, "bf16", seed=83, n_q=4)
    q, k, v = make_qkv(w)
    g = torch.ones(3000)
    g[900:1800] = 4.0
    g[1800:] = 40.0
    k = (k.float() * g[None, None, :, None]).to(torch.bfloat16)
    o, lse = fa.attention_decode(*to_dev(q, k, v), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), w.scale, True, q_index=oracle.decode_positions(4, 3000))
    tol_o, tol_l = TOL["bf16"]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert float(np.abs(o - ro).max()) <= tol_o
    assert float((np.abs(lse - rl) / np.maximum(1.0, np.abs(rl))).max()) <= tol_l


@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_decode_unusual_scales(gpu, scale):
    _decode_check(1, 2, 3, 2000, 128, True, seed=78, scale=scale)


def test_decode_workload_sampled_heads(gpu):
    w = WORKLOADS["bf16_decode_32k"]
    _decode_check(w.B, w.H, w.nq, w.N, w.d, w.causal, seed=w.seed, heads=[(0, 0), (1, 17), (3, 31)])


def test_decode_equals_prefill_rows(gpu):
    # Nq = Nk: decode and the prefill kernel compute the same attention
    w = custom(1, 2, 300, 128, True, "bf16", seed=79)
    q, k, v = to_dev(*make_qkv(w))
    o1, l1 = fa.attention_decode(q, k, v, causal=True)
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_decode_rejects_small_workspace(gpu):
    w = custom(1, 2, 500, 128, True, "bf16", seed=80, n_q=2)
    q, k, v = to_dev(*make_qkv(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    need = fa.fa_fwd_decode_workspace_bytes(1, 2, 2, 500, 128)
    ws = torch.empty(need - 4, dtype=torch.uint8, device=q.device)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_decode(q, k, v, o, lse, w.scale, True, ws)
    assert e.value.status == -6


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("P,d", [(1, 128), (3, 64), (16, 128)])
def test_lse_merge_matches_oracle(gpu, P, d, out_dtype):
    g = torch.Generator().manual_seed(P * 100 + d)
    B, H, N = 2, 3, 57
    o_parts = torch.randn((P, B, H, N, d), generator=g)
    lse_parts = torch.randn((P, B, H, N), generator=g) * 3.0
    if P > 1:                                  # some rows saw no key in some parts
        lse_parts[0, :, :, ::5] = float("-inf")
    o, lse = fa.lse_merge(o_parts.cuda(), lse_parts.cuda(), out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(o_parts.double().numpy(), lse_parts.double().numpy())
    tol = 1e-5 if out_dtype == torch.float32 else 2 ** -7
    assert float(np.abs(f64(o) - ro).max()) <= tol * max(1.0, float(np.abs(ro).max()))
    assert float(np.abs(f64(lse) - rl).max()) <= 1e-5 * max(1.0, float(np.abs(rl).max()))


def test_lse_merge_all_parts_empty(gpu):
    o_parts = torch.ones((2, 1, 1, 3, 64), device="cuda")
    lse_parts = torch.full((2, 1, 1, 3), float("-inf"), device="cuda")
    o, lse = fa.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == float("-inf"))


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_identical_keys_at_large_size(gpu, noalloc):
    """Four queries against 4M keys of one head (1 GiB per K and V tensor; many split-KV chunks): with one key
    vector repeated, query i (bottom-right aligned) sees Nk - Nq + i + 1 keys with equal weight, so O_i is the
    mean of those values and LSE_i = scale q_i.k + ln(count) (sums in float64 by torch on the device)."""
    Nq, Nk, d = 4, 1 << 22, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    q = torch.randn(1, 1, Nq, d, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 1, 1, d, generator=g, device="cuda").to(torch.bfloat16).expand(1, 1, Nk, d).contiguous()
    v = torch.randn(1, 1, Nk, d, generator=g, device="cuda").to(torch.bfloat16)
    scale = d ** -0.5
    if noalloc:
        o = torch.empty_like(q)
        lse = torch.empty(1, 1, Nq, dtype=torch.float32, device="cuda")
        fa.fa_fwd_decode_noalloc(q, k, v, o, lse, scale, True)
    else:
        o, lse = fa.attention_decode(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    prefix = torch.cumsum(v[0, 0].double(), dim=0)
    err_o = err_l = 0.0
    for i in range(Nq):
        cnt = Nk - Nq + i + 1
        err_o = max(err_o, float((o[0, 0, i].double() - prefix[cnt - 1] / cnt).abs().max()))
        ref_l = scale * float(q[0, 0, i].double() @ k[0, 0, 0].double()) + float(np.log(cnt))
        err_l = max(err_l, abs(float(lse[0, 0, i]) - ref_l) / max(1.0, abs(ref_l)))
    log(f"[decode large] Nk={Nk} noalloc={noalloc}: max|dO|={err_o:.3g} max rel dLSE={err_l:.3g}")
    assert err_o <= TOL["bf16"][0] and err_l <= TOL["bf16"][1]


@pytest.mark.parametrize("causal", [True, False])
def test_ring_attention_shards_on_one_gpu(gpu, causal):
    """The sharded decomposition ring attention would run across devices, emulated on one GPU: the sequence is
    cut into 4 shards; query shard i attends to every key shard j (causal: j < i in full, j = i with the causal
    mask, j > i not at all) with fa_fwd, and fa_lse_merge combines the partial (O, LSE) of each query shard.  The
    result matches the float64 oracle on the whole sequence at the bf16 tolerances."""
    g, B, H, N, d = 4, 1, 4, 2048, 128
    w = custom(B, H, N, d, causal, "bf16", seed=606)
    q, k, v = to_dev(*make_qkv(w))
    n = N // g
    outs, lses = [], []
    for i in range(g):
        qi = q[:, :, i * n:(i + 1) * n].contiguous()
        parts_o = torch.zeros(g, B, H, n, d, dtype=torch.float32, device="cuda")
        parts_l = torch.full((g, B, H, n), float("-inf"), dtype=torch.float32, device="cuda")
        for j in range(g):
            if causal and j > i:
                continue                        # a shard of later keys: an empty part (LSE = -inf)
            kj = k[:, :, j * n:(j + 1) * n].contiguous()
            vj = v[:, :, j * n:(j + 1) * n].contiguous()
            o, lse = fa.attention(qi, kj, vj, causal=causal and j == i, scale=w.scale)
            parts_o[j] = o.float()
            parts_l[j] = lse
        o_i, lse_i = fa.lse_merge(parts_o, parts_l)
        outs.append(o_i)
        lses.append(lse_i)
    torch.cuda.synchronize()
    o_all = torch.cat(outs, dim=2).double().cpu().numpy()
    lse_all = torch.cat(lses, dim=2).double().cpu().numpy()
    o_ref, lse_ref = oracle.attention(f64(q), f64(k), f64(v), w.scale, causal)
    err_o = float(np.abs(o_all - o_ref).max())
    err_l = float((np.abs(lse_all - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max())
    log(f"[ring emulation] {g} shards, causal={causal}: max|dO|={err_o:.3g} max rel dLSE={err_l:.3g}")
    assert err_o <= TOL["bf16"][0] and err_l <= TOL["bf16"][1]
