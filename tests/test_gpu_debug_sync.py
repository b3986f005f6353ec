"""Race check: every entry point gives bitwise-equal results from libfa.so and
from libfa_debugsync.so, the same sources built with FA_DEBUG_SYNC.  That build
waits for all memory operations and all waves at every LDS buffer hand-off (a
tile DMA's issue, a phase boundary), so nothing is in flight while a wave
computes.  The kernels are deterministic, so any difference means that the
regular build reads an LDS buffer before its DMA has landed or overwrites one
that another wave is still reading.  Shapes: the full-size workloads plus
ragged and odd-sized cases (tails of tiles, work lists that are not multiples
of the XCD count, causal and not)."""
import pytest
import torch

import io_aware_exact_16_amd as fa
from io_aware_exact_16_amd import binding
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_dout, make_qkv

from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


def both_builds(run):
    """run() -> tuple of tensors, once per library; the results as CPU byte views."""
    outs = []
    for debug in (False, True):
        if debug:
            with fa.debug_sync_build() as lib:
                assert binding._cur() is lib and lib._name.endswith("libfa_debugsync.so")
                res = run()
        else:
            assert binding._cur()._name.endswith("libfa.so")
            res = run()
        torch.cuda.synchronize()
        outs.append([t.detach().contiguous().view(torch.uint8).cpu() for t in res])
    return outs


def assert_bitwise_equal(name, outs):
    fast, slow = outs
    assert len(fast) == len(slow)
    for i, (a, b) in enumerate(zip(fast, slow)):
        nd = int((a != b).sum())
        assert nd == 0, f"{name}: output {i} differs in {nd} of {a.numel()} bytes between the regular and the debug-sync build"
    log(f"[{name}] {len(fast)} outputs bitwise equal")


FWD_CASES = [
    WORKLOADS["bf16_causal_8k"],                  # persistent ping-pong kernel, full size
    WORKLOADS["bf16_causal_2k"],
    custom(3, 5, 5000, 128, True, "bf16", seed=51),   # 15 heads: one global work list; ragged last block
    custom(1, 2, 300, 128, True, "bf16", seed=52),
    custom(2, 3, 3000, 128, False, "bf16", seed=53),  # streaming kernel, d = 128
    custom(2, 3, 3000, 64, True, "bf16", seed=54),    # streaming kernel, d = 64, causal
    WORKLOADS["bf16_d64_4k"],
    custom(1, 2, 300, 64, False, "f32", seed=55),
]


@pytest.mark.parametrize("w", FWD_CASES, ids=lambda w: w.name)
def test_fwd(gpu, w):
    q, k, v = to_dev(*make_qkv(w))

    def run():
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        return o, lse

    assert_bitwise_equal(w.name, both_builds(run))


@pytest.mark.parametrize("name,B,H,N,causal", [
    ("fp8_causal_8k", 2, 16, 8192, True),
    ("fp8_ragged", 1, 3, 1000, True),
    ("fp8_noncausal", 1, 3, 1000, False),
])
def test_fp8_quantisers_and_attention(gpu, name, B, H, N, causal):
    w = WORKLOADS[name] if name in WORKLOADS else custom(B, H, N, 128, causal, "bf16", seed=N + H)
    q, k, v = to_dev(*make_qkv(w))
    scale = 128 ** -0.5

    def run():
        (q8, qs), (k8, ks), (v8, vs) = fa.quant_qkv_fp8(q, k, v)
        o, lse = fa.attention_fp8(q8, k8, v8, qs, ks, vs, causal=causal, scale=scale)
        qm8, qmx = fa.quant_mx_fp8(q)
        km8, kmx = fa.quant_mx_fp8(k)
        x8, xs = fa.quant_fp8(v, hadamard=False)
        o_mx, lse_mx = fa.attention_fp8_ex(qm8, km8, v8, qs, ks, vs, q_mx=qmx, k_mx=kmx, causal=causal, scale=scale)
        (_, _), (_, _), (vh8, vhs) = fa.quant_qkv_fp8(q, k, v, hadamard_v=True)
        o_vh, lse_vh = fa.attention_fp8_ex(q8, k8, vh8, qs, ks, vhs, causal=causal, scale=scale, v_hadamard=True)
        return (q8, qs, k8, ks, v8, vs, o, lse, qm8, qmx, km8, kmx, x8, xs, o_mx, lse_mx, vh8, vhs, o_vh, lse_vh)

    assert_bitwise_equal(name, both_builds(run))


@pytest.mark.parametrize("w", [WORKLOADS["bf16_decode_32k"], custom(2, 3, 1000, 128, True, "bf16", seed=61, n_q=5)],
                         ids=lambda w: w.name)
def test_decode(gpu, w):
    q, k, v = to_dev(*make_qkv(w))

    def run():
        o, lse = fa.attention_decode(q, k, v, causal=w.causal, scale=w.scale)
        o2 = torch.empty_like(q)
        lse2 = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        fa.fa_fwd_decode_noalloc(q, k, v, o2, lse2, w.scale, w.causal)
        return o, lse, o2, lse2

    assert_bitwise_equal(w.name, both_builds(run))


@pytest.mark.parametrize("w", [WORKLOADS["bf16_causal_8k_bwd"], custom(1, 3, 1000, 128, True, "bf16", seed=71),
                               custom(1, 3, 1000, 64, False, "bf16", seed=72)], ids=lambda w: w.name)
def test_bwd(gpu, w):
    q, k, v = to_dev(*make_qkv(w))
    do = to_dev(make_dout(w))[0]
    o, lse = fa.attention(q, k, v, causal=w.causal, scale=w.scale)   # one forward, shared by both builds

    def run():
        return fa.attention_bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)

    assert_bitwise_equal(w.name, both_builds(run))


# ---------------------------------------------------------------------------
# Grid-order independence: the same heads computed in one call (persistent work
# lists dealt over every compute unit, heads grouped per XCD) and one head per
# call (a different grid, a different workgroup for every item, other items
# resident beside it) must agree bit for bit.  A kernel that let one work item
# see another's LDS contents, or that depended on which workgroup ran an item,
# would differ here.
def per_head(t, b, h):
    return t[b:b + 1, h:h + 1].contiguous()


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 8, 4096, 128, True), (1, 8, 2048, 64, False), (1, 5, 1000, 128, True)])
def test_grid_order_fwd(gpu, B, H, N, d, causal):
    w = custom(B, H, N, d, causal, "bf16", seed=N + d + H)
    q, k, v = to_dev(*make_qkv(w))
    o, lse = fa.attention(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            o1, lse1 = fa.attention(per_head(q, b, h), per_head(k, b, h), per_head(v, b, h), causal=causal,
                                    scale=w.scale)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16), per_head(o, b, h).view(torch.int16)), (b, h)
            assert torch.equal(lse1.view(torch.int32), per_head(lse, b, h).view(torch.int32)), (b, h)
    log(f"[grid order] {B}x{H} heads, N={N}, d={d}, causal={causal}: one call == one call per head")


def test_grid_order_fp8(gpu):
    w = custom(2, 8, 4096, 128, True, "bf16", seed=4242, outlier_frac=0.001)
    q, k, v = to_dev(*make_qkv(w))
    (q8, qs), (k8, ks), (v8, vs) = fa.quant_qkv_fp8(q, k, v)
    o, lse = fa.attention_fp8(q8, k8, v8, qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            (q81, qs1), (k81, ks1), (v81, vs1) = fa.quant_qkv_fp8(per_head(q, b, h), per_head(k, b, h),
                                                                  per_head(v, b, h))
            o1, lse1 = fa.attention_fp8(q81, k81, v81, qs1, ks1, vs1, causal=True)
            torch.cuda.synchronize()
            for x1, x in ((q81, q8), (k81, k8), (v81, v8)):
                assert torch.equal(x1, per_head(x, b, h)), (b, h)
            for s1, s in ((qs1, qs), (ks1, ks), (vs1, vs)):
                assert torch.equal(s1.view(torch.int32), s[b:b + 1, h:h + 1].contiguous().view(torch.int32)), (b, h)
            assert torch.equal(o1.view(torch.int16), per_head(o, b, h).view(torch.int16)), (b, h)
            assert torch.equal(lse1.view(torch.int32), per_head(lse, b, h).view(torch.int32)), (b, h)
    log(f"[grid order] FP8: quantiser and attention, one call == one call per head ({w.B * w.H} heads)")


def test_grid_order_bwd(gpu):
    w = custom(1, 6, 1000, 128, True, "bf16", seed=777, backward=True)
    q, k, v = to_dev(*make_qkv(w))
    do = to_dev(make_dout(w))[0]
    o, lse = fa.attention(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for h in range(w.H):
        g1 = fa.attention_bwd(per_head(q, 0, h), per_head(k, 0, h), per_head(v, 0, h), per_head(o, 0, h),
                              per_head(lse, 0, h), per_head(do, 0, h), causal=True, scale=w.scale)
        torch.cuda.synchronize()
        for x1, x in zip(g1, (dq, dk, dv)):
            assert torch.equal(x1.view(torch.int16), per_head(x, 0, h).view(torch.int16)), h
    log(f"[grid order] backward: one call == one call per head ({w.H} heads)")
