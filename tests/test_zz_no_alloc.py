"""fa_fwd_decode_noalloc (partial results in the library's static device
scratch; allocates nothing) against fa_fwd_decode (caller workspace): the same
kernels, so the results must be identical bit for bit, and both within the
bf16 tolerance of the float64 oracle.  Two calls in a row, the second on a
smaller input; no device allocation during a call; sizes beyond the scratch
are rejected."""
import numpy as np
import pytest
import torch

import io_aware_exact_16_amd as fa
import oracle
from io_aware_exact_16_amd.workloads import WORKLOADS, custom, make_qkv

from gpu_helpers import compare, f64, log, to_dev

pytestmark = pytest.mark.gpu


def _both(w):
    q, k, v = make_qkv(w)
    qd, kd, vd = to_dev(q, k, v)
    o_ws, lse_ws = fa.attention_decode(qd, kd, vd, causal=w.causal, scale=w.scale)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=qd.device)
    fa.fa_fwd_decode_noalloc(qd, kd, vd, o, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    return (q, k, v), (o, lse), (o_ws, lse_ws)


def _check(w, rows_heads=None):
    log(f"[noalloc] B={w.B} H={w.H} Nq={w.nq} Nk={w.N} d={w.d} causal={w.causal} "
        f"(workspace {fa.fa_fwd_decode_workspace_bytes(w.B, w.H, w.nq, w.N, w.d)} B)")
    (q, k, v), (o, lse), (o_ws, lse_ws) = _both(w)
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    heads = rows_heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    qn, kn, vn = f64(q), f64(k), f64(v)
    qi = oracle.decode_positions(w.nq, w.N)
    for (b, h) in heads:
        o_ref, lse_ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], w.scale,
                                          w.causal, q_index=qi)
        compare(f64(o)[b:b + 1, h:h + 1], f64(lse)[b:b + 1, h:h + 1], o_ref, lse_ref, "bf16")


def test_two_calls_second_smaller(gpu):
    w1 = WORKLOADS["bf16_decode_32k"]                                    # 4 x 32 heads, one query, 32k keys
    w2 = custom(1, 3, 1000, 64, True, "bf16", seed=71, n_q=40)           # smaller: 3 heads, 40 queries, d = 64
    _check(w1, rows_heads=[(0, 0), (1, 7), (3, 31)])
    _check(w2)


def test_non_causal_several_query_groups(gpu):
    _check(custom(2, 4, 3000, 128, False, "bf16", seed=72, n_q=70))


def test_allocates_nothing(gpu):
    w = WORKLOADS["bf16_decode_32k"]
    q, k, v = to_dev(*make_qkv(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.fa_fwd_decode_noalloc(q, k, v, o, lse, w.scale, w.causal)      # first call may load code objects
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        fa.fa_fwd_decode_noalloc(q, k, v, o, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes"


def test_sizes_beyond_the_scratch_are_rejected(gpu):
    B, H, Nq, Nk, d = 4, 32, 64, 8192, 128
    assert fa.fa_fwd_decode_workspace_bytes(B, H, Nq, Nk, d) > fa.binding.FA_DECODE_SCRATCH_BYTES
    q = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(B, H, Nk, d, dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_decode_noalloc(q, k, k.clone(), o, lse, 0.1, True)
    assert e.value.status == -7
