"""Concurrent calls: the library keeps no state between calls (fa_fwd_decode_noalloc aside, whose static
scratch is documented as shared), so host threads that each drive their own stream get exactly the results of
the same calls made one after another.  Five threads run the bf16 forward (persistent and streaming kernels),
the split-KV decode with its own workspace, the backward with its own workspace and the FP8 path (quantiser and
attention) three times each on their own streams, at the same time; every result must equal the serial run's
bit for bit."""
import threading

import pytest
import torch

import io_aware_exact_16_amd as fa
from io_aware_exact_16_amd.workloads import custom, make_dout, make_qkv

from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


def _cases():
    q1, k1, v1 = to_dev(*make_qkv(custom(2, 8, 2048, 128, True, "bf16", seed=501)))
    q2, k2, v2 = to_dev(*make_qkv(custom(2, 8, 2048, 64, False, "bf16", seed=502)))
    wd = custom(2, 8, 8192, 128, True, "bf16", seed=503, n_q=4)
    q3, k3, v3 = to_dev(*make_qkv(wd))
    wb = custom(1, 8, 1024, 128, True, "bf16", seed=504, backward=True)
    q4, k4, v4 = to_dev(*make_qkv(wb))
    do4 = to_dev(make_dout(wb))[0]
    o4, lse4 = fa.attention(q4, k4, v4, causal=True)
    q5, k5, v5 = to_dev(*make_qkv(custom(1, 8, 2048, 128, True, "bf16", seed=505, outlier_frac=0.001)))
    torch.cuda.synchronize()

    def fp8():
        (q8, qs), (k8, ks), (v8, vs) = fa.quant_qkv_fp8(q5, k5, v5)
        return (q8, qs, k8, ks, v8, vs) + fa.attention_fp8(q8, k8, v8, qs, ks, vs, causal=True)

    return [
        ("bf16 causal d=128", lambda: fa.attention(q1, k1, v1, causal=True)),
        ("bf16 non-causal d=64", lambda: fa.attention(q2, k2, v2, causal=False)),
        ("decode", lambda: fa.attention_decode(q3, k3, v3, causal=True)),
        ("backward", lambda: fa.attention_bwd(q4, k4, v4, o4, lse4, do4, causal=True)),
        ("fp8", fp8),
    ]


def test_concurrent_calls_from_threads(gpu):
    cases = _cases()
    ref = []
    for _, run in cases:
        ref.append([t.clone() for t in run()])
    torch.cuda.synchronize()

    results = [None] * len(cases)
    errors = []
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                outs = [cases[i][1]() for _ in range(3)]
            s.synchronize()
            results[i] = outs
        except Exception as e:          # reported by the main thread
            errors.append((cases[i][0], repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for (name, _), want, got in zip(cases, ref, results):
        for rep in got:
            assert len(rep) == len(want)
            for a, b in zip(rep, want):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
        log(f"[concurrency] {name}: 3 concurrent runs equal the serial run")
