#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: for the bf16/fp32 workloads one fa_fwd call;
for the FP8 workload one fa_qkv_fp8_quant launch (Hadamard transform and
per-block FP8 quantisation of Q and K, V quantised without the transform and
with power-of-two block scales) followed by fa_fwd_fp8; for the decode workload one
fa_fwd_decode call (split-KV kernel + merge); for the backward workload one
fa_bwd call (the dQ kernel, which also forms Delta, then the dK/dV kernel), with the forward's O and
LSE computed once beforehand.  W untimed steps, then K timed
steps bracketed by device synchronisation, timed with HIP events on the stream
the kernels are launched on.  Prints ONE JSON line.

Throughput counts attention FLOPs as 4*B*H*N^2*d (halved when causal) per
step; the decode workload, which is bound by reading K and V, reports its
algorithmic HBM bytes per second against the 8 TB/s HBM peak instead; the
backward workload counts the usual 2.5 times the forward's FLOPs (five
products of the forward's size).  The roofline object reports the dominant
kernel (the attention kernel; for the backward, its whole two-kernel
launch sequence) against the MI355X dense matrix peak of its input type; "traffic" is the HBM
byte count per launch measured with hardware counters (profiles/traffic.json),
or null when that kernel's source changed since the counters were taken.
The cpu_baseline object times the float64 CPU oracle on a bounded sample of
the same workload (whole heads) on this host.

    python bench.py --copy-calibration    # a plain copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # MI355X dense, published
PEAK_HBM_GBS = 8000.0                                         # MI355X HBM3E, published


def kernel_source(w) -> str:
    """Source file of the attention kernel that runs this workload."""
    if w.backward:
        return "attn_bwd.hip"
    if w.n_q > 0:
        return "attn_decode.hip"
    if w.dtype == "bf16":
        return "attn_bf16_pp.hip" if (w.causal and w.d == 128) else "attn_bf16.hip"
    return {"fp8": "attn_fp8.hip", "f32": "attn_f32.hip"}[w.dtype]


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(name: str) -> str:
    """sha256 of a kernel source together with the local headers it includes (recursively)."""
    csrc = os.path.join(ROOT, "io_aware_exact_16_amd", "csrc")
    h, seen, todo = hashlib.sha256(), set(), [os.path.join(csrc, name)]
    while todo:
        path = os.path.normpath(todo.pop(0))
        if path in seen:
            continue
        seen.add(path)
        with open(path, "rb") as f:
            data = f.read()
        h.update(data)
        for line in data.decode(errors="replace").splitlines():
            line = line.strip()
            if line.startswith('#include "'):
                todo.append(os.path.join(os.path.dirname(path), line.split('"')[1]))
    return h.hexdigest()


def measured_traffic(workload: str, kernel_src: str):
    """HBM bytes per launch from profiles/traffic.json, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_sha(kernel_src):
        return None
    return rec.get("traffic_bytes")


def copy_calibration(steps: int) -> None:
    import torch
    n = 256 * 1024 * 1024                      # 1 GiB of float32 read, 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": steps}))


def cpu_baseline(w, q, k, v, budget_s: float, do=None):
    """Time the float64 oracle on whole heads of the workload until about budget_s
    (for the backward workload: oracle.attention_bwd with the upstream gradient do)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    threadpool_limits(len(os.sched_getaffinity(0)), user_api="blas")   # one BLAS thread per usable core
    qn = q.float().numpy().astype(np.float64)
    kn = k.float().numpy().astype(np.float64)
    vn = v.float().numpy().astype(np.float64)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_used = 0, 0.0
    decode = w.n_q > 0
    per_head = (w.hbm_bytes if decode else w.flops) / len(heads)   # bytes (decode) or FLOPs per head
    q_index = oracle.decode_positions(w.nq, w.N) if decode else None
    don = do.float().numpy().astype(np.float64) if do is not None else None
    for (b, h) in heads:
        t0 = time.perf_counter()
        if don is not None:
            oracle.attention_bwd(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1],
                                 don[b:b + 1, h:h + 1], w.scale, w.causal)
        else:
            oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], w.scale, w.causal,
                             q_index=q_index)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= budget_s:
            break
    blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    cores = len(os.sched_getaffinity(0))
    value = done * per_head / t_used / (1e9 if decode else 1e12)
    return {"value": value, "unit": "GB/s" if decode else "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) pairs, full rows, float64, {t_used:.1f} s, "
                      f"{blas} BLAS threads"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps; also brings the GPU clock to its steady state")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.steps)
        return 0

    import io_aware_exact_16_amd as fa
    from io_aware_exact_16_amd.workloads import HEADLINE, WORKLOADS, make_dout, make_qkv

    w = WORKLOADS[args.workload or HEADLINE]
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    stream = torch.cuda.current_stream(dev)

    if w.dtype == "fp8":
        nb = -(-w.N // 128)
        q8, k8, v8 = (torch.empty(qd.shape, dtype=torch.uint8, device=dev) for _ in range(3))
        qs, ks, vs = (torch.empty((w.B, w.H, nb), dtype=torch.float32, device=dev) for _ in range(3))
        o = torch.empty(qd.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        # The quantiser reads 201 MB of bf16 inputs per step, close to the 256 MB
        # last-level cache: successive steps alternate between two resident
        # copies of Q, K, V so that no step finds its inputs already cached.
        sets = [(qd, kd, vd), tuple(t.clone() for t in (qd, kd, vd))]
        turn = [0]

        def step(record=None):
            xq, xk, xv = sets[turn[0]]
            turn[0] ^= 1
            fa.fa_qkv_fp8_quant(xq, xk, xv, q8, k8, v8, qs, ks, vs, fa.FA_QUANT_HADAMARD_QK | fa.FA_QUANT_POW2_SCALE_V)
            if record is not None:
                record[0].record(stream)
            fa.fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, w.scale, w.causal)
            if record is not None:
                record[1].record(stream)
    elif w.backward:                          # backward step: fa_bwd on the forward's O and LSE
        do = make_dout(w)
        dod = do.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        fa.fa_fwd(qd, kd, vd, o, lse, w.scale, w.causal)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)

        def step(record=None):
            if record is not None:
                record[0].record(stream)
            fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, w.scale, w.causal, ws)
            if record is not None:
                record[1].record(stream)
    elif w.n_q > 0:                           # decode step: split-KV kernel + merge, caller-owned workspace
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_fwd_decode_workspace_bytes(w.B, w.H, w.nq, w.N, w.d), dtype=torch.uint8, device=dev)

        def step(record=None):
            if record is not None:
                record[0].record(stream)
            fa.fa_fwd_decode(qd, kd, vd, o, lse, w.scale, w.causal, ws)
            if record is not None:
                record[1].record(stream)
    else:
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

        def step(record=None):
            if record is not None:
                record[0].record(stream)
            fa.fa_fwd(qd, kd, vd, o, lse, w.scale, w.causal)
            if record is not None:
                record[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, events around every attention launch on the launch stream
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(pairs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    kern_ms = [a.elapsed_time(b) for a, b in pairs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = total_ms / args.steps

    dtype = w.dtype
    if w.n_q > 0:
        # a decode step reads K and V once and does little arithmetic per byte: HBM-bound
        metric = "decode attention fwd: algorithmic HBM GB/s (Q,K,V read once, O,LSE written once), 1 GPU"
        unit, work, peak, bound = "GB/s", w.hbm_bytes / 1e9, PEAK_HBM_GBS, "hbm"
    elif w.backward:
        metric = "attention bwd TFLOPS (10*B*H*N^2*d, x1/2 causal: dQ, dK, dV) and % of MFMA peak, 1 GPU"
        unit, work, peak, bound = "TFLOP/s", w.flops / 1e12, PEAK_TFLOPS[dtype], "mfma"
    else:
        metric = "attention fwd TFLOPS (4*B*H*N^2*d, x1/2 causal) and % of MFMA peak, 1 GPU"
        unit, work, peak, bound = "TFLOP/s", w.flops / 1e12, PEAK_TFLOPS[dtype], "mfma"
    value = work / (ms_per_step * 1e-3)
    achieved = work / (kern_avg_ms * 1e-3)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name, kernel_source(w))}
    eprint("[bench] launch times (ms): " + " ".join(f"{t:.4f}" for t in kern_ms))
    eprint(f"[bench] {w.name}: step {ms_per_step:.4f} ms, attention launch(es) avg {kern_avg_ms:.4f} ms "
           f"(min {min(kern_ms):.4f}), {achieved:.1f} {unit} = {100 * achieved / peak:.1f}% of {peak} peak")

    cpu = None
    if not args.no_cpu_baseline:
        eprint("[bench] timing the CPU oracle on a sample of the workload ...")
        cpu = cpu_baseline(w, q, k, v, args.cpu_budget, do=do if w.backward else None)
        eprint(f"[bench] cpu_baseline: {cpu}")

    line = {
        "metric": metric,
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32"}[dtype], "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   **({"Nq": w.nq} if w.n_q > 0 else {}),
                   **({"pass": "backward", "dout_dist": "iid N(0,1)"} if w.backward else {}),
                   "input_dist": f"iid N(0,{w.std}^2)" + (f", {w.outlier_frac:.1%} coords = +-{w.outlier_value:g}"
                                                         if w.outlier_frac else ""),
                   "seed": w.seed},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
