"""Seeded synthetic attention inputs.

This module only draws random numbers: Q, K, V with the shapes and value
distributions of the attention workloads below, rounded to the storage type
the kernels read, and the sparse +-20 outlier substitution used for the FP8
workload.  It holds none of the attention or quantisation arithmetic, so both
the CPU oracle's tests and the GPU path can take their inputs from it.

Draw order for one workload (fixed, so every consumer sees identical tensors):
Q, K, V from N(0, std^2) in float32; then, for the sparse-outlier workload
only, a Bernoulli mask for Q, the signs for Q, a Bernoulli mask for K and the
signs for K (selected coordinates are replaced, not added to, by
+-outlier_value); then, for the channel-outlier workload only, a random
permutation of the d channels whose first channel_outliers entries are the
channels multiplied by channel_scale in both Q and K.
The float32 draws are finally rounded (round to nearest even) to bfloat16
for every workload whose source precision is bf16; the fp32 workload keeps
the float32 draws.  A backward workload's upstream gradient dO comes from
make_dout, a generator of its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str              # "f32" | "bf16" | "fp8" (fp8: bf16 source, quantised on the GPU)
    seed: int
    std: float = 1.0
    outlier_frac: float = 0.0
    outlier_value: float = 20.0
    n_q: int = 0            # decode shape: n_q queries (the last n_q of N tokens) against N keys; 0 = N queries
    backward: bool = False  # the workload is the backward pass (gradients for an upstream dO)
    channel_outliers: int = 0     # Q and K: this many channels (the same for every token and head) scaled up
    channel_scale: float = 1.0    # ... by this factor

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def nq(self) -> int:
        return self.n_q if self.n_q > 0 else self.N

    @property
    def flops(self) -> float:
        """Attention FLOPs counted the usual way: 4*B*H*N^2*d, halved when causal.  For a
        decode shape: 4*d per visible (query, key) pair."""
        if self.backward:         # five products of the forward's size instead of two
            return 2.5 * self.with_shape(backward=False).flops
        if self.n_q > 0:
            pairs = self.n_q * self.N - (self.n_q * (self.n_q - 1) // 2 if self.causal else 0)
            return 4.0 * self.B * self.H * pairs * self.d
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    @property
    def hbm_bytes(self) -> float:
        """Algorithmic HBM traffic of one forward: Q, K, V read once, O and LSE written once."""
        es = 4 if self.dtype == "f32" else 2
        return float(self.B * self.H * ((2 * self.N + 2 * self.nq) * self.d * es + 4 * self.nq))

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads: a tiny fp32 case, bf16 causal and non-causal cases, the FP8
# causal case with outliers, its bf16 twin at the same 8k shape, a 32k-token
# layer shaped like a 7B model's attention (32 heads of 128), and one decode
# step (one new token per sequence) against that layer's 32k-token keys.
WORKLOADS = {
    "f32_tiny": Workload("f32_tiny", 1, 1, 128, 64, False, "f32", seed=1001),
    "bf16_causal_2k": Workload("bf16_causal_2k", 4, 16, 2048, 128, True, "bf16", seed=1002),
    "bf16_d64_4k": Workload("bf16_d64_4k", 8, 32, 4096, 64, False, "bf16", seed=1003),
    "fp8_causal_8k": Workload("fp8_causal_8k", 2, 16, 8192, 128, True, "fp8", seed=1004,
                              outlier_frac=0.001, outlier_value=20.0),
    "bf16_causal_8k": Workload("bf16_causal_8k", 2, 16, 8192, 128, True, "bf16", seed=1006),
    "bf16_causal_32k": Workload("bf16_causal_32k", 1, 32, 32768, 128, True, "bf16", seed=1005, std=0.5),
    # one decode step of four 32k-token sequences through the 7B-shaped layer
    "bf16_decode_32k": Workload("bf16_decode_32k", 4, 32, 32768, 128, True, "bf16", seed=1007, n_q=1),
    # the FP8 case with structured outliers: 4 channels of Q and K (shared, as outlier features of a model's
    # hidden state would be) carry 8x the standard deviation of the others
    "fp8_channels_8k": Workload("fp8_channels_8k", 2, 16, 8192, 128, True, "fp8", seed=1009, channel_outliers=4,
                                channel_scale=8.0),
    # the backward pass at the headline 8k shape (dO drawn by make_dout)
    "bf16_causal_8k_bwd": Workload("bf16_causal_8k_bwd", 2, 16, 8192, 128, True, "bf16", seed=1008, backward=True),
}
# The 8k-token causal bf16 workload is the headline throughput point.
HEADLINE = "bf16_causal_8k"


def _outliers(x: torch.Tensor, g: torch.Generator, frac: float, value: float) -> torch.Tensor:
    mask = torch.rand(x.shape, generator=g) < frac
    sign = torch.randint(0, 2, x.shape, generator=g, dtype=torch.int8).to(torch.float32) * 2.0 - 1.0
    return torch.where(mask, sign * value, x)


def make_qkv(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous CPU tensors: q [B, H, nq, d], k and v [B, H, N, d].

    dtype float32 for the fp32 workload, bfloat16 otherwise (the FP8 workload's
    tensors are the bf16 source values that the quantiser reads).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn((w.B, w.H, w.nq, w.d), generator=g, dtype=torch.float32) * w.std
    k = torch.randn(shape, generator=g, dtype=torch.float32) * w.std
    v = torch.randn(shape, generator=g, dtype=torch.float32) * w.std
    if w.outlier_frac > 0.0:
        q = _outliers(q, g, w.outlier_frac, w.outlier_value)
        k = _outliers(k, g, w.outlier_frac, w.outlier_value)
    if w.channel_outliers > 0:
        ch = torch.randperm(w.d, generator=g)[:w.channel_outliers]
        q[..., ch] *= w.channel_scale
        k[..., ch] *= w.channel_scale
    if w.dtype in ("bf16", "fp8"):
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_dout(w: Workload, seed: int | None = None):
    """The upstream gradient dO for a backward workload: N(0, 1) of O's shape
    [B, H, nq, d], rounded to bfloat16, from a generator of its own (seed + 7919)
    so that Q, K, V are the same tensors make_qkv returns."""
    g = torch.Generator(device="cpu")
    g.manual_seed((w.seed if seed is None else seed) + 7919)
    do = torch.randn((w.B, w.H, w.nq, w.d), generator=g, dtype=torch.float32)
    return do.to(torch.bfloat16).contiguous()


def custom(B: int, H: int, N: int, d: int, causal: bool, dtype: str = "bf16", seed: int = 7,
           std: float = 1.0, outlier_frac: float = 0.0, n_q: int = 0, backward: bool = False) -> Workload:
    """An ad-hoc workload (edge shapes in tests) drawn by the same recipe."""
    return Workload(f"custom_{B}x{H}x{N}x{d}", B, H, N, d, causal, dtype, seed=seed, std=std,
                    outlier_frac=outlier_frac, n_q=n_q, backward=backward)
