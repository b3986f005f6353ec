"""CPU oracle for the fused attention path: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Importers allowed: the tests under ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``.  The
HIP library and its Python binding never import or call anything here, and
nothing here imports them: the two implementations share no code.

  attention.attention  -- softmax(scale Q K^T + causal mask) V and LSE, by the
                          definition (full score rows, float64)
  merge.lse_merge      -- combine partial attentions over disjoint key sets
                          through their LSEs; merge.decode_positions gives the
                          query positions of a decode step
  backward.attention_bwd -- dQ, dK, dV of the attention definition for an
                          upstream gradient dO (chain rule, full rows)
  fp8.*                -- Sylvester Hadamard matrix, E4M3 encode/decode from
                          the bit layout, per-block quantisation, and attention
                          on dequantised FP8 operands

Every function is pinned by tests against closed forms, special cases,
brute force and library routines; none is marked "parity unpinned".
"""
from .attention import attention
from .merge import lse_merge, decode_positions
from .backward import attention_bwd
from .fp8 import (sylvester_hadamard, orthonormal_hadamard, e4m3_decode, e4m3_encode,
                  quantize_blocks, quotients, pow2_split, pow2_scale, dequantize_blocks, quantize_mx, dequantize_mx,
                  attention_fp8, E4M3_MAX,
                  BLOCK)

__all__ = ["attention", "attention_bwd", "lse_merge", "decode_positions", "sylvester_hadamard", "orthonormal_hadamard", "e4m3_decode", "e4m3_encode",
           "quantize_blocks", "quotients", "pow2_split", "pow2_scale", "dequantize_blocks", "quantize_mx",
           "dequantize_mx", "attention_fp8", "E4M3_MAX",
           "BLOCK"]
