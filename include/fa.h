/*
 * fa.h -- C ABI of the fused exact-attention forward library (libfa.so), gfx950.
 *
 * What is computed.  Per (batch b, head h) the library returns
 *     O = softmax(scale * Q K^T + mask) V      and      LSE_i = ln sum_j exp(scale * q_i . k_j)
 * (the sum over the keys row i may see), computed tile by tile with a running
 * (online) softmax so that the N x N score matrix never exists in memory:
 *   - "Flash Attention" glossary page (news.hamidun.com), second paragraph:
 *     tiles small enough for on-chip memory, a numerically stable online
 *     softmax accumulating partial results, the full matrix never written to
 *     HBM, memory linear in N;
 *   - "FlashAttention-3 (PT)", section "FlashAttention e FlashAttention-2":
 *     tiling in on-chip SRAM and fusion of the matmuls and softmax into one
 *     kernel, no intermediate results in global memory.
 * The FP8 variant follows "FlashAttention-3 (PT)", section "Inovacoes
 * tecnicas", item 3: Q and K are multiplied by an orthogonal (Hadamard)
 * matrix before FP8 quantisation ("incoherent processing"), which leaves
 * Q K^T unchanged.
 *
 * Conventions shared by every entry point.
 *   Layout:   Q, K, V, O are [B, H, N, d] contiguous row-major (d fastest);
 *             LSE is [B, H, N] float32; FP8 tensors are E4M3 bytes (OCP "fn"
 *             variant: bias 7, max 448, no infinities) in the same layout;
 *             FP8 block scales are [B, H, ceil(N/128)] float32, one per
 *             (b, h, block of 128 consecutive tokens).
 *   Causal:   square, top-left aligned: key j is visible to query i iff j <= i.
 *   Pointers: all tensor pointers are DEVICE pointers owned by the caller.
 *             Inputs are only read.  Outputs must not overlap inputs or each
 *             other (identical pointers are rejected; partial overlap is the
 *             caller's error and is not detected).
 *   Stream:   `stream` is a hipStream_t (NULL = the default stream).  Work is
 *             enqueued asynchronously on it; the call never synchronises.
 *             Results are valid once the caller has synchronised that stream.
 *   Memory:   the library allocates nothing; concurrent calls from several host
 *             threads are safe (fa_fwd_decode and fa_bwd take their scratch space
 *             from the caller), except fa_fwd_decode_noalloc, whose static device
 *             scratch is shared by all its calls on one GPU.
 *   Errors:   arguments are checked before any HIP call.  On a negative status
 *             nothing has been enqueued and the outputs are untouched, except
 *             FA_ERR_LAUNCH, which reports a failed kernel launch.  Device
 *             faults surface at the caller's next synchronisation.  NaN or Inf
 *             in the inputs is not an error; it propagates to the outputs
 *             that depend on it (a NaN in Q or K: O and LSE of the rows whose
 *             scores it enters; in V: that column of O in the rows that see
 *             the key).  A non-finite V element also reaches that column in
 *             the rows of its 64-key tile that the causal mask hides from it
 *             (their zero weight times the value).  In fa_bwd a non-finite
 *             input can likewise reach the gradients of the other rows and
 *             keys of its tiles.  In the FP8 quantisers a
 *             NaN element leaves its block's scale to the other elements and
 *             becomes a NaN code (with the transform: its token's whole row
 *             of codes).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype {
  FA_F32 = 0,       /* float32 tensors */
  FA_BF16 = 1,      /* bfloat16 tensors */
  FA_FP8_E4M3 = 2   /* E4M3 bytes (only through fa_fwd_fp8 / fa_hadamard_fp8_quant) */
};

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,         /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,        /* B, H or N < 1, or a size exceeds the limits: the grid, 64-bit offsets,
                               and N * d * 4 < 2^32 (one head's K or V is addressed with 32-bit offsets) */
  FA_ERR_DTYPE = -3,        /* unknown dtype code, or FA_FP8_E4M3 passed to fa_fwd */
  FA_ERR_UNSUPPORTED = -4,  /* head dimension not supported for this dtype/entry point */
  FA_ERR_LAUNCH = -5,       /* the kernel launch failed (hipGetLastError) */
  FA_ERR_ARG = -6,          /* non-finite scale, flag not 0/1, an output aliasing an input, or a
                               workspace smaller than required */
  FA_ERR_SCRATCH = -7       /* fa_fwd_decode_noalloc: the sizes need more than its static scratch */
};

/*
 * fa_fwd -- fused attention forward in float32 or bfloat16: O = softmax(scale
 * Q K^T + mask) V and its LSE, tile by tile with the online softmax, the score
 * matrix never in HBM ("Flash Attention" glossary page, second paragraph;
 * "FlashAttention-3 (PT)", section "FlashAttention e FlashAttention-2").
 *   q, k, v : [B,H,N,d] inputs, dtype `dtype` (FA_F32 or FA_BF16).
 *   o       : [B,H,N,d] output, same dtype as the inputs.
 *   lse     : [B,H,N] float32 output, natural-log units of the scaled scores.
 *   B, H, N : batch, heads, tokens (>= 1 each); d : head dimension, 64 or 128.
 *   scale   : any finite float multiplying Q K^T (usually 1/sqrt(d)).
 *   causal  : 0 or 1.
 * bf16 runs the products on bf16 matrix cores with float32 accumulation and a
 * float32 softmax; f32 runs entirely in float32 arithmetic.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_fp8 -- fused attention forward on per-block-scaled E4M3 operands
 * ("FlashAttention-3 (PT)", section "Inovacoes tecnicas", item 3: low-precision
 * FP8 matrix products, with Q and K made incoherent by an orthogonal
 * transform; section "Novos recursos de hardware": FP8 doubles the matrix
 * throughput).
 *   q8, k8, v8        : [B,H,N,128] E4M3 bytes (typically from fa_qkv_fp8_quant,
 *                       with the Hadamard matrix applied to q and k and not to v).
 *   q_scale, k_scale,
 *   v_scale           : [B,H,ceil(N/128)] float32 block scales; element value = code * scale.
 *   o                 : [B,H,N,128] bfloat16 output;  lse : [B,H,N] float32 output.
 *   d                 : must be 128.
 * S = scale * (q8 k8^T) runs on FP8 matrix cores with the two block scales
 * folded into the softmax exponent.  P is quantised to E4M3 as 128 p r, where
 * r in (1/2, 1] is the mantissa of the key block's V scale over the head's
 * largest, whose power of two goes into the matrix instruction's E8M0 scale of
 * the V operand (r = 1 everywhere when the V scales are powers of two, as
 * fa_qkv_fp8_quant's FA_QUANT_POW2_SCALE_V makes them); 1/128 and the largest
 * V scale are undone in float32.  The running reference maximum moves only when
 * a tile's largest score exceeds it by more than 1.8 in the exp2 domain, so
 * every p <= 2^1.8 and 128 p r <= 445.7 stays in E4M3's range (448).  (The dtype argument of fa_fwd has no room for
 * the block scales, hence a separate entry point.)
 */
int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
               const float* q_scale, const float* k_scale, const float* v_scale,
               void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Flags of fa_fwd_fp8_ex. */
enum fa_fp8_flags {
  FA_FP8_V_HADAMARD = 1   /* v8 holds the codes of V H / sqrt(128) (fa_qkv_fp8_quant with
                             FA_QUANT_HADAMARD_V); the output is transformed back, O = O' H / sqrt(128) */
};

/*
 * fa_fwd_fp8_ex -- fa_fwd_fp8 with two variants of the FP8 path (same passage):
 *   q_mx, k_mx : NULL, or both [B,H,N,4] E8M0 codes (fa_mx_fp8_quant): one
 *                power-of-two scale 2^(code - 127) per 32 coordinates of each
 *                token, multiplying q8 / k8 on top of their block scales (pass
 *                block scales of 1 for pure MX operands); the matrix
 *                instruction applies them per lane in S = Q K^T.  One of the two
 *                NULL: FA_ERR_ARG.
 *   flags      : 0 or FA_FP8_V_HADAMARD (other bits: FA_ERR_ARG).
 * Everything else as fa_fwd_fp8, which equals fa_fwd_fp8_ex(..., NULL, NULL, ..., 0).
 */
int fa_fwd_fp8_ex(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  const uint8_t* q_mx, const uint8_t* k_mx, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal, int flags, void* stream);

/*
 * fa_hadamard_fp8_quant -- incoherent processing and per-block FP8 quantisation
 * ("FlashAttention-3 (PT)", section "Inovacoes tecnicas", item 3: Q and K are
 * multiplied by an orthogonal matrix, for example a Hadamard matrix, before
 * FP8 quantisation, which spreads outliers; the matrix cancels in Q K^T).
 *   x        : [B,H,N,d] input, in_dtype FA_BF16 or FA_F32.
 *   x8       : [B,H,N,d] E4M3 output bytes.
 *   scales   : [B,H,ceil(N/128)] float32 output block scales.
 *   hadamard : 1 = first multiply every row by the Sylvester Hadamard matrix of
 *              order d divided by sqrt(d) (d must be 128); 0 = quantise x as is
 *              (any d in {64,128}).
 * Per block of 128 tokens (fewer in the last block): amax = max |y| over the
 * block, s = amax / 448 (s = 1 when amax = 0), code = E4M3 round-to-nearest-even
 * of y / s.  The transform and the quotient are formed in float32 (butterfly
 * error at most log2(d) 2^-24 times the row's l1 norm), so a quotient that lies
 * within that error of an E4M3 rounding boundary may go to either neighbour;
 * all other codes are the correctly rounded E4M3 of y / s.  One head of x must
 * be below 4 GiB (N d sizeof(element) < 2^32), else FA_ERR_SHAPE.
 */
int fa_hadamard_fp8_quant(const void* x, int in_dtype, uint8_t* x8, float* scales,
                          int B, int H, int N, int d, int hadamard, void* stream);

/*
 * fa_mx_fp8_quant -- MX-style FP8 quantisation (a variant of incoherent
 * processing's quantisation step, same passage as fa_hadamard_fp8_quant): every
 * group of 32 consecutive coordinates of a token row shares one power-of-two
 * scale X = 2^E, E = ceil(log2(amax / 448)) clamped to [-127, 127], so the
 * group's largest magnitude lands in (224, 448] and nothing clips; code =
 * E4M3 round-to-nearest-even of y / X.
 *   x        : [B,H,N,128] input, in_dtype FA_BF16 or FA_F32.
 *   x8       : [B,H,N,128] E4M3 output bytes.
 *   e8m0     : [B,H,N,4] output, E + 127 per group (0 for an all-zero group,
 *              whose codes are zero); the layout fa_fwd_fp8_ex reads.
 *   hadamard : 1 = first the normalised Hadamard transform, as in
 *              fa_hadamard_fp8_quant (then E and the quotient are formed in
 *              float32 from the float32 transform: codes within that error of a
 *              rounding boundary may go to either neighbour); 0 = none, and
 *              y / X is exact.
 */
int fa_mx_fp8_quant(const void* x, int in_dtype, uint8_t* x8, uint8_t* e8m0, int B, int H, int N, int d,
                    int hadamard, void* stream);

/* Flags of fa_qkv_fp8_quant. */
enum fa_quant_flags {
  FA_QUANT_HADAMARD_QK = 1,   /* Q and K through the normalised Hadamard transform first */
  FA_QUANT_HADAMARD_V = 2,    /* V through it too */
  FA_QUANT_POW2_SCALE_V = 4   /* V's block scale is the power of two 2^ceil(log2(amax / 448)) (at least
                                 2^-126): the E8M0 form, which fa_fwd_fp8 applies exactly in its matrix
                                 instruction, so the V scale never rounds inside P */
};

/*
 * fa_qkv_fp8_quant -- per-block FP8 quantisation of Q, K and V of one attention
 * call in a single launch (same passage as fa_hadamard_fp8_quant).
 *   q, k, v        : [B,H,N,128] inputs, in_dtype FA_BF16 or FA_F32.
 *   q8, k8, v8     : [B,H,N,128] E4M3 outputs;  q_scale, k_scale, v_scale :
 *                    [B,H,ceil(N/128)] float32 outputs.
 *   d              : must be 128.
 *   flags          : an OR of fa_quant_flags (other bits: FA_ERR_ARG).
 * Q and K: as fa_hadamard_fp8_quant(hadamard = FA_QUANT_HADAMARD_QK set).  V: the
 * same with its own transform flag; with FA_QUANT_POW2_SCALE_V its scale is
 * s = 2^E, E = ceil(log2(amax / 448)), code = E4M3(y / s) (without the
 * transform y / s = x 2^-E is exact, so every code is the correctly rounded
 * one).  No output may equal an input or another output (FA_ERR_ARG).
 */
int fa_qkv_fp8_quant(const void* q, const void* k, const void* v, int in_dtype, uint8_t* q8, uint8_t* k8,
                     uint8_t* v8, float* q_scale, float* k_scale, float* v_scale, int B, int H, int N, int d,
                     int flags, void* stream);

/*
 * Split-KV forward for a few queries against a long key sequence (a decode
 * step of long-context inference), and the merge of partial attentions.
 * "Flash Attention" glossary page, second paragraph: the online softmax
 * accumulates partial results block by block; fourth paragraph: ring attention
 * spreads the tiling over devices.  Both rest on the identity, for disjoint
 * key parts p with partial results O_p (normalised by their own sum) and LSE_p:
 *     LSE = ln sum_p exp(LSE_p),    O = sum_p exp(LSE_p - LSE) O_p.
 */

/*
 * fa_fwd_decode_workspace_bytes -- device workspace fa_fwd_decode needs for
 * these sizes (0 when the sizes are invalid).  Host-only; no HIP call.
 */
size_t fa_fwd_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * fa_fwd_decode -- attention of Nq queries against Nk keys, bfloat16.
 *   q          : [B,H,Nq,d] bf16;  k, v : [B,H,Nk,d] bf16;  d is 64 or 128.
 *   o          : [B,H,Nq,d] bf16 output;  lse : [B,H,Nq] float32 output.
 *   causal     : 0 or 1.  With 1 the queries are the last Nq of the Nk tokens:
 *                query i sits at position Nk - Nq + i and sees keys
 *                0 .. Nk - Nq + i (Nq <= Nk is required).
 *   workspace  : caller-owned device buffer of at least
 *                fa_fwd_decode_workspace_bytes(B,H,Nq,Nk,d) bytes; its contents
 *                are overwritten and meaningless afterwards.  Calls that share a
 *                workspace must not run concurrently.
 * The keys are cut into chunks; one kernel writes every chunk's partial O
 * (float32) and LSE into the workspace, a second merges them (two launches on
 * `stream`).  The result equals fa_fwd on the same rows up to rounding.
 */
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_decode_noalloc -- fa_fwd_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels, with the partial results in a
 * library-owned static device array of 16 MiB (FA_DECODE_SCRATCH_BYTES) instead
 * of a caller workspace.  Arguments, layout and results as fa_fwd_decode.
 *   Sizes whose fa_fwd_decode_workspace_bytes exceeds FA_DECODE_SCRATCH_BYTES
 *   return FA_ERR_SCRATCH before any HIP call.
 *   The call allocates nothing (no hipMalloc, no allocating library routine);
 *   each GPU holds its own copy of the array from the library's first use on
 *   it until the process ends, and its address is looked up once per device.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (two streams, or two host threads) race and give wrong results;
 *   serialise them on one stream.  The array needs no clearing: every call
 *   writes every partial result it reads.
 */
#define FA_DECODE_SCRATCH_BYTES (16u * 1024u * 1024u)
int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/*
 * fa_lse_merge -- combine P partial attentions of the same queries over
 * disjoint key sets (for instance the shards of ring attention).
 *   o_parts    : [P,B,H,N,d] float32, part p normalised by its own sum.
 *   lse_parts  : [P,B,H,N] float32, natural-log units; -inf marks a part in
 *                which the row saw no key (that part is ignored).
 *   o          : [B,H,N,d] output, o_dtype FA_F32 or FA_BF16;  lse : [B,H,N] float32.
 *   d          : 64 or 128.  A row whose parts are all -inf gets O = 0, LSE = -inf.
 */
int fa_lse_merge(const float* o_parts, const float* lse_parts, int P, int B, int H, int N, int d,
                 void* o, int o_dtype, float* lse, void* stream);

/*
 * fa_bwd_workspace_bytes -- device workspace fa_bwd needs for these sizes
 * (0 when the sizes are invalid).  Host-only; no HIP call.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd -- backward pass of fa_fwd (bfloat16): the gradients of
 * L = sum(dO * O) with respect to Q, K and V.  The pages motivate the method
 * by the training of large models ("FlashAttention-3 (PT)", introduction and
 * section "Desempenho e importancia"; "Flash Attention" glossary page, third
 * paragraph) but print no formula for this pass; it is the chain rule
 * through the definition above, with P = exp(scale Q K^T - LSE) recomputed
 * tile by tile from the saved LSE (no N x N matrix in memory):
 *     dV = P^T dO,  dS = P * (dO V^T - Delta),  Delta_i = dO_i . O_i,
 *     dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, o, dout : [B,H,N,d] bfloat16; o and lse as returned by fa_fwd for
 *                      the same q, k, v, scale and causal flag.
 *   lse              : [B,H,N] float32 (natural-log units).
 *   dq, dk, dv       : [B,H,N,d] bfloat16 outputs, written in full.
 *   d in {64, 128}; dtype must be FA_BF16 (FA_ERR_DTYPE otherwise).
 *   workspace        : device memory owned by the caller, at least
 *                      fa_bwd_workspace_bytes(B,H,N,d) bytes (FA_ERR_ARG
 *                      otherwise); it receives Delta and LSE log2(e), float32
 *                      [B,H,N] each (8 B*H*N bytes, rounded up).  Calls that
 *                      share a workspace must not run concurrently.
 * Two kernels on `stream`; the results are deterministic (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
