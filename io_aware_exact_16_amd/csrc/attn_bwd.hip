// Backward pass of fused exact attention, bf16 in / bf16 gradients, float32
// arithmetic, gfx950.
//
// The pages motivate FlashAttention by the training of large models
// ("FlashAttention-3 (PT)", introduction and section "Desempenho e
// importancia"; "Flash Attention" glossary page, third paragraph), which runs
// this pass; they print no formula for it.  It is the chain rule through the
// forward definition, for an upstream gradient dO:
//     P = exp(scale Q K^T - LSE)   (recomputed tile by tile from the saved LSE)
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta_i = dO_i . O_i,
//     dQ = scale dS K,  dK = scale dS^T Q.
// As in the forward, no N x N matrix is ever written to HBM: S, P, dP and dS
// exist one register tile at a time.
//
// Three kernels on the caller's stream:
//  * prep: Delta_i = sum_d dO_id O_id and LSE_i log2(e), one row per d/8 lanes
//    (HBM bound: reads O and dO once);
//  * dK/dV: one workgroup = 4 waves = 256 keys; each wave keeps its 64 keys of
//    K and V in registers as matrix-instruction operands, with the dK and dV
//    accumulators (float32, 256 registers per lane, AGPRs included), while
//    32-query tiles of Q, dO, LSE and Delta stream through LDS by DMA, double
//    buffered.  Per tile and wave: S = Q K^T and dP = dO V^T (row reads of the
//    tiles), P and dS in registers, then dV^T += dO^T P and dK^T += Q^T dS
//    (transposed reads, ds_read_b64_tr_b16).  The accumulator layout makes P
//    and dS directly the B operands of the last two products, as in the
//    forward;
//  * dQ: one workgroup = 4 waves = 128 queries, the forward's structure: Q and
//    dO stay in registers, 64-key tiles of K and V stream through LDS, and per
//    tile S^T = K Q^T, dP^T = V dO^T, dS^T in registers, dQ^T += K^T dS^T.
// The dQ kernel recomputes S and dP, so the pass does 7 tile products instead
// of 5; in exchange no workgroup ever adds into another's output (no atomics,
// deterministic results).  Causal work skips the tiles above the diagonal in
// both kernels and masks only the tiles that cross it or the sequence end.
//
// Register layouts of the 32x32x16 bf16 instruction: attn_bf16_common.h.
#include "attn_bf16_common.h"

namespace fa {
namespace {

using namespace bf16k;

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// prep: Delta and LSE * log2(e), float32 [B*H*N]
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const uint16_t* __restrict__ O,
                                                            const uint16_t* __restrict__ dO,
                                                            const float* __restrict__ LSE, float* __restrict__ L2,
                                                            float* __restrict__ Dl, long rows) {
  constexpr int LPR = D / 8;              // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;          // rows per workgroup
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(O + row * D + 8 * sub);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + row * D + 8 * sub);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(av[i] & 0xFFFF0000u), __uint_as_float(bv[i] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < rows && sub == 0) {
    Dl[row] = acc;
    L2[row] = LSE[row] * LOG2E;
  }
}

// ---------------------------------------------------------------------------
// dK / dV
constexpr int KV_NT = 256;   // 4 waves
constexpr int KV_KW = 64;    // keys per wave
constexpr int KV_BK = 256;   // keys per workgroup
constexpr int KV_TQ = 32;    // queries per tile

// One 32-query tile of one wave (64 keys).  qt / ot: LDS tiles of Q and dO
// (row-major, swizzled like the forward's K tile); l2t / dlt: the tile's
// LSE log2(e) and Delta.  Accumulator register r of half-wave h belongs to
// query row 16 (r / 8) + 8 h + r % 8 of the tile (rows permuted through
// key_of_arow in the A-operand reads) and to key column kw0 + 32 kb + lane % 32.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dkdv_tile(const char* qt, const char* ot, const float* l2t, const float* dlt,
                                          const uint32_t (&koff)[D / 16], const uint32_t (&voff)[D / 32][2],
                                          const bf16x8 (&kf)[2][D / 16], const char* vw, const uint32_t (&vboff)[D / 16],
                                          f32x16 (&dka)[2][D / 32], f32x16 (&dva)[2][D / 32], float c, int q0,
                                          int kw0, int N, int half, int l32) {
  constexpr int QC_BYTES = 16 * D * 2;   // one 16-row chunk of the tile
  // S = Q K^T, then P = exp2(c s - LSE log2 e) in place (and its bf16 copy)
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(qt + koff[dc]);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[0][dc], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[1][dc], s[1], 0, 0, 0);
  }
  bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
  for (int qc = 0; qc < 2; ++qc) {
    const float4 la = *reinterpret_cast<const float4*>(l2t + 16 * qc + 8 * half);
    const float4 lb = *reinterpret_cast<const float4*>(l2t + 16 * qc + 8 * half + 4);
    const float l2v[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * qc + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -l2v[e]));
        if (MASK) {
          const int q = q0 + 16 * qc + 8 * half + e, key = kw0 + 32 * kb + l32;
          if (key >= N || (CAUSAL && key > q)) p = 0.0f;
        }
        s[kb][r] = p;
        pb[kb][qc][e] = (__bf16)p;
      }
  }

  // dP = dO V^T, then dS = P (dP - Delta), rounded to bf16
  f32x16 dp[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[kb][r] = 0.0f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ot + koff[dc]);
    const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(vw + vboff[dc]);
    const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(vw + vboff[dc] + 32 * D * 2);
    dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v0, dp[0], 0, 0, 0);
    dp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v1, dp[1], 0, 0, 0);
  }
#pragma unroll
  for (int qc = 0; qc < 2; ++qc) {
    const float4 da = *reinterpret_cast<const float4*>(dlt + 16 * qc + 8 * half);
    const float4 db = *reinterpret_cast<const float4*>(dlt + 16 * qc + 8 * half + 4);
    const float dlv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * qc + e;
        dsb[kb][qc][e] = (__bf16)(s[kb][r] * (dp[kb][r] - dlv[e]));
      }
  }

  // dV^T += dO^T P, dK^T += Q^T dS (A operands: transposed reads of the tiles)
#pragma unroll
  for (int qc = 0; qc < 2; ++qc)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x4_t o0 = tr_read(ot + voff[db][0] + qc * QC_BYTES);
      const bf16x4_t o1 = tr_read(ot + voff[db][1] + qc * QC_BYTES);
      const bf16x8 oa = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
      dva[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb[0][qc], dva[0][db], 0, 0, 0);
      dva[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb[1][qc], dva[1][db], 0, 0, 0);
      const bf16x4_t a0 = tr_read(qt + voff[db][0] + qc * QC_BYTES);
      const bf16x4_t a1 = tr_read(qt + voff[db][1] + qc * QC_BYTES);
      const bf16x8 qa = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      dka[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsb[0][qc], dka[0][db], 0, 0, 0);
      dka[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsb[1][qc], dka[1][db], 0, 0, 0);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(KV_NT, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nkb, int total, float c, float scale) {
  constexpr int CPR = D / 8;
  constexpr int TILE_CHUNKS = KV_TQ * CPR;
  constexpr int NW = KV_NT / 64;
  constexpr int LPW = TILE_CHUNKS / KV_NT;
  __shared__ uint4 qbuf0[TILE_CHUNKS], qbuf1[TILE_CHUNKS], obuf0[TILE_CHUNKS], obuf1[TILE_CHUNKS];
  __shared__ float lbuf0[KV_TQ], lbuf1[KV_TQ], dbuf0[KV_TQ], dbuf1[KV_TQ];
  __shared__ uint4 vsm[KV_BK * CPR];         // this workgroup's V rows, 64 per wave, swizzled

  const int L = xcd_logical_id(blockIdx.x, total);
  const int bh = L / nkb;
  const int k0 = (L - bh * nkb) * KV_BK;     // causal: low key blocks (the most work) first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + KV_KW * wave;
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t nbytes = (uint32_t)N * D * 2;

  // K of this wave's keys as B operands in registers: lane holds key
  // kw0 + 32 kb + l32, dims 16 dc + 8 half + 0..7 (zeros past the end of the
  // sequence).  V, the B operand of dP, waits in LDS (registers are short):
  // the wave's 64 rows by DMA, in the swizzled row layout, read back with the
  // same lane pattern.
  bf16x8 kf[2][D / 16];
  {
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + hoff), 0, nbytes, 0x00020000);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t off = (uint32_t)((kw0 + 32 * kb + l32) * D + 8 * half) * 2;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        kf[kb][dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 32 * dc, 0, 0));
    }
  }
  uint4* vw = vsm + wave * KV_KW * CPR;
  {
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + hoff), 0, nbytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < KV_KW * CPR / 64; ++i) {
      const int pos = i * 64 + lane, row = pos / CPR, slot = pos % CPR;
      lds_dma16(vrs, vw + i * 64, (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2, (uint32_t)kw0 * D * 2);
    }
  }
  uint32_t vboff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) vboff[dc] = 16 * lds_chunk<D>(l32, 2 * dc + half);

  // LDS byte offsets: row reads (A operand, rows permuted) and transposed reads
  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  uint32_t voff[D / 32][2];
  {
    const int b16 = lane >> 4, j16 = lane & 15;
    const int row = 8 * (b16 >> 1) + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * (b16 & 1) + 4 * (j16 & 3);
      voff[db][0] = 16 * lds_chunk<D>(row, dcol >> 3) + 2 * (dcol & 7);
      voff[db][1] = 16 * lds_chunk<D>(row + 4, dcol >> 3) + 2 * (dcol & 7);
    }
  }

  // tile DMA: Q and dO rows (swizzled), LSE log2 e and Delta (wave 0, 8 lanes each);
  // rows past the end of the sequence read as zeros, which makes their terms vanish
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(L2 + (size_t)bh * N), 0, (uint32_t)N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Dl + (size_t)bh * N), 0, (uint32_t)N * 4, 0x00020000);
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane, row = pos / CPR, slot = pos % CPR;
    lane_off[i] = (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2;
  }
  auto issue_tile = [&](int q0, uint4* qd, uint4* od, float* ld, float* dd) {
    const uint32_t base = (uint32_t)q0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      lds_dma16(qrs, qd + slot0, lane_off[i], base);
      lds_dma16(ors, od + slot0, lane_off[i], base);
    }
    if (wave == 0 && lane < KV_TQ / 4) {
      lds_dma16(lrs, ld, 16 * lane, (uint32_t)q0 * 4);
      lds_dma16(drs, dd, 16 * lane, (uint32_t)q0 * 4);
    }
  };

  f32x16 dka[2][D / 32], dva[2][D / 32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dka[kb][db][r] = 0.0f;
        dva[kb][db][r] = 0.0f;
      }

  const int qstart = CAUSAL ? k0 : 0;        // queries before the first key see none of these keys
  const int ntiles = (N - qstart + KV_TQ - 1) / KV_TQ;
  const bool active = kw0 < N;
  const bool ktail = kw0 + KV_KW > N;

  auto step = [&](int t, const uint4* qc, const uint4* oc, const float* lc, const float* dlc, uint4* qn, uint4* on,
                  float* ln, float* dn) {
    const int q0 = qstart + t * KV_TQ;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this wave's part of tile t has landed
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's reads of the other buffers are done
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_tile(q0 + KV_TQ, qn, on, ln, dn);
    if (!active || (CAUSAL && q0 + KV_TQ - 1 < kw0)) return;   // no query of the tile sees these keys
    const char* qt = reinterpret_cast<const char*>(qc);
    const char* ot = reinterpret_cast<const char*>(oc);
    const char* vwc = reinterpret_cast<const char*>(vw);
    if (ktail || (CAUSAL && q0 < kw0 + KV_KW - 1))
      dkdv_tile<D, CAUSAL, true>(qt, ot, lc, dlc, koff, voff, kf, vwc, vboff, dka, dva, c, q0, kw0, N, half, l32);
    else
      dkdv_tile<D, CAUSAL, false>(qt, ot, lc, dlc, koff, voff, kf, vwc, vboff, dka, dva, c, q0, kw0, N, half, l32);
  };

  issue_tile(qstart, qbuf0, obuf0, lbuf0, dbuf0);
  for (int t = 0; t < ntiles; t += 2) {
    step(t, qbuf0, obuf0, lbuf0, dbuf0, qbuf1, obuf1, lbuf1, dbuf1);
    if (t + 1 < ntiles) step(t + 1, qbuf1, obuf1, lbuf1, dbuf1, qbuf0, obuf0, lbuf0, dbuf0);
  }

  // dK = scale dK^T acc, dV = dV^T acc; lane holds key kw0 + 32 kb + l32,
  // register 4 a + i of block db is dim 32 db + 8 a + 4 half + i
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw0 + 32 * kb + l32;
    if (key >= N) continue;
    uint16_t* krow = dK + hoff + (size_t)key * D;
    uint16_t* vrow = dV + hoff + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * half;
        const bf16x4_t wk = {(__bf16)(dka[kb][db][4 * a + 0] * scale), (__bf16)(dka[kb][db][4 * a + 1] * scale),
                             (__bf16)(dka[kb][db][4 * a + 2] * scale), (__bf16)(dka[kb][db][4 * a + 3] * scale)};
        const bf16x4_t wv = {(__bf16)dva[kb][db][4 * a + 0], (__bf16)dva[kb][db][4 * a + 1],
                             (__bf16)dva[kb][db][4 * a + 2], (__bf16)dva[kb][db][4 * a + 3]};
        *reinterpret_cast<bf16x4_t*>(krow + d0) = wk;
        *reinterpret_cast<bf16x4_t*>(vrow + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
constexpr int DQ_NT = 256;   // 4 waves, 32 queries each
constexpr int DQ_BR = 128;   // queries per workgroup

// One 64-key tile of one wave.  Lane holds query qi; register r of 32-key block
// kb is key j0 + 32 kb + 16 (r / 8) + 8 half + r % 8 (A-operand rows permuted).
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dq_tile(const char* kt, const char* vt, const uint32_t (&koff)[D / 16],
                                        const uint32_t (&voff)[D / 32][2], const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&of)[D / 16], f32x16 (&dqa)[D / 32], float c, float l2,
                                        float dl, int j0, int qi, int N, int half) {
  constexpr int KB_BYTES = 32 * D * 2;
  constexpr int KC_BYTES = 16 * D * 2;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb) {
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.0f;
      dp[r] = 0.0f;
    }
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + koff[dc] + kb * KB_BYTES);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s, 0, 0, 0);
    }
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + koff[dc] + kb * KB_BYTES);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[dc], dp, 0, 0, 0);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
      if (MASK) {
        const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
        if (key >= N || (CAUSAL && key > qi)) p = 0.0f;
      }
      dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl));
    }
    // dQ^T += K^T dS^T (A operand: transposed reads of the K tile)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int kc = 2 * kb + h;
        const bf16x4_t k0 = tr_read(kt + voff[db][0] + kc * KC_BYTES);
        const bf16x4_t k1 = tr_read(kt + voff[db][1] + kc * KC_BYTES);
        const bf16x8 ka = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsb[h], dqa[db], 0, 0, 0);
      }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DQ_NT, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    uint16_t* __restrict__ dQ, int N, int nqb, int total, float c, float scale) {
  constexpr int CPR = D / 8;
  constexpr int TILE_CHUNKS = BC * CPR;
  constexpr int NW = DQ_NT / 64;
  constexpr int LPW = TILE_CHUNKS / DQ_NT;
  __shared__ uint4 kbuf0[TILE_CHUNKS], kbuf1[TILE_CHUNKS], vbuf0[TILE_CHUNKS], vbuf1[TILE_CHUNKS];

  const int L = xcd_logical_id(blockIdx.x, total);
  const int bh = L / nqb;
  int qb = L - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;             // longest query blocks first
  const int q0 = qb * DQ_BR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int qw = q0 + 32 * wave;
  const int qi = qw + l32;
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t nbytes = (uint32_t)N * D * 2;

  // Q^T and dO^T as B operands: lane holds query qi, dims 16 dc + 8 half + 0..7
  bf16x8 qf[D / 16], of[D / 16];
  {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + hoff), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + hoff), 0, nbytes, 0x00020000);
    const uint32_t off = (uint32_t)(qi * D + 8 * half) * 2;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      qf[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 32 * dc, 0, 0));
      of[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ors, off + 32 * dc, 0, 0));
    }
  }
  const float l2 = qi < N ? L2[(size_t)bh * N + qi] : 0.0f;
  const float dl = qi < N ? Dl[(size_t)bh * N + qi] : 0.0f;

  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  uint32_t voff[D / 32][2];
  {
    const int b16 = lane >> 4, j16 = lane & 15;
    const int key = 8 * (b16 >> 1) + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * (b16 & 1) + 4 * (j16 & 3);
      voff[db][0] = 16 * lds_chunk<D>(key, dcol >> 3) + 2 * (dcol & 7);
      voff[db][1] = 16 * lds_chunk<D>(key + 4, dcol >> 3) + 2 * (dcol & 7);
    }
  }

  const int kend = CAUSAL ? min(N, q0 + DQ_BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + hoff), 0, nbytes, 0x00020000);
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane, row = pos / CPR, slot = pos % CPR;
    lane_off[i] = (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2;
  }
  auto issue_tile = [&](int j0, uint4* kd, uint4* vd) {
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      lds_dma16(krs, kd + slot0, lane_off[i], base);
      lds_dma16(vrs, vd + slot0, lane_off[i], base);
    }
  };

  f32x16 dqa[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.0f;

  auto step = [&](int t, const uint4* kc, const uint4* vc, uint4* kn, uint4* vn) {
    const int j0 = t * BC;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_tile(j0 + BC, kn, vn);
    if (CAUSAL && j0 > qw + 31) return;      // the whole tile is above this wave's diagonal
    const char* kt = reinterpret_cast<const char*>(kc);
    const char* vt = reinterpret_cast<const char*>(vc);
    if ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw))
      dq_tile<D, CAUSAL, true>(kt, vt, koff, voff, qf, of, dqa, c, l2, dl, j0, qi, N, half);
    else
      dq_tile<D, CAUSAL, false>(kt, vt, koff, voff, qf, of, dqa, c, l2, dl, j0, qi, N, half);
  };

  issue_tile(0, kbuf0, vbuf0);
  for (int t = 0; t < ntiles; t += 2) {
    step(t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 < ntiles) step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }

  if (qi < N) {
    uint16_t* row = dQ + hoff + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * half;
        const bf16x4_t w = {(__bf16)(dqa[db][4 * a + 0] * scale), (__bf16)(dqa[db][4 * a + 1] * scale),
                            (__bf16)(dqa[db][4 * a + 2] * scale), (__bf16)(dqa[db][4 * a + 3] * scale)};
        *reinterpret_cast<bf16x4_t*>(row + d0) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* l2, float* dl, int B, int H, int N, float scale,
                  hipStream_t stream) {
  const long rows = (long)B * H * N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((attn_bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), lse, l2, dl, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c = (float)((double)scale * 1.4426950408889634);
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  const int nkb = (N + KV_BK - 1) / KV_BK;
  const int tkv = nkb * B * H;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3(tkv), dim3(KV_NT), 0, stream, Q, K, V, dO, l2, dl,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, nkb, tkv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (N + DQ_BR - 1) / DQ_BR;
  const int tq = nqb * B * H;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3(tq), dim3(DQ_NT), 0, stream, Q, K, V, dO, l2, dl,
                     static_cast<uint16_t*>(dq), N, nqb, tq, c, scale);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  const size_t one = ((size_t)B * H * N * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;
}

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
                                int d, float scale, bool causal, hipStream_t stream) {
  const size_t one = attn_bwd_workspace_bytes(B, H, N) / 2;
  float* l2 = static_cast<float*>(workspace);
  float* dl = reinterpret_cast<float*>(static_cast<char*>(workspace) + one);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, dout, dq, dk, dv, l2, dl, B, H, N, scale, stream)
                  : launch<128, false>(q, k, v, o, lse, dout, dq, dk, dv, l2, dl, B, H, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, dout, dq, dk, dv, l2, dl, B, H, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, dout, dq, dk, dv, l2, dl, B, H, N, scale, stream);
}

}  // namespace fa
