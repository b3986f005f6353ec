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
// Kernels on the caller's stream, in this order:
//  * dQ pass: 8 waves of 32 queries (Q and dO in registers), 64-key tiles of
//    K and V rows through LDS; per tile S^T = K Q^T, dP^T = V dO^T, dS^T,
//    dQ^T += K^T dS^T.  It also forms Delta_i = dO_i . O_i and LSE_i log2(e)
//    of its queries and leaves them in the workspace for
//  * the dK/dV pass: 8 waves (two per SIMD) own 128 keys in four groups of 32.
//    For each group one wave holds K and forms S, P and dV^T += dO^T P; the
//    other holds V, forms dP, then dS = P (dP - Delta) (P passed through LDS)
//    and dK^T += Q^T dS.  64-query tiles of Q and dO rows, LSE and Delta
//    stream through LDS by DMA.
// A product that sums over tokens (dV = P^T dO, dK = dS^T Q, dQ = dS K) needs
// its A operand with 8 consecutive tokens per lane; it comes from the row
// tile in LDS through transposing reads (ds_read_b64_tr_b16), as the forward
// reads V^T, so no transposed copy is ever written to or read from HBM.
// The accumulator layout of the 32x32x16 instruction makes P and dS directly
// the B operands of the products that consume them, as in the forward.  The
// pass does 7 tile products instead of 5 (the dQ pass forms S and dP again),
// and in exchange no workgroup ever adds into another's output: no atomics,
// deterministic results.  Causal work skips the tiles above the diagonal and
// masks only those that cross it or the end of the sequence.
//
// Register layouts of the 32x32x16 bf16 instruction: attn_bf16_common.h.
#include "attn_bf16_common.h"

namespace fa {
namespace {

using namespace bf16k;

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// dK and dV in one pass, split between two wave roles.  One workgroup = 8
// waves, two per SIMD, owns 128 keys.  Waves 0..3 ("P waves") each own 32
// keys with K in registers; waves 4..7 ("dS waves") own the same four 32-key
// groups with V in registers.  Each wave holds one accumulator set (64
// registers, not 128), so two waves fit on every SIMD, one of each role
// (hardware waves go to SIMDs round-robin: P wave w and dS wave w + 4 share
// one), and one's vector work runs beside the other's matrix products.  Per
// 64-query tile, two phases split by a barrier (each handles the tile in
// two 32-query halves):
//   1. P waves: S = Q K^T, P (stored to LDS as float32);
//      dS waves: dP = dO V^T, kept as dP - Delta;
//   2. P waves: dV^T += dO^T P;  dS waves: dS = P (dP - Delta), dK^T += Q^T dS.
// Both roles compute P, dP and dS exactly as a single wave would.  The tiles
// of Q and dO rows, LSE and Delta stream through LDS by DMA from the end of
// the sequence down (every workgroup of a head reads the same tile at about
// the same time, so the head's query-side data passes through the XCD's L2
// once), double buffered, each slot its own __shared__ object so that reading
// one slot never waits for the DMA into the other.  The A operands of the two
// token-summing products (dO^T, Q^T: 8 consecutive queries per lane) come
// from the row tiles through transposing LDS reads, so no d-major copies are
// fetched: the pass is bound by its tile stream, and this halves it.
constexpr int KV_NT = 512;   // 8 waves, two per SIMD
constexpr int KV_KW = 32;    // keys per wave
constexpr int KV_BK = 128;   // keys per workgroup
constexpr int KV_TQ = 64;    // queries per tile
constexpr int KV_NH = KV_TQ / 32;   // 32-query halves of a tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(KV_NT, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nkb, int total, float c, float scale) {
  constexpr int CPR = D / 8;
  constexpr int ROW_CHUNKS = KV_TQ * CPR;
  constexpr int P_CHUNKS = 4 * KV_KW * KV_TQ / 4;          // float32 P of the four 32-key groups
  constexpr int KB_BYTES = 32 * D * 2;                     // 32 query rows of a row tile
  constexpr int KC_BYTES = 16 * D * 2;                     // 16 query rows of a row tile
  constexpr int RPW = ROW_CHUNKS / KV_NT;                  // DMA instructions per wave and tensor
  static_assert(ROW_CHUNKS % KV_NT == 0, "whole DMA instructions per wave and tensor");
  __shared__ uint4 qr0[ROW_CHUNKS], qr1[ROW_CHUNKS], or0[ROW_CHUNKS], or1[ROW_CHUNKS];
  __shared__ float lb0[KV_TQ], lb1[KV_TQ], db0[KV_TQ], db1[KV_TQ];
  __shared__ uint4 pbuf[P_CHUNKS];
  // slot S of each buffer, S known at compile time
  auto QR = [&](auto sc) { return reinterpret_cast<const char*>(decltype(sc)::value ? qr1 : qr0); };
  auto OR = [&](auto sc) { return reinterpret_cast<const char*>(decltype(sc)::value ? or1 : or0); };
  auto LB = [&](auto sc) { return decltype(sc)::value ? lb1 : lb0; };
  auto DB = [&](auto sc) { return decltype(sc)::value ? db1 : db0; };

  const int L = xcd_logical_id(blockIdx.x, total);
  const int bh = L / nkb;
  const int k0 = (L - bh * nkb) * KV_BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < 4;
  const int grp = wave & 3;                  // 32-key group, shared by P wave grp and dS wave grp + 4
  const int half = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + KV_KW * grp;
  const int key = kw0 + l32;
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t nbytes = (uint32_t)N * D * 2;

  // K (P waves) or V (dS waves) of this wave's keys: the B operand of S or dP
  bf16x8 kv[D / 16];
  {
    const uint16_t* src = pwave ? K : V;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + hoff), 0, nbytes, 0x00020000);
    const uint32_t off = (uint32_t)(key * D + 8 * half) * 2;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      kv[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * dc, 0, 0));
  }
  // LDS byte offsets: koff, the row-permuted A operand of S / dP (query rows);
  // voff, the transposing reads of the dO^T / Q^T A operand (rows d of block
  // db, queries 8 half + 0..3 and + 4..7 of a 16-query chunk)
  uint32_t koff[D / 16], voff[D / 32][2];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  {
    const int b16 = lane >> 4, j16 = lane & 15;
    const int tok = 8 * (b16 >> 1) + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * (b16 & 1) + 4 * (j16 & 3);
      voff[db][0] = 16 * lds_chunk<D>(tok, dcol >> 3) + 2 * (dcol & 7);
      voff[db][1] = 16 * lds_chunk<D>(tok + 4, dcol >> 3) + 2 * (dcol & 7);
    }
  }
  // this lane's float32 P values 4 j .. 4 j + 3 of its group's tile: lane-linear,
  // so the stores and loads of a wave each cover 1 KB of consecutive bytes
  char* const pw = reinterpret_cast<char*>(pbuf) + grp * (KV_KW * KV_TQ * 4) + 16 * lane;

  // DMA: per-lane offsets fixed, and per-tile buffer descriptors (scalar
  // registers) that start at the tile and end where the tensor ends, so rows
  // past the end read as zeros.  (A VGPR that addressed a DMA in flight is
  // not rewritten before that DMA completes, so per-tile vector offsets could
  // make the compiler wait for the prefetch.)
  uint32_t row_off[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int slot = i * KV_NT + tid, r = slot / CPR, ch = slot % CPR;
    row_off[i] = (uint32_t)(r * D + 8 * (ch ^ swz<D>(r))) * 2;
  }
  const uint32_t lane_off = 16 * lane;
  const char* qh = reinterpret_cast<const char*>(Q + hoff);
  const char* oh = reinterpret_cast<const char*>(dO + hoff);
  const char* lh = reinterpret_cast<const char*>(L2 + (size_t)bh * N);
  const char* dh = reinterpret_cast<const char*>(Dl + (size_t)bh * N);
  auto rsrc_at = [](const char* base, uint32_t off, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), 0, bytes - off, 0x00020000);
  };
  const int qstart = CAUSAL ? k0 : 0;
  const int ntiles = (N - qstart + KV_TQ - 1) / KV_TQ;
  const int qtop = qstart + (ntiles - 1) * KV_TQ;
  auto tile_q0 = [&](int t) { return qtop - t * KV_TQ; };
  // Q rows, dO rows, LSE and Delta of tile t into slot S
  auto issue_tile = [&](auto sc, int t) {
    constexpr int S = decltype(sc)::value;
    const uint32_t rb = (uint32_t)tile_q0(t) * D * 2;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      lds_dma16(rsrc_at(qh, rb, nbytes), (S ? qr1 : qr0) + i * KV_NT + 64 * wave, row_off[i], 0);
      lds_dma16(rsrc_at(oh, rb, nbytes), (S ? or1 : or0) + i * KV_NT + 64 * wave, row_off[i], 0);
    }
    if (wave == 0 && lane < KV_TQ / 4) {
      const uint32_t lb = (uint32_t)tile_q0(t) * 4;
      lds_dma16(rsrc_at(lh, lb, (uint32_t)N * 4), S ? lb1 : lb0, lane_off, 0);
      lds_dma16(rsrc_at(dh, lb, (uint32_t)N * 4), S ? db1 : db0, lane_off, 0);
    }
  };

  f32x16 acc[D / 32];                        // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // acc[db] += A^T B over the tile's queries, A^T read transposed from the
  // row tile at rt (dO rows for dV, Q rows for dK), B = b[qc] (P or dS) for
  // queries 16 qc .. 16 qc + 15
  auto tr_products = [&](const char* rt, const bf16x8 (&b)[2 * KV_NH]) __attribute__((always_inline)) {
#pragma unroll
    for (int qc = 0; qc < 2 * KV_NH; ++qc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x4_t v0 = tr_read(rt + voff[db][0] + qc * KC_BYTES);
        const bf16x4_t v1 = tr_read(rt + voff[db][1] + qc * KC_BYTES);
        const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, b[qc], acc[db], 0, 0, 0);
      }
  };

  // P wave, phase 1 of tile t (slot S): S = Q K^T, P (stored), one 32-query
  // half at a time; returns P as the bf16 B operands of phase 2.  MASK
  // (uniform) marks tiles that cross the diagonal or the end of the sequence;
  // it guards only the zeroing of P, so both kinds of tile share one copy of
  // the matrix code.
  auto p_phase1 = [&](auto sc, bool mask, int q0, bf16x8 (&pb)[2 * KV_NH]) __attribute__((always_inline)) {
    const char* qt = QR(sc);
    const float* l2t = LB(sc);
#pragma unroll
    for (int h = 0; h < KV_NH; ++h) {
      bf16x8 qa[D / 16];
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) qa[dc] = *reinterpret_cast<const bf16x8*>(qt + h * KB_BYTES + koff[dc]);
      float l2v[16];
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const float4 la = *reinterpret_cast<const float4*>(l2t + 32 * h + 16 * qc + 8 * half);
        const float4 lb = *reinterpret_cast<const float4*>(l2t + 32 * h + 16 * qc + 8 * half + 4);
        l2v[8 * qc + 0] = la.x, l2v[8 * qc + 1] = la.y, l2v[8 * qc + 2] = la.z, l2v[8 * qc + 3] = la.w;
        l2v[8 * qc + 4] = lb.x, l2v[8 * qc + 5] = lb.y, l2v[8 * qc + 6] = lb.z, l2v[8 * qc + 7] = lb.w;
      }
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[dc], kv[dc], s, 0, 0, 0);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2v[r]));
      if (mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * h + 16 * (r / 8) + 8 * half + r % 8;
          if (key >= N || (CAUSAL && key > q)) p[r] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(pw + 1024 * (4 * h + j)) =
            make_float4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
#pragma unroll
      for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[2 * h + qc][e] = (__bf16)p[8 * qc + e];
    }
  };

  // dS wave, phase 1 of tile t (slot S): dP = dO V^T, returned as dP - Delta
  auto d_phase1 = [&](auto sc, f32x16 (&dpm)[KV_NH]) __attribute__((always_inline)) {
    const char* ot = OR(sc);
    const float* dlt = DB(sc);
#pragma unroll
    for (int h = 0; h < KV_NH; ++h) {
      bf16x8 oa[D / 16];
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) oa[dc] = *reinterpret_cast<const bf16x8*>(ot + h * KB_BYTES + koff[dc]);
      float dl[16];
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const float4 da = *reinterpret_cast<const float4*>(dlt + 32 * h + 16 * qc + 8 * half);
        const float4 dbv = *reinterpret_cast<const float4*>(dlt + 32 * h + 16 * qc + 8 * half + 4);
        dl[8 * qc + 0] = da.x, dl[8 * qc + 1] = da.y, dl[8 * qc + 2] = da.z, dl[8 * qc + 3] = da.w;
        dl[8 * qc + 4] = dbv.x, dl[8 * qc + 5] = dbv.y, dl[8 * qc + 6] = dbv.z, dl[8 * qc + 7] = dbv.w;
      }
      f32x16 dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.0f;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[dc], kv[dc], dp, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) dpm[h][r] = dp[r] - dl[r];
    }
  };

  // dS wave, phase 2: dS = P (dP - Delta) with the P the P wave just stored,
  // then dK^T += Q^T dS
  auto d_phase2 = [&](auto sc, const f32x16 (&dpm)[KV_NH]) __attribute__((always_inline)) {
    bf16x8 dsb[2 * KV_NH];
#pragma unroll
    for (int h = 0; h < KV_NH; ++h) {
      float pp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(pw + 1024 * (4 * h + j));
        pp[4 * j] = v.x, pp[4 * j + 1] = v.y, pp[4 * j + 2] = v.z, pp[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[2 * h + qc][e] = (__bf16)(pp[8 * qc + e] * dpm[h][8 * qc + e]);
    }
    tr_products(QR(sc), dsb);
  };

  // Every wave takes every tile of its workgroup's query range: a tile wholly
  // above a wave's part of the diagonal gives P = 0 and adds exact zeros, and
  // such tiles are about 1 % of the work.  With no per-wave skipping the loop
  // bodies have no data-dependent branches around the matrix code.
  const bool ktail = kw0 + KV_KW > N;
  // Step t (S = t % 2).  Phase 1 starts when the DMA of tile t (issued one
  // step earlier) has landed and every wave is done with the previous step's
  // LDS reads; it fetches tile t + 1 into the other slot.  Phase 2 starts when
  // every P wave has stored the tile's P.  The two roles run their own copies
  // of the loop (same barriers), so each keeps its accumulators in place.
  auto phase1 = [&](auto sc, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_tile(IC<1 - S>{}, t + 1);
    FA_SYNC_POINT();
  };
  auto phase2 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
  };
  auto pstep = [&](auto sc, int t) __attribute__((always_inline)) {
    phase1(sc, t);
    const int q0 = tile_q0(t);
    bf16x8 pb[2 * KV_NH];
    p_phase1(sc, ktail || (CAUSAL && q0 < kw0 + KV_KW - 1), q0, pb);
    phase2();
    tr_products(OR(sc), pb);
    FA_SYNC_POINT();
  };
  auto dstep = [&](auto sc, int t) __attribute__((always_inline)) {
    phase1(sc, t);
    f32x16 dpm[KV_NH];
    d_phase1(sc, dpm);
    phase2();
    d_phase2(sc, dpm);
    FA_SYNC_POINT();
  };

  issue_tile(IC<0>{}, 0);
  if (pwave) {
    int t = 0;
    for (; t + 2 <= ntiles; t += 2) {
      pstep(IC<0>{}, t);
      pstep(IC<1>{}, t + 1);
    }
    if (t < ntiles) pstep(IC<0>{}, t);
  } else {
    int t = 0;
    for (; t + 2 <= ntiles; t += 2) {
      dstep(IC<0>{}, t);
      dstep(IC<1>{}, t + 1);
    }
    if (t < ntiles) dstep(IC<0>{}, t);
  }

  if (key < N) {
    uint16_t* row = (pwave ? dV : dK) + hoff + (size_t)key * D;
    const float f = pwave ? 1.0f : scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * half;
        const bf16x4_t w = {(__bf16)(acc[db][4 * a + 0] * f), (__bf16)(acc[db][4 * a + 1] * f),
                            (__bf16)(acc[db][4 * a + 2] * f), (__bf16)(acc[db][4 * a + 3] * f)};
        *reinterpret_cast<bf16x4_t*>(row + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
constexpr int DQ_NT = 512;   // 8 waves, two per SIMD, 32 queries each
constexpr int DQ_BR = 256;   // queries per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DQ_NT, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ L2, float* __restrict__ Dl, uint16_t* __restrict__ dQ, int N, int nqb, int total, float c,
    float scale) {
  constexpr int CPR = D / 8;
  constexpr int NW = DQ_NT / 64;
  constexpr int TILE_CHUNKS = BC * CPR;            // row-major 64-key tile
  constexpr int LPW = TILE_CHUNKS / DQ_NT;         // DMA instructions per wave, tensor and tile
  constexpr int KB_BYTES = 32 * D * 2;             // 32 key rows
  constexpr int KC_BYTES = 16 * D * 2;             // 16 key rows
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
  float dl = 0.0f;                           // Delta of query qi, this lane's half of the dims first
  {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + hoff), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + hoff), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void*)(O + hoff), 0, nbytes, 0x00020000);
    const uint32_t off = (uint32_t)(qi * D + 8 * half) * 2;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      qf[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 32 * dc, 0, 0));
      of[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ors, off + 32 * dc, 0, 0));
    }
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 32 * dc, 0, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = __builtin_fmaf((float)of[dc][e], (float)o8[e], dl);
    }
  }
  // Delta_i = dO_i . O_i and LSE_i log2(e) of this wave's queries, which the
  // dK/dV pass (launched after this one) reads from the workspace
  dl = wave_halves_sum(dl);
  const float l2 = qi < N ? LSE[(size_t)bh * N + qi] * LOG2E : 0.0f;
  if (qi < N && half == 0) {
    L2[(size_t)bh * N + qi] = l2;
    Dl[(size_t)bh * N + qi] = dl;
  }

  // LDS byte offsets: K / V rows (A operand of S^T and dP^T, rows permuted)
  // and the transposing reads of K^T (A operand of dQ^T: rows d of block db,
  // keys 8 half + 0..3 and + 4..7 of a 16-key chunk) from the same K tile
  uint32_t koff[D / 16], voff[D / 32][2];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  {
    const int b16 = lane >> 4, j16 = lane & 15;
    const int tok = 8 * (b16 >> 1) + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * (b16 & 1) + 4 * (j16 & 3);
      voff[db][0] = 16 * lds_chunk<D>(tok, dcol >> 3) + 2 * (dcol & 7);
      voff[db][1] = 16 * lds_chunk<D>(tok + 4, dcol >> 3) + 2 * (dcol & 7);
    }
  }

  const int kend = CAUSAL ? min(N, q0 + DQ_BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + hoff), 0, nbytes, 0x00020000);
  uint32_t row_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane;
    const int r = pos / CPR, ch = pos % CPR;
    row_off[i] = (uint32_t)(r * D + 8 * (ch ^ swz<D>(r))) * 2;
  }
  auto issue_tile = [&](int j0, uint4* kd, uint4* vd) {
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      lds_dma16(krs, kd + slot0, row_off[i], base);
      lds_dma16(vrs, vd + slot0, row_off[i], base);
    }
  };

  f32x16 dqa[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.0f;

  // one 64-key tile: register r of 32-key block kb is key j0 + 32 kb + 16 (r / 8) + 8 half + r % 8
  auto tile = [&](auto maskc, const char* kt, const char* vt, int j0) {
    constexpr bool MASK = decltype(maskc)::value;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      __builtin_amdgcn_sched_barrier(0);     // one 32-key block's registers at a time
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
      }
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kt + koff[dc] + kb * KB_BYTES), qf[dc], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(vt + koff[dc] + kb * KB_BYTES), of[dc], dp, 0, 0, 0);
      }
      // keep 8 operand reads in flight ahead of the matrix ops
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < D / 8 - 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * h + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
          if (MASK) {
            const int key = j0 + 32 * kb + 16 * h + 8 * half + e;
            if (key >= N || (CAUSAL && key > qi)) p = 0.0f;
          }
          b[e] = (__bf16)(p * (dp[r] - dl));
        }
        // dQ^T += K^T dS^T: A operand read transposed from the K tile, keys 16 kc .. 16 kc + 15
        const int kc = 2 * kb + h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x4_t v0 = tr_read(kt + voff[db][0] + kc * KC_BYTES);
          const bf16x4_t v1 = tr_read(kt + voff[db][1] + kc * KC_BYTES);
          const bf16x8 ka = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, b, dqa[db], 0, 0, 0);
        }
      }
    }
  };

  // ANY = false: the tile is known to need no mask
  auto step = [&](auto anyc, int t, const uint4* kc, const uint4* vc, uint4* kn, uint4* vn) {
    const int j0 = t * BC;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_tile(j0 + BC, kn, vn);
    FA_SYNC_POINT();
    if (CAUSAL && j0 > qw + 31) return;      // the whole tile is above this wave's diagonal
    const char* kt = reinterpret_cast<const char*>(kc);
    const char* vt = reinterpret_cast<const char*>(vc);
    if (decltype(anyc)::value && ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw))) tile(IC<1>{}, kt, vt, j0);
    else tile(IC<0>{}, kt, vt, j0);
  };

  issue_tile(0, kbuf0, vbuf0);
  int t = 0;
  if (!CAUSAL)                               // only the last tile can need a mask: keep it out of the loop
    for (; t + 2 < ntiles; t += 2) {
      step(IC<0>{}, t, kbuf0, vbuf0, kbuf1, vbuf1);
      step(IC<0>{}, t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    }
  for (; t < ntiles; t += 2) {
    step(IC<1>{}, t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 < ntiles) step(IC<1>{}, t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
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

// Workspace: LSE log2 e and Delta, float32 [B*H*N] each, 256-byte aligned.
struct Ws {
  float* l2;
  float* dl;
  size_t bytes;
};

Ws carve(void* base, int B, int H, int N) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t f = up((size_t)B * H * N * sizeof(float));
  char* p = static_cast<char*>(base);
  return Ws{reinterpret_cast<float*>(p), reinterpret_cast<float*>(p + f), 2 * f};
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, const Ws& w, int B, int H, int N, float scale, hipStream_t stream) {
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  const float c = (float)((double)scale * 1.4426950408889634);
  const int nqb = (N + DQ_BR - 1) / DQ_BR;
  const int tq = nqb * B * H;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3(tq), dim3(DQ_NT), 0, stream, Q, K, V, dO,
                     static_cast<const uint16_t*>(o), lse, w.l2, w.dl, static_cast<uint16_t*>(dq), N, nqb, tq, c,
                     scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (N + KV_BK - 1) / KV_BK;
  const int tkv = nkb * B * H;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3(tkv), dim3(KV_NT), 0, stream, Q, K, V, dO, w.l2, w.dl,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, nkb, tkv, c, scale);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return carve(nullptr, B, H, N).bytes;
}

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
                                int d, float scale, bool causal, hipStream_t stream) {
  const Ws w = carve(workspace, B, H, N);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream)
                  : launch<128, false>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream);
}

}  // namespace fa
