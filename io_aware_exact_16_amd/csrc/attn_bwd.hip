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
// Kernels on the caller's stream:
//  * Delta pass: Delta_i = sum_d dO_id O_id and LSE_i log2(e);
//  * transpose pass: d-major copies of Q, dO and K in tiles of 64 tokens
//    ([tile][d][64], zero past the end of the sequence).  A product that sums
//    over tokens (dV = P^T dO, dK = dS^T Q, dQ = dS K) needs its LDS operand
//    with 8 consecutive tokens per lane; from a d-major tile that is one
//    16-byte LDS read instead of two transposing 8-byte reads, which run at
//    less than half the byte rate.  All backward kernels stay clear of the
//    LDS bandwidth limit this way (HBM cost: three bf16 copies, a few percent
//    of the pass);
//  * dK/dV pass: 8 waves (two per SIMD) own 128 keys in four groups of 32.
//    For each group one wave holds K and forms S, P and dV^T += dO^T P; the
//    other holds V, forms dP and, one tile later, dS = P (dP - Delta) (P
//    passed through LDS) and dK^T += Q^T dS.  32-query tiles of Q, dO, their
//    d-major copies, LSE and Delta stream through LDS by DMA.
//  * dQ pass: 8 waves of 32 queries (Q and dO in registers), 64-key tiles of
//    K, V and K's d-major copy through LDS; per tile S^T = K Q^T,
//    dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
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
constexpr int TT = 64;       // tokens per d-major tile

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
// transpose: X [B*H][N][D] -> XT [B*H][nb][D][TT] for three tensors in one launch
struct XT3 {
  const uint16_t* x[3];
  uint16_t* xt[3];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_transpose_kernel(XT3 a, int N, int nb, int tiles) {
  constexpr int CPR = D / 8;
  constexpr int PAD = D + 8;                 // padded row: 16-byte aligned, staggered banks
  __shared__ uint16_t t[TT * PAD];
  const int which = blockIdx.x / tiles;
  const int blk = blockIdx.x - which * tiles;   // = bh * nb + tile
  const int bh = blk / nb, r0 = (blk - bh * nb) * TT;
  const uint16_t* X = a.x[which] + (size_t)bh * N * D;
  for (int i = threadIdx.x; i < TT * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r0 + r < N) u = *reinterpret_cast<const uint4*>(X + (size_t)(r0 + r) * D + 8 * ch);
    *reinterpret_cast<uint4*>(&t[r * PAD + 8 * ch]) = u;
  }
  __syncthreads();
  uint16_t* XT = a.xt[which] + (size_t)blk * D * TT;
  for (int i = threadIdx.x; i < D * (TT / 8); i += 256) {
    const int d = i / (TT / 8), j = i % (TT / 8);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(8 * j + 2 * e) * PAD + d] | ((uint32_t)t[(8 * j + 2 * e + 1) * PAD + d] << 16);
    *reinterpret_cast<uint4*>(XT + (size_t)d * TT + 8 * j) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// LDS offset (16-byte chunks) of chunk c of row d in a d-major tile of W
// tokens (W/8 chunks per row), swizzled so that 16 lanes reading the same
// chunk of 16 consecutive rows hit distinct banks.
template <int W>
__device__ __forceinline__ int tchunk(int d, int c) {
  return W == 32 ? d * 4 + (c ^ ((d >> 2) & 3)) : d * 8 + (c ^ ((d >> 1) & 7));
}

// ---------------------------------------------------------------------------
// dK and dV in one pass, split between two wave roles.  One workgroup = 8
// waves, two per SIMD, owns 128 keys.  Waves 0..3 ("P waves") each own 32
// keys with K in registers: per query tile they form S = Q K^T, P, store P
// (float32) in LDS and add dV^T += dO^T P.  Waves 4..7 ("dS waves") own the
// same four 32-key groups with V in registers: per tile they form dP = dO V^T
// and keep dP - Delta in registers; one step later they read that tile's P,
// form dS = P (dP - Delta) and add dK^T += Q^T dS.  Each wave holds one
// accumulator set (64 registers, not 128), so two waves fit on every SIMD, one
// of each role (hardware waves go to SIMDs round-robin: P wave w and dS wave
// w + 4 share one), and one's softmax runs beside the other's matrix products.
// Both roles compute P, dP and dS exactly as a single wave would.
// 32-query tiles of Q, dO, their d-major copies, LSE and Delta stream through
// LDS by DMA from the end of the sequence down (every workgroup of a head reads
// the same tile at about the same time, so the head's query-side data passes
// through the XCD's L2 once).  Every buffer has two slots, each its own
// __shared__ object, and the unrolled loops name the slot at compile time: the
// compiler then knows that reading one slot does not alias the DMA in flight
// into the other, and only the step barrier waits for the DMA.  The d-major Q
// tile, which the dS waves use one step late, is fetched one step late too.
constexpr int KV_NT = 512;   // 8 waves, two per SIMD
constexpr int KV_KW = 32;    // keys per wave
constexpr int KV_BK = 128;   // keys per workgroup
constexpr int KV_TQ = 32;    // queries per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(KV_NT, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ QT, const uint16_t* __restrict__ dOT,
    const float* __restrict__ L2, const float* __restrict__ Dl, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int N, int nkb, int nb, int total, float c, float scale) {
  constexpr int CPR = D / 8;
  constexpr int NW = KV_NT / 64;
  constexpr int ROW_CHUNKS = KV_TQ * CPR;
  constexpr int T_CHUNKS = D * (KV_TQ / 8);
  constexpr int P_CHUNKS = 4 * KV_KW * KV_TQ / 4;          // float32 P of the four 32-key groups
  constexpr int RPW = (ROW_CHUNKS + KV_NT - 1) / KV_NT;   // DMA instructions per wave and row tile
  constexpr int TPW = (T_CHUNKS + KV_NT - 1) / KV_NT;
  __shared__ uint4 qr0[ROW_CHUNKS], qr1[ROW_CHUNKS], or0[ROW_CHUNKS], or1[ROW_CHUNKS];
  __shared__ uint4 ot0[T_CHUNKS], ot1[T_CHUNKS], qt0[T_CHUNKS], qt1[T_CHUNKS];
  __shared__ uint4 pb0[P_CHUNKS], pb1[P_CHUNKS];
  __shared__ float lb0[KV_TQ], lb1[KV_TQ], db0[KV_TQ], db1[KV_TQ];
  // slot S of each buffer, S known at compile time
  auto QR = [&](auto sc) { return reinterpret_cast<char*>(decltype(sc)::value ? qr1 : qr0); };
  auto OR = [&](auto sc) { return reinterpret_cast<char*>(decltype(sc)::value ? or1 : or0); };
  auto OT = [&](auto sc) { return reinterpret_cast<char*>(decltype(sc)::value ? ot1 : ot0); };
  auto QTB = [&](auto sc) { return reinterpret_cast<char*>(decltype(sc)::value ? qt1 : qt0); };
  auto PB = [&](auto sc) { return reinterpret_cast<char*>(decltype(sc)::value ? pb1 : pb0); };
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
  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  uint32_t toff[2];
#pragma unroll
  for (int qc = 0; qc < 2; ++qc) toff[qc] = 16 * tchunk<KV_TQ>(l32, 2 * qc + half);
  // this lane's float32 P values 4 j .. 4 j + 3 of its group's tile: lane-linear,
  // so the stores and loads of a wave each cover 1 KB of consecutive bytes
  const uint32_t poff = grp * (KV_KW * KV_TQ * 4) + 16 * lane;

  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + hoff), 0, nbytes, 0x00020000);
  const size_t thoff = (size_t)bh * nb * D * TT;
  const uint32_t tbytes = (uint32_t)nb * D * TT * 2;
  const __amdgpu_buffer_rsrc_t qtrs = __builtin_amdgcn_make_buffer_rsrc((void*)(QT + thoff), 0, tbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t otrs = __builtin_amdgcn_make_buffer_rsrc((void*)(dOT + thoff), 0, tbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(L2 + (size_t)bh * N), 0, (uint32_t)N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Dl + (size_t)bh * N), 0, (uint32_t)N * 4, 0x00020000);
  uint32_t row_off[RPW], t_off[TPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int slot = (i * NW + wave) * 64 + lane, r = slot / CPR, ch = slot % CPR;
    row_off[i] = (uint32_t)(r * D + 8 * (ch ^ swz<D>(r))) * 2;
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int slot = (i * NW + wave) * 64 + lane, d = slot / (KV_TQ / 8), cc = slot % (KV_TQ / 8);
    t_off[i] = (uint32_t)(d * TT * 2 + 16 * (cc ^ ((d >> 2) & 3)));
  }
  const int qstart = CAUSAL ? k0 : 0;
  const int ntiles = (N - qstart + KV_TQ - 1) / KV_TQ;
  const int qtop = qstart + (ntiles - 1) * KV_TQ;
  auto tile_q0 = [&](int t) { return qtop - t * KV_TQ; };
  auto tile_tb = [&](int t) { return (uint32_t)((tile_q0(t) / TT) * D * TT + tile_q0(t) % TT) * 2; };
  // rows of Q and dO, d-major dO, LSE and Delta of tile t into slot S
  auto issue_rows = [&](auto sc, int t) {
    const uint32_t rb = (uint32_t)tile_q0(t) * D * 2, tb = tile_tb(t);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if ((i * NW + wave) * 64 < ROW_CHUNKS) {
        lds_dma16(qrs, QR(sc) + 16 * (i * NW + wave) * 64, row_off[i], rb);
        lds_dma16(ors, OR(sc) + 16 * (i * NW + wave) * 64, row_off[i], rb);
      }
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      if ((i * NW + wave) * 64 < T_CHUNKS) lds_dma16(otrs, OT(sc) + 16 * (i * NW + wave) * 64, t_off[i], tb);
    if (wave == 0 && lane < KV_TQ / 4) {
      lds_dma16(lrs, LB(sc), 16 * lane, (uint32_t)tile_q0(t) * 4);
      lds_dma16(drs, DB(sc), 16 * lane, (uint32_t)tile_q0(t) * 4);
    }
  };
  // d-major Q of tile t into slot S
  auto issue_qt = [&](auto sc, int t) {
    const uint32_t tb = tile_tb(t);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      if ((i * NW + wave) * 64 < T_CHUNKS) lds_dma16(qtrs, QTB(sc) + 16 * (i * NW + wave) * 64, t_off[i], tb);
  };
  // start of step t (S = t % 2): wait for this wave's DMA and LDS stores, meet
  // the other waves, then fetch the rows of tile t + 1 and the d-major Q of tile t
  auto sync_issue = [&](auto sc, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_rows(IC<1 - S>{}, t + 1);
    if (t < ntiles) issue_qt(sc, t);
  };

  f32x16 acc[D / 32];                        // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // P wave, tile t in slot S: S = Q K^T, P (stored), dV^T += dO^T P.  All of
  // the tile's LDS operands are read first.  MASK (uniform) marks tiles that
  // cross the diagonal or the end of the sequence; it guards only the zeroing
  // of P, so both kinds of tile share one copy of the matrix code and the
  // accumulators never change registers.
  auto p_tile = [&](auto sc, bool mask, int q0) __attribute__((always_inline)) {
    const char* qt = QR(sc);
    const char* ott = OT(sc);
    const float* l2t = LB(sc);
    bf16x8 qa[D / 16], oa[2][D / 32];
    float l2v[16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) qa[dc] = *reinterpret_cast<const bf16x8*>(qt + koff[dc]);
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      const float4 la = *reinterpret_cast<const float4*>(l2t + 16 * qc + 8 * half);
      const float4 lb = *reinterpret_cast<const float4*>(l2t + 16 * qc + 8 * half + 4);
      l2v[8 * qc + 0] = la.x, l2v[8 * qc + 1] = la.y, l2v[8 * qc + 2] = la.z, l2v[8 * qc + 3] = la.w;
      l2v[8 * qc + 4] = lb.x, l2v[8 * qc + 5] = lb.y, l2v[8 * qc + 6] = lb.z, l2v[8 * qc + 7] = lb.w;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oa[qc][db] = *reinterpret_cast<const bf16x8*>(ott + toff[qc] + db * 32 * KV_TQ * 2);
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
        const int q = q0 + 16 * (r / 8) + 8 * half + r % 8;
        if (key >= N || (CAUSAL && key > q)) p[r] = 0.0f;
      }
    }
    char* pw = PB(sc) + poff;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(pw + 1024 * j) = make_float4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[8 * qc + e];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[qc][db], pb, acc[db], 0, 0, 0);
    }
  };

  // dS wave, step t (S = t % 2): dP of tile t (NEW, kept as dP - Delta in
  // dnew) and dS and dK^T += Q^T dS of tile t - 1 (PREV, slot 1 - S, whose P
  // the P waves stored one step earlier, with dP - Delta in dprev).  Both
  // halves in one block, all LDS operands read first, so the compiler can
  // interleave one tile's matrix products with the other's vector work.
  auto ds_step = [&](auto sc, auto newc, auto prevc, f32x16& dnew, const f32x16& dprev)
      __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    constexpr bool NEW = decltype(newc)::value, PREV = decltype(prevc)::value;
    bf16x8 oa[D / 16], qa[2][D / 32];
    float dl[16], pp[16];
    if (NEW) {
      const char* ot = OR(sc);
      const float* dlt = DB(sc);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) oa[dc] = *reinterpret_cast<const bf16x8*>(ot + koff[dc]);
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const float4 da = *reinterpret_cast<const float4*>(dlt + 16 * qc + 8 * half);
        const float4 dbv = *reinterpret_cast<const float4*>(dlt + 16 * qc + 8 * half + 4);
        dl[8 * qc + 0] = da.x, dl[8 * qc + 1] = da.y, dl[8 * qc + 2] = da.z, dl[8 * qc + 3] = da.w;
        dl[8 * qc + 4] = dbv.x, dl[8 * qc + 5] = dbv.y, dl[8 * qc + 6] = dbv.z, dl[8 * qc + 7] = dbv.w;
      }
    }
    if (PREV) {
      const char* qtt = QTB(IC<1 - S>{});
      const char* pr = PB(IC<1 - S>{}) + poff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(pr + 1024 * j);
        pp[4 * j] = v.x, pp[4 * j + 1] = v.y, pp[4 * j + 2] = v.z, pp[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          qa[qc][db] = *reinterpret_cast<const bf16x8*>(qtt + toff[qc] + db * 32 * KV_TQ * 2);
    }
    f32x16 dp;
    if (NEW) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.0f;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[dc], kv[dc], dp, 0, 0, 0);
    }
    if (PREV) {
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        bf16x8 dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[e] = (__bf16)(pp[8 * qc + e] * dprev[8 * qc + e]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[qc][db], dsb, acc[db], 0, 0, 0);
      }
    }
    if (NEW) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dnew[r] = dp[r] - dl[r];
    }
  };

  // Every wave takes every tile of its workgroup's query range: a tile wholly
  // above a wave's part of the diagonal gives P = 0 and adds exact zeros, and
  // such tiles are about 1 % of the work.  With no per-wave skipping the loop
  // bodies have no data-dependent branches around the matrix code.
  const bool ktail = kw0 + KV_KW > N;
  auto pmask = [&](int t) { return ktail || (CAUSAL && tile_q0(t) < kw0 + KV_KW - 1); };
  issue_rows(IC<0>{}, 0);
  if (pwave) {
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      sync_issue(IC<0>{}, t);
      p_tile(IC<0>{}, pmask(t), tile_q0(t));
      sync_issue(IC<1>{}, t + 1);
      p_tile(IC<1>{}, pmask(t + 1), tile_q0(t + 1));
    }
    if (t < ntiles) {                        // t = ntiles - 1, even
      sync_issue(IC<0>{}, t);
      p_tile(IC<0>{}, pmask(t), tile_q0(t));
      sync_issue(IC<1>{}, ntiles);           // the dS waves' last step reads the last P
    } else {
      sync_issue(IC<0>{}, ntiles);
    }
  } else {
    // steps 0 .. ntiles: dP of tile t and dK of tile t - 1; d0 and d1
    // alternate as the two tiles' dP - Delta
    f32x16 d0, d1;
#pragma unroll
    for (int r = 0; r < 16; ++r) d1[r] = 0.0f;
    sync_issue(IC<0>{}, 0);
    ds_step(IC<0>{}, IC<1>{}, IC<0>{}, d0, d1);
    int t = 1;
    for (; t + 1 < ntiles; t += 2) {
      sync_issue(IC<1>{}, t);
      ds_step(IC<1>{}, IC<1>{}, IC<1>{}, d1, d0);
      sync_issue(IC<0>{}, t + 1);
      ds_step(IC<0>{}, IC<1>{}, IC<1>{}, d0, d1);
    }
    if (t < ntiles) {                        // t odd, ntiles = t + 1
      sync_issue(IC<1>{}, t);
      ds_step(IC<1>{}, IC<1>{}, IC<1>{}, d1, d0);
      sync_issue(IC<0>{}, ntiles);
      ds_step(IC<0>{}, IC<0>{}, IC<1>{}, d0, d1);
    } else {                                 // t = ntiles, odd
      sync_issue(IC<1>{}, ntiles);
      ds_step(IC<1>{}, IC<0>{}, IC<1>{}, d1, d0);
    }
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
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ KT, const float* __restrict__ L2,
    const float* __restrict__ Dl, uint16_t* __restrict__ dQ, int N, int nqb, int nb, int total, float c,
    float scale) {
  constexpr int CPR = D / 8;
  constexpr int NW = DQ_NT / 64;
  constexpr int TILE_CHUNKS = BC * CPR;            // row-major 64-key tile; also the d-major tile's size
  constexpr int LPW = TILE_CHUNKS / DQ_NT;         // DMA instructions per wave, tensor and tile
  constexpr int KB_BYTES = 32 * D * 2;
  __shared__ uint4 kbuf0[TILE_CHUNKS], kbuf1[TILE_CHUNKS], vbuf0[TILE_CHUNKS], vbuf1[TILE_CHUNKS];
  __shared__ uint4 tbuf0[TILE_CHUNKS], tbuf1[TILE_CHUNKS];

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

  // LDS byte offsets: K / V rows (A operand of S^T and dP^T, rows permuted) and
  // the d-major K tile (A operand of dQ^T: row 32 db + l32, chunk 2 kc + half)
  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  uint32_t toff[BC / 16];
#pragma unroll
  for (int kc = 0; kc < BC / 16; ++kc) toff[kc] = 16 * tchunk<BC>(l32, 2 * kc + half);

  const int kend = CAUSAL ? min(N, q0 + DQ_BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(KT + (size_t)bh * nb * D * TT), 0, (uint32_t)nb * D * TT * 2, 0x00020000);
  uint32_t row_off[LPW], t_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane;
    const int r = pos / CPR, ch = pos % CPR;
    row_off[i] = (uint32_t)(r * D + 8 * (ch ^ swz<D>(r))) * 2;
    const int d = pos / (BC / 8), cc = pos % (BC / 8);
    t_off[i] = (uint32_t)(d * TT * 2 + 16 * (cc ^ ((d >> 1) & 7)));
  }
  auto issue_tile = [&](int j0, uint4* kd, uint4* vd, uint4* td) {
    const uint32_t base = (uint32_t)j0 * D * 2;            // j0 is a multiple of TT: tile j0 / TT
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      lds_dma16(krs, kd + slot0, row_off[i], base);
      lds_dma16(vrs, vd + slot0, row_off[i], base);
      lds_dma16(trs, td + slot0, t_off[i], base);
    }
  };

  f32x16 dqa[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.0f;

  // one 64-key tile: register r of 32-key block kb is key j0 + 32 kb + 16 (r / 8) + 8 half + r % 8
  auto tile = [&](auto maskc, const char* kt, const char* vt, const char* tt, int j0) {
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
      for (int dc = 0; dc < D / 16; ++dc)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kt + koff[dc] + kb * KB_BYTES), qf[dc], s, 0, 0, 0);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(vt + koff[dc] + kb * KB_BYTES), of[dc], dp, 0, 0, 0);
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
        // dQ^T += K^T dS^T: A operand from the d-major K tile, keys 16 kc .. 16 kc + 15
        const int kc = 2 * kb + h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(tt + toff[kc] + db * 32 * BC * 2), b, dqa[db], 0, 0, 0);
      }
    }
  };

  // ANY = false: the tile is known to need no mask
  auto step = [&](auto anyc, int t, const uint4* kc, const uint4* vc, const uint4* tc, uint4* kn, uint4* vn,
                  uint4* tn) {
    const int j0 = t * BC;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    if (t + 1 < ntiles) issue_tile(j0 + BC, kn, vn, tn);
    if (CAUSAL && j0 > qw + 31) return;      // the whole tile is above this wave's diagonal
    const char* kt = reinterpret_cast<const char*>(kc);
    const char* vt = reinterpret_cast<const char*>(vc);
    const char* tt = reinterpret_cast<const char*>(tc);
    if (decltype(anyc)::value && ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw))) tile(IC<1>{}, kt, vt, tt, j0);
    else tile(IC<0>{}, kt, vt, tt, j0);
  };

  issue_tile(0, kbuf0, vbuf0, tbuf0);
  int t = 0;
  if (!CAUSAL)                               // only the last tile can need a mask: keep it out of the loop
    for (; t + 2 < ntiles; t += 2) {
      step(IC<0>{}, t, kbuf0, vbuf0, tbuf0, kbuf1, vbuf1, tbuf1);
      step(IC<0>{}, t + 1, kbuf1, vbuf1, tbuf1, kbuf0, vbuf0, tbuf0);
    }
  for (; t < ntiles; t += 2) {
    step(IC<1>{}, t, kbuf0, vbuf0, tbuf0, kbuf1, vbuf1, tbuf1);
    if (t + 1 < ntiles) step(IC<1>{}, t + 1, kbuf1, vbuf1, tbuf1, kbuf0, vbuf0, tbuf0);
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

// Workspace: LSE log2 e and Delta (float32 [B*H*N] each), then the d-major
// copies of Q, dO and K (bf16 [B*H][ceil(N/64)][d][64] each), 256-byte aligned.
struct Ws {
  float* l2;
  float* dl;
  uint16_t* qt;
  uint16_t* ot;
  uint16_t* kt;
  size_t bytes;
};

Ws carve(void* base, int B, int H, int N, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t f = up((size_t)B * H * N * sizeof(float));
  const size_t t = up((size_t)B * H * ((N + TT - 1) / TT) * d * TT * 2);
  char* p = static_cast<char*>(base);
  return Ws{reinterpret_cast<float*>(p), reinterpret_cast<float*>(p + f), reinterpret_cast<uint16_t*>(p + 2 * f),
            reinterpret_cast<uint16_t*>(p + 2 * f + t), reinterpret_cast<uint16_t*>(p + 2 * f + 2 * t),
            2 * f + 3 * t};
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, const Ws& w, int B, int H, int N, float scale, hipStream_t stream) {
  const long rows = (long)B * H * N;
  constexpr int RPB = 256 / (D / 8);
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  hipLaunchKernelGGL((attn_bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(o), dO, lse, w.l2, w.dl, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (N + TT - 1) / TT;
  const int tiles = B * H * nb;
  const XT3 xa{{Q, dO, K}, {w.qt, w.ot, w.kt}};
  hipLaunchKernelGGL((bwd_transpose_kernel<D>), dim3(3 * tiles), dim3(256), 0, stream, xa, N, nb, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c = (float)((double)scale * 1.4426950408889634);
  const int nkb = (N + KV_BK - 1) / KV_BK;
  const int tkv = nkb * B * H;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3(tkv), dim3(KV_NT), 0, stream, Q, K, V, dO, w.qt, w.ot,
                     w.l2, w.dl, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, nkb, nb, tkv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (N + DQ_BR - 1) / DQ_BR;
  const int tq = nqb * B * H;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3(tq), dim3(DQ_NT), 0, stream, Q, K, V, dO, w.kt, w.l2,
                     w.dl, static_cast<uint16_t*>(dq), N, nqb, nb, tq, c, scale);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) { return carve(nullptr, B, H, N, d).bytes; }

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
                                int d, float scale, bool causal, hipStream_t stream) {
  const Ws w = carve(workspace, B, H, N, d);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream)
                  : launch<128, false>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, N, scale, stream);
}

}  // namespace fa
