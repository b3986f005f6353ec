// Fused exact causal attention forward, head dimension 128, bf16 in / bf16
// out, float32 softmax, gfx950: the persistent ping-pong kernel.
//
// Method ("Flash Attention" glossary page, second paragraph; "FlashAttention-3
// (PT)", section "FlashAttention e FlashAttention-2"): the key/value sequence
// is walked tile by tile with a running row maximum and row sum (online
// softmax), the partial output is rescaled when the maximum grows, the 1/l
// normalisation is deferred to the end, and the score matrix never reaches
// HBM.  "FlashAttention-3 (PT)", section "Inovacoes tecnicas", item 1 hides
// slow steps such as the softmax behind the matrix products of another group
// of warps ("ping-pong" scheduling); this kernel does that with CDNA4 waves.
//
// gfx950 mapping:
//  * persistent: one workgroup per compute unit walks a static list of work
//    items (head, block of 256 query rows).  Heads are split into 8 sets, one
//    per XCD (workgroup g runs on XCD g % 8), so the workgroups of an XCD
//    stream the same heads' K/V through its L2; within a set the items go head
//    by head, longest query block first, dealt to the set's workgroups in
//    snake order, which gives every workgroup the same number of causal tiles.
//    No workgroup waits for a slot, and the two waves that share a SIMD
//    belong to the same workgroup, so neither finishes early.
//  * 8 waves = 2 groups of 4; waves w and w + 4 share a SIMD (measured), each
//    wave owns 32 query rows, and the 8 waves share every K/V tile in LDS.
//  * phases: in even phase 2j group 0 runs the matrix half
//    M(j) = { O^T += V_(j-1)^T P_(j-1)^T ; S_j^T = K_j Q^T } while group 1
//    runs the softmax of tile j-1; in odd phase 2j+1 the roles swap.  So each
//    SIMD has one wave on the matrix cores and one on the VALU.  An s_barrier
//    opens every even phase; the swap into the odd phase is not synchronised
//    (a wave goes on as soon as its own half is done), since no LDS buffer
//    changes hands there: the odd barrier only held early waves back.
//  * tiles of 64 keys are DMA'd HBM/L2 -> LDS (buffer_load ... lds, no
//    staging registers) into two K and two V buffers: K_j in phase 2j - 2,
//    V_j in phase 2j, each two phases before its first use; every even phase
//    boundary waits for the DMAs of two phases earlier.  The barrier is a
//    plain s_barrier: a __syncthreads() fence would wait for the DMAs just
//    issued.
//  * Q: each wave DMAs its own 32 rows of the next item into LDS during the
//    current item's last tiles and reads Q^T into registers at item start.
//  * scores are computed transposed, S^T = K Q^T, so each lane holds 16 keys
//    of one query (per-lane softmax state, one half-wave exchange); the output
//    is accumulated transposed, O^T += V^T P^T, with the score registers
//    rounded to bf16 as the B operand and V^T read from the row-major LDS tile
//    by ds_read_b64_tr_b16;
//  * exp2 with the scale folded into one FMA; the reference maximum only moves
//    when a tile's maximum exceeds it by more than 2^8 (exp2 domain).
#include "attn_bf16_common.h"

namespace fa {
namespace {

using namespace bf16k;

constexpr int D = 128;            // head dimension
constexpr int NWAVE = 8;          // waves per workgroup: two groups of four
constexpr int NT = 64 * NWAVE;    // threads per workgroup
constexpr int BR = 32 * NWAVE;    // query rows per work item (32 per wave)
constexpr int CPR = D / 8;        // 16-byte chunks per row
constexpr int TILE_CHUNKS = BC * CPR;
constexpr int LPW = TILE_CHUNKS / NT;   // DMA instructions per wave and tile

// S^T = K Q^T for one 64-key tile and this wave's 32 queries.
__device__ __forceinline__ void score_tile(const char* kt, const uint32_t (&koff)[D / 16], const bf16x8 (&qf)[D / 16],
                                           f32x16 (&s)[BC / 32]) {
  constexpr int KB_BYTES = 32 * D * 2;   // one 32-key block of the tile
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + koff[dc] + kb * KB_BYTES);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[kb], 0, 0, 0);
    }
  // keep 8 K-operand reads in flight ahead of the matrix ops
  constexpr int NMF = (D / 16) * (BC / 32);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < NMF - 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// O^T += V^T P^T for one 64-key tile.
__device__ __forceinline__ void pv_tile(const char* vt, const uint32_t (&voff)[D / 32][2], const bf16x8 (&pb)[BC / 16],
                                        f32x16 (&acc)[D / 32]) {
  constexpr int KC_BYTES = 16 * D * 2;   // one 16-key chunk of the tile
#pragma unroll
  for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x4_t v0 = tr_read(vt + voff[db][0] + kc * KC_BYTES);
      const bf16x4_t v1 = tr_read(vt + voff[db][1] + kc * KC_BYTES);
      const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], acc[db], 0, 0, 0);
    }
  // keep 8 transposed reads (4 matrix ops' operands) in flight
  constexpr int NMF = (D / 32) * (BC / 16);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < NMF - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Both products of a matrix half, O^T += V_(j-1)^T P_(j-1)^T and
// S_j^T = K_j Q^T, with their matrix ops alternating.  The P V operands come
// through the slower transposed LDS reads and the S operands through 16-byte
// reads; alternating the two streams spreads the LDS traffic evenly over the
// matrix work instead of running the LDS-heavy half first, and the matrix core
// never drains between the two products.
__device__ __forceinline__ void pv_score_tile(const char* vt, const char* kt, const uint32_t (&voff)[D / 32][2],
                                              const uint32_t (&koff)[D / 16], const bf16x8 (&pb)[BC / 16],
                                              const bf16x8 (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                              f32x16 (&s)[BC / 32]) {
  constexpr int KB_BYTES = 32 * D * 2;   // one 32-key block of the K tile
  constexpr int KC_BYTES = 16 * D * 2;   // one 16-key chunk of the V tile
  constexpr int NSTEP = (D / 32) * (BC / 16);
  static_assert(NSTEP == (D / 16) * (BC / 32), "both products have the same number of matrix ops");
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    const int kc = i / (D / 32), db = i % (D / 32);
    const bf16x4_t v0 = tr_read(vt + voff[db][0] + kc * KC_BYTES);
    const bf16x4_t v1 = tr_read(vt + voff[db][1] + kc * KC_BYTES);
    const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], acc[db], 0, 0, 0);
    const int dc = i / (BC / 32), kb = i % (BC / 32);
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + koff[dc] + kb * KB_BYTES);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[kb], 0, 0, 0);
  }
  // three steps of reads (2 transposed + 1 plain each) in flight ahead of the matrix ops
  __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
  for (int i = 0; i < NSTEP - 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
}

// p = exp2(c s - m2) for this lane's 32 scores of one tile, rounded to bf16
// as the B operand of P V; returns the lane's float32 sum of p (summing the
// bf16-rounded p would cost up to 2^-9 relative in l, i.e. in LSE, on rows
// with few keys).  Masked keys give exact zeros, also when c = 0.
template <bool MASK>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 16], float m2, float c) {
  float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float s0 = s[kc >> 1][8 * (kc & 1) + e], s1 = s[kc >> 1][8 * (kc & 1) + e + 1];
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -m2));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -m2));
      if (MASK) {
        p0 = s0 == -INFINITY ? 0.0f : p0;
        p1 = s1 == -INFINITY ? 0.0f : p1;
      }
      rs[e >> 1] += p0 + p1;
      pb[kc][e] = (__bf16)p0;
      pb[kc][e + 1] = (__bf16)p1;
    }
  return (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// Online softmax of one tile: mask (MASK: the tile crosses this wave's
// diagonal or the end of the sequence), p against the running reference
// maximum m2, and the row sum.  The reference only has to keep every p
// finite and in range, so the tile maximum is not formed on the common path:
// p is computed against the current m2 first, and only if a lane's sum of its
// 32 p exceeds 2^8 (some p may be above 2^8), or is not finite (the first
// tile, where m2 = -inf), does the wave form the tile maximum, move m2 to it,
// rescale O and l, and compute p again.  A lane sum of at most 2^8 bounds each
// of its p by 2^8, which is exact in float32 and in bf16 range.
template <bool MASK>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 16], f32x16 (&acc)[D / 32],
                                             float& m2, float& lsum, float c, int j0, int qi, int N, int half) {
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
        if (key >= N || key > qi) s[kb][r] = -INFINITY;
      }
  }
  float part = exp_tile<MASK>(s, pb, m2, c);
  if (__any(!(part <= 256.0f))) {
    float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // 4 independent chains
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pm[(kb * 2 + (r >> 3)) & 3] = fmaxf(pm[(kb * 2 + (r >> 3)) & 3], s[kb][r]);
    float tmax = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
    tmax = wave_halves_max(tmax);
    const float tm2 = tmax * c;
    if (tm2 > m2) {
      const float alpha = __builtin_amdgcn_exp2f(m2 - tm2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m2 = tm2;
    }
    part = exp_tile<MASK>(s, pb, m2, c);
  }
  lsum += part;
}

__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int nqb, int BH, int groups, float c,
    uint32_t qflip) {
  // Separate objects, so that the compiler never orders a read of one buffer
  // after a DMA into the other.  The larger alignment places the four tile
  // buffers ahead of the Q rows, in the first 64 KB of LDS, where every tile
  // read addresses its buffer through the 16-bit immediate offset instead of
  // a per-read address add.
  __shared__ __attribute__((aligned(256))) uint4 kbuf0[TILE_CHUNKS], kbuf1[TILE_CHUNKS];
  __shared__ __attribute__((aligned(256))) uint4 vbuf0[TILE_CHUNKS], vbuf1[TILE_CHUNKS];
  __shared__ uint4 qsm[BR * CPR];            // the item's Q rows (swizzled), each wave's own 32 rows

  // Static work list: workgroup g serves heads [xg * hx, (xg + 1) * hx) with
  // the other workgroups of its set; item k of the set is (head k / nqb, query
  // block nqb - 1 - k % nqb); round r hands item r * S + s (even r) or
  // r * S + S - 1 - s (odd r) to the set's workgroup s.
  const int G = gridDim.x, g = blockIdx.x;
  const int xg = g % groups, sl = g / groups, S = G / groups;
  const int hx = BH / groups, nloc = hx * nqb;
  auto item = [&](int r, int& bh, int& qb) -> bool {
    const int k = r * S + ((r & 1) ? S - 1 - sl : sl);
    if (k >= nloc) return false;
    const int hl = k / nqb;
    bh = xg * hx + hl;
    qb = nqb - 1 - (k - hl * nqb);
    return true;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;

  // Q rows: each wave DMAs its own 32 rows; row r's chunk cc sits at
  // r * CPR + (cc ^ (r % CPR)), so the 16-byte reads below are conflict-free.
  constexpr int QPW = 32 * CPR / 64;         // Q DMA instructions per wave
  uint32_t q_lane_off[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int pos = i * 64 + lane, rl = pos / CPR, cc = (pos % CPR) ^ (rl % CPR);
    q_lane_off[i] = (uint32_t)((32 * wave + rl) * D + 8 * cc) * 2;
  }
  auto issue_q = [&](int bh, int qb) {       // rows past N read as zeros
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Q + (size_t)bh * N * D), 0, (uint32_t)N * D * 2, 0x00020000);
    const uint32_t base = (uint32_t)(qb * BR) * D * 2;
#pragma unroll
    for (int i = 0; i < QPW; ++i) lds_dma16(qrs, &qsm[wave * 32 * CPR + i * 64], q_lane_off[i], base);
  };
  bf16x8 qf[D / 16];                         // Q^T B operand: query qi, dims 16*dc + 8*half + 0..7
  auto read_q = [&]() {
    const int r = 32 * wave + l32;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      uint4 u = qsm[r * CPR + ((2 * dc + half) ^ (r % CPR))];
      u.x ^= qflip; u.y ^= qflip; u.z ^= qflip; u.w ^= qflip;   // negative scale: negate Q
      qf[dc] = __builtin_bit_cast(bf16x8, u);
    }
  };

  // this lane's LDS byte offsets: K operand rows (first 32-key block) ...
  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
  // ... and transposed V reads (first 16-key chunk; keys +0..3 and +4..7)
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

  // K/V tile DMA: instruction i of wave w fills the 64 consecutive 16-byte
  // slots starting at (i * NWAVE + w) * 64, each lane the global chunk that
  // the swizzled layout keeps in its slot; the tile's start goes in soffset.
  const uint32_t nbytes = (uint32_t)N * D * 2;
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NWAVE + wave) * 64 + lane, row = pos / CPR, slot = pos % CPR;
    lane_off[i] = (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2;
  }
  auto issue_tile = [&](const uint16_t* T, uint4* dst, int bh, int j0) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(T + (size_t)bh * N * D), 0, nbytes, 0x00020000);
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) lds_dma16(rs, dst + (i * NWAVE + wave) * 64, lane_off[i], base);
  };

  int bh, qb;
  item(0, bh, qb);                           // the grid never exceeds the number of items
  issue_tile(K, kbuf0, bh, 0);
  issue_q(bh, qb);
  __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
  __syncthreads();

  for (int r = 0;; ++r) {
    int nbh = 0, nqbk = 0;
    const bool more = item(r + 1, nbh, nqbk);
    const int q0 = qb * BR;
    const int qw = q0 + 32 * wave;           // first query row of this wave
    const int qi = qw + l32;                 // this lane's query
    const int ntiles = (min(N, q0 + BR) + BC - 1) / BC;
    const int nt2 = (ntiles + 1) & ~1;       // even: the buffers restart at 0 with every item

    read_q();                                // landed: waited for at the previous even boundary
    FA_SYNC_POINT();
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    float m2 = -INFINITY;   // reference maximum, exp2 domain (c * raw score)
    float lsum = 0.0f;      // this half-wave's share of the row sum
    f32x16 s[BC / 32];
    bf16x8 pb[BC / 16];

    // tile j holds keys this wave sees (tiles wholly above its diagonal are skipped)
    auto active = [&](int j) { return j < ntiles && j * BC <= qw + 31; };
    auto epilogue = [&]() {                  // O = O / l, LSE = ln 2 * (m2 + log2 l)
      const float ltot = wave_halves_sum(lsum);
      if (qi < N) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = O + (size_t)bh * N * D + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * db + 8 * a + 4 * half;
            const bf16x4_t w = {(__bf16)(acc[db][4 * a + 0] * inv), (__bf16)(acc[db][4 * a + 1] * inv),
                                (__bf16)(acc[db][4 * a + 2] * inv), (__bf16)(acc[db][4 * a + 3] * inv)};
            *reinterpret_cast<bf16x4_t*>(orow + d0) = w;
          }
        if (half == 0) LSE[(size_t)bh * N + qi] = (m2 + __log2f(ltot)) * 0.69314718055994531f;
      }
    };

    // Phase p of the item (tile j = p / 2, JP = j & 1).  The item has
    // 2 * nt2 + 2 phases; group 0 runs M(j) in phase 2j, group 1 in 2j + 1.
    auto phase = [&](int p, auto jpc) {
      constexpr int JP = decltype(jpc)::value;
      const int j = p >> 1;
      const bool odd = p & 1;
      if (!odd) {
        if (p != 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the DMAs of phase p - 2 landed
        __asm__ volatile("s_barrier" ::: "memory");
      }
      uint4* const kcur = JP ? kbuf1 : kbuf0;   // K_j
      uint4* const knext = JP ? kbuf0 : kbuf1;  // K_(j+1)
      uint4* const vcur = JP ? vbuf1 : vbuf0;   // V_j (loaded now, read in phases 2j + 2, 2j + 3)
      uint4* const vprev = JP ? vbuf0 : vbuf1;  // V_(j-1)
      if (!odd) {
        if (j + 1 < ntiles) issue_tile(K, knext, bh, (j + 1) * BC);
        else if (j + 1 == nt2 && more) {     // the next item's first K tile and Q rows
          issue_tile(K, knext, nbh, 0);
          issue_q(nbh, nqbk);
        }
        if (j < ntiles) issue_tile(V, vcur, bh, j * BC);
      }
      FA_SYNC_POINT();
      if ((grp == 0) == !odd) {              // matrix half
        const bool do_pv = j >= 1 && active(j - 1), do_s = active(j);
        if (do_pv && do_s) {
          pv_score_tile(reinterpret_cast<const char*>(vprev), reinterpret_cast<const char*>(kcur), voff, koff, pb, qf,
                        acc, s);
        } else {
          if (do_pv) pv_tile(reinterpret_cast<const char*>(vprev), voff, pb, acc);
          if (do_s) score_tile(reinterpret_cast<const char*>(kcur), koff, qf, s);
        }
        if (j == nt2) epilogue();
      } else {                               // softmax half: tile j (group 0) or j - 1 (group 1)
        const int js = odd ? j : j - 1;
        if (js >= 0 && active(js)) {
          const int j0 = js * BC;
          if ((j0 + BC > N) || (j0 + BC - 1 > qw))
            softmax_tile<true>(s, pb, acc, m2, lsum, c, j0, qi, N, half);
          else
            softmax_tile<false>(s, pb, acc, m2, lsum, c, j0, qi, N, half);
        }
      }
      FA_SYNC_POINT();
    };
    for (int j = 0; j < nt2; j += 2) {
      phase(2 * j, IC<0>{});
      phase(2 * j + 1, IC<0>{});
      phase(2 * j + 2, IC<1>{});
      phase(2 * j + 3, IC<1>{});
    }
    phase(2 * nt2, IC<0>{});
    phase(2 * nt2 + 1, IC<0>{});

    if (!more) break;
    bh = nbh;
    qb = nqbk;
  }
}

}  // namespace

hipError_t launch_attn_bf16_pp(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int N, float scale, hipStream_t stream) {
  const int nqb = (N + BR - 1) / BR;
  const int BH = B * H;
  const int total = nqb * BH;
  // one persistent workgroup per resident slot, never more than there are items
  const long slots = device_slots(reinterpret_cast<const void*>(&attn_fwd_bf16_pp_kernel), NT);
  if (slots <= 0) return hipErrorInvalidDevice;
  int grid = total < slots ? total : (int)slots;
  int groups = 1;
  if (BH % 8 == 0 && grid >= 8) {            // one head set per XCD
    grid -= grid % 8;
    groups = 8;
  }
  const float c = (float)((double)__builtin_fabsf(scale) * 1.4426950408889634);
  const uint32_t qflip = scale < 0.0f ? 0x80008000u : 0u;
  hipLaunchKernelGGL(attn_fwd_bf16_pp_kernel, dim3(grid), dim3(NT), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                     lse, N, nqb, BH, groups, c, qflip);
  return hipGetLastError();
}

}  // namespace fa
