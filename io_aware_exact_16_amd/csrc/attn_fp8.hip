// Fused exact attention forward on per-block-scaled E4M3 operands, gfx950.
//
// The FP8 variant of the method ("FlashAttention-3 (PT)", section "Inovacoes
// tecnicas", item 3: FP8 doubles the matrix throughput; Q and K are made
// incoherent with an orthogonal Hadamard transform before quantisation, which
// leaves Q K^T unchanged) with the same tiling / online softmax as the bf16
// kernel ("Flash Attention" glossary page, second paragraph).
//
// Persistent: one workgroup (4 waves, 128 query rows per work item) per
// resident slot, three slots per compute unit for causal attention, walking a
// static balanced list of (head, query block) items grouped per XCD.
//
// Inputs are E4M3 codes with one float32 scale per (b, h, 128-token block).
//  * S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales)
//    over the codes; the two block scales fold into the softmax constant of
//    the tile: c_t = |scale| log2(e) s_q s_k.
//  * P is quantised to E4M3 for the second product jointly with the V-block
//    scale relative to the head's largest: s_v / max s_v = 2^E r with
//    E = ceil(log2 of the ratio) and 1/2 < r <= 1; P holds E4M3(128 p r) and
//    the power of two 2^E goes in as the E8M0 block scale of the V operand of
//    v_mfma_scale_f32_32x32x64_f8f6f4.  One accumulator serves every V block,
//    128 p r stays in E4M3's normal range whatever the blocks' magnitudes (an
//    all-zero block has s_v = 1), and in the block with the largest scale
//    r = 1, so a row's largest weight is stored exactly.  The factor 128 r is
//    folded into the exp2 argument (no extra multiply), l accumulates
//    p = P / (128 r) in float32, and O = acc max s_v / (128 l).  The per-block
//    constants are formed once per 128-key block (two tiles).  (A power-of-two
//    factor only shifts E4M3's grid: 128 stores every normal-range weight as
//    256 would; it moves the subnormal start from 2^-14 to 2^-13 of the
//    reference and buys one more binade of slack below.)
//  * The reference maximum moves only when a tile's maximum exceeds it by
//    more than 1.8 in the exp2 domain, so p <= 2^1.8 and 128 p r <= 445.7,
//    inside E4M3 range (448).  On inputs with large outliers a wave's 32 rows
//    moved it (and rescaled O) on about half of the tiles at a slack of 0.8;
//    at 1.8 that is rare.
//  * Layouts as in the bf16 kernel (S^T and O^T accumulators; per-lane
//    softmax state).  32x32x64 FP8 MFMA operands: lane l holds row (col)
//    l % 32; its bytes 0..15 are k = 16 (l / 32) + 0..15 and bytes 16..31 are
//    k = 32 + 16 (l / 32) + 0..15 (measured through the E8M0 block scales, whose
//    32-element blocks are k = 0..31 and 32..63).  V^T comes
//    from the row-major LDS tile through ds_read_b64_tr_b8: within each
//    16-lane group, lane 2r + c names the 8 bytes at [r][8c..8c+7] of an
//    8 x 16 byte tile and lane j receives column j (verified on gfx950).
#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int D = 128;    // head dimension (bytes per row)
constexpr int BR = 128;   // query rows per workgroup = one scaling block
constexpr int BC = 64;    // key rows per tile (half a scaling block)
constexpr int NT = 256;   // threads per workgroup
constexpr int QBLK = 128; // tokens per scaling block

// Position (16-byte units) of chunk ch (0..7) of tile row `row` in LDS.  The
// XOR swizzle makes both read patterns conflict-free: 16 lanes reading 16 B
// of 16 different rows (K operand) and 32 lanes reading 8 B from 8 rows x 2
// chunks (transposed V operand).
__device__ __forceinline__ int lds_chunk8(int row, int ch) {
  const int s = (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
  return row * (D / 16) + (ch ^ s);
}

// Same A-row to key permutation as the bf16 kernel: the accumulator registers
// 0..7 (8..15) of half-wave h then hold keys 8h + r (16 + 8h + r - 8).
__device__ __forceinline__ int key_of_arow(int m) {
  return (m & 0x13) | ((m >> 1) & 0x4) | ((m << 1) & 0x8);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset + soffset, 0, 0, 0);
}

__device__ __forceinline__ i32x2 tr8_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // E4M3 x E4M3 (format code 0 for both), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Same product with the A operand's values multiplied by 2^(ea - 127) (E8M0
// block scale in byte 0 of ea, the same for every lane and 32-element block).
__device__ __forceinline__ f32x16 mfma_fp8_scaled_a(const i32x8& a, const i32x8& b, const f32x16& c, int ea) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, 127);
}

// S-product variant with both operands scaled per lane (MX-style E8M0 scales
// of the 32 coordinates each lane holds, in byte 0 of sa / sb).
__device__ __forceinline__ f32x16 mfma_fp8_scaled_ab(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa,
                                                     uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voffset + soffset, 0, 0, 0);
}

// O = O' H / sqrt(d) for the Hadamard variant of V (the normalised Sylvester
// matrix is symmetric and its own inverse), on this lane's half of one
// query's output: register r = 4a + e of acc[db] holds coordinate
// 32 db + 8 a + 4 half + e, so six of the seven butterfly stages are in
// registers and the stage over coordinate bit 2 pairs lane l with l ^ 32.
// The 1 / sqrt(d) is left to the caller.
__device__ __forceinline__ void fwht_o(f32x16 (&acc)[4], int half) {
#pragma unroll
  for (int bit = 1; bit < 16; bit <<= 1) {   // e bits (coordinate bits 0, 1), a bits (3, 4)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(r & bit)) {
          const float x = acc[db][r], y = acc[db][r | bit];
          acc[db][r] = x + y;
          acc[db][r | bit] = x - y;
        }
  }
#pragma unroll
  for (int bit = 1; bit < 4; bit <<= 1)      // db bits (coordinate bits 5, 6)
#pragma unroll
    for (int db = 0; db < 4; ++db)
      if (!(db & bit)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = acc[db][r], y = acc[db | bit][r];
          acc[db][r] = x + y;
          acc[db | bit][r] = x - y;
        }
      }
  const float sgn = half ? -1.0f : 1.0f;     // coordinate bit 2: half 0 keeps x + y, half 1 keeps x - y
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t u = __float_as_uint(acc[db][r]);
      const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      // p[0]: the lower half-wave's value of this column, p[1]: the upper one's
      acc[db][r] = __builtin_fmaf(__uint_as_float(p[1]), sgn, __uint_as_float(p[0]));
    }
}

// Constants of one 128-key block: c_t = softmax constant with the Q and K
// block scales folded in; lr = log2(P_SCALE r); inv_r = 1 / (P_SCALE r); ve = E8M0
// code of 2^E, where s_v / max s_v = 2^E r, 1/2 < r <= 1.  A ratio below
// 2^-127 leaves part of its magnitude in r, which then loses precision in P's
// subnormals (such a block's contribution is below 2^-118 of the largest).
constexpr float P_SCALE = 128.0f;      // P holds E4M3(P_SCALE p r)
constexpr float P_SCALE_LOG2 = 7.0f;

struct BlockK {
  float c_t, lr, inv_r;
  int ve;
};

__device__ __forceinline__ BlockK block_consts(float c_q, float ks, float ratio) {
  int E;
  float r = frexpf(ratio, &E);               // ratio = r 2^E, 1/2 <= r < 1
  if (r == 0.5f) {                           // a power of two: r = 1
    r = 1.0f;
    E -= 1;
  }
  if (E < -127) {
    r = ldexpf(r, E + 127);
    E = -127;
  }
  BlockK b;
  b.c_t = c_q * ks;
  b.lr = P_SCALE_LOG2 + __log2f(r);
  b.inv_r = 1.0f / (P_SCALE * r);
  b.ve = E + 127;
  return b;
}

__device__ __forceinline__ float wave_halves_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float wave_halves_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int V>
struct IC {
  static constexpr int value = V;
};

constexpr float P_SLACK = 1.8f;   // log2 of the allowed growth of p above 1: P_SCALE 2^1.8 <= 448

constexpr int VMCNT(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// One 64-key tile of one wave, with the constants of its 128-key block.
template <bool CAUSAL, bool MASK, bool MX>
__device__ __forceinline__ void tile_math(const char* kt, const char* vt, const uint32_t (&koff)[2][2],
                                          const uint32_t (&voff)[4], const i32x8 (&qf)[2], f32x16 (&acc)[4],
                                          float& m2, float& lsum, const BlockK& bk, int j0, int qi, int N,
                                          int half, const uint32_t* kmx, int arow, uint32_t qsc) {
  const float c_t = bk.c_t;
  // MX: the E8M0 scales of this lane's K row (4 per key, one per 32 coordinates),
  // shifted so that byte 2 dc holds the group of d-chunk dc this lane reads
  uint32_t kw[2] = {0u, 0u};
  if (MX) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kw[kb] = kmx[arow + 32 * kb] >> (8 * half);
  }
  constexpr int KB_BYTES = 32 * D;   // one 32-key block of the tile
  constexpr int KG_BYTES = 16 * D;   // 16 keys
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int dc = 0; dc < 2; ++dc)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(kt + koff[dc][0] + kb * KB_BYTES);
      const uint4 a1 = *reinterpret_cast<const uint4*>(kt + koff[dc][1] + kb * KB_BYTES);
      const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      if (MX)
        s[kb] = mfma_fp8_scaled_ab(a, qf[dc], s[kb], kw[kb] >> (16 * dc), qsc >> (16 * dc));
      else
        s[kb] = mfma_fp8(a, qf[dc], s[kb]);
    }

  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
        if (key >= N || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
      }
  }
  float pm[2] = {-INFINITY, -INFINITY};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) pm[kb] = fmaxf(pm[kb], s[kb][r]);
  const float tm2 = wave_halves_max(fmaxf(pm[0], pm[1])) * c_t;
  // The reference moves only when the tile maximum exceeds it by more than
  // P_SLACK (exp2 domain), so p <= 2^1.8 < 3.49 and 128 r p <= 445.7 stays
  // inside E4M3 range (448); moving it on every growth of any row's maximum
  // would rescale O on most early tiles.
  if (__any(tm2 > m2 + P_SLACK)) {
    const float mnew = fmaxf(m2, tm2);
    const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    lsum *= alpha;
    m2 = mnew;
  }

  // P'' = 128 r exp2(c_t s - m2), quantised to E4M3 (round to nearest even);
  // the byte for key slot e of the B operand comes from register (e / 16, e % 16)
  const float off = bk.lr - m2;
  i32x8 pq;
  float rs[2];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float p[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float sv = s[w >> 2][4 * (w & 3) + y];
      p[y] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c_t, off));
      if (MASK) p[y] = sv == -INFINITY ? 0.0f : p[y];
    }
    const float g = (p[0] + p[1]) + (p[2] + p[3]);
    rs[w & 1] = w < 2 ? g : rs[w & 1] + g;
    // the first convert fills bytes 0..1 and the second bytes 2..3, so the
    // register's old contents do not matter: p[0]'s bits (dead after this)
    // stand in for them and no zero has to be materialised
    uint32_t b = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
    pq[w] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], b, true);
  }
  lsum += (rs[0] + rs[1]) * bk.inv_r;

  // O^T += V^T P^T: the A operand for d-block db gathers keys 16g + 8h + 0..7 (g = 0..3)
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    i32x8 va;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const i32x2 v = tr8_read(vt + voff[db] + g * KG_BYTES);
      va[2 * g] = v[0];
      va[2 * g + 1] = v[1];
    }
    acc[db] = mfma_fp8_scaled_a(va, pq, acc[db], bk.ve);
  }
}

template <bool CAUSAL, bool MX, bool VHAD>
// Three waves per SIMD for causal attention: this kernel is bound by its
// softmax VALU work, and a third resident wave fills more of the VALU's idle
// cycles (the causal build fits 168 VGPRs, spilling one value used only at
// the start and in the epilogue); the non-causal build would spill in its tile
// loop at that bound and keeps two.
__global__ __launch_bounds__(NT, CAUSAL ? 3 : 2) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    const uint8_t* __restrict__ QMX, const uint8_t* __restrict__ KMX, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int nqb, int BH, int groups, float c0, uint32_t qflip) {
  constexpr int TILE_CHUNKS = BC * D / 16;   // 16-byte chunks per K (or V) tile
  constexpr int NW = NT / 64;
  constexpr int LPW = TILE_CHUNKS / NT;      // DMA instructions per wave, tensor and tile
  __shared__ uint4 smem[2][2][TILE_CHUNKS];  // [buffer][K | V][chunk]
  __shared__ uint32_t kmxs[MX ? 2 : 1][MX ? BC : 1];   // MX: the K tile's E8M0 scales, 4 per key

  // Persistent: workgroup g walks a static list of work items (head, block of
  // 128 query rows).  Heads are split into `groups` sets (8 when the heads
  // divide evenly: workgroup g runs on XCD g % 8, so the workgroups of an XCD
  // stream the same heads' K/V through its L2); within a set the items go head
  // by head, each head's blocks longest first, dealt to the set's workgroups in
  // snake order (s, S - 1 - s, s, ...), which balances the causal work.  Every
  // slot stays occupied until the list runs out (a grid of one workgroup per
  // item left a third of the slots idle in launch gaps and the tail).
  const int G = gridDim.x, g = blockIdx.x;
  const int xg = g % groups, sl = g / groups, S = G / groups;
  const int hx = BH / groups, nloc = hx * nqb;
  auto item = [&](int r, int& bh_, int& qb_) -> bool {
    const int k = r * S + ((r & 1) ? S - 1 - sl : sl);
    if (k >= nloc) return false;
    const int hl = k / nqb;
    bh_ = xg * hx + hl;
    qb_ = k - hl * nqb;
    if (CAUSAL) qb_ = nqb - 1 - qb_;         // longest query blocks first
    return true;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nsb = (N + QBLK - 1) / QBLK;     // scaling blocks per head
  const int arow = key_of_arow(l32);

  // this lane's LDS byte offsets: K operand rows (two 16-byte chunks per d-half) ...
  uint32_t koff[2][2];
#pragma unroll
  for (int dc = 0; dc < 2; ++dc)
#pragma unroll
    for (int i = 0; i < 2; ++i)   // the same 16-byte chunks of the key row as Q's (see below)
      koff[dc][i] = 16 * lds_chunk8(key_of_arow(l32), MX ? 4 * dc + 2 * i + half : 4 * dc + 2 * half + i);
  // ... and 8-bit transposed V reads (keys 8*(G/2) + r of the first group, d-block db)
  uint32_t voff[4];
  {
    const int GG = lane >> 4, j = lane & 15, r = j >> 1, cc = j & 1;
    const int key = 8 * (GG >> 1) + r;
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] = 16 * lds_chunk8(key, 2 * db + (GG & 1)) + 8 * cc;
  }
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane, row = pos / (D / 16), slot = pos % (D / 16);
    const int sw = (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
    lane_off[i] = (uint32_t)(row * D + 16 * (slot ^ sw));
  }

  for (int r = 0;; ++r) {
    int bh, qb;
    if (!item(r, bh, qb)) break;
    const int q0 = qb * BR;
    const int qw = q0 + 32 * wave;
    const int qi = qw + l32;
    const size_t hoff = (size_t)bh * N * D;
    const float* vsh = VS + (size_t)bh * nsb;
    const float* ksh = KS + (size_t)bh * nsb;

    // largest V-block scale of the head (every lane of the wave ends with it)
    float svmax = 0.0f;
    for (int i = lane; i < nsb; i += 64) svmax = fmaxf(svmax, vsh[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) svmax = fmaxf(svmax, __shfl_xor(svmax, off));
    const float c_q = c0 * QS[(size_t)bh * nsb + q0 / QBLK];

    // Q^T as the B operand: lane holds query qi and two 16-byte chunks of d-chunk
    // dc.  The matrix instruction takes bytes 0..15 of half-wave h as k = 16 h +
    // 0..15 and bytes 16..31 as k = 32 + 16 h + 0..15; any placement shared by Q
    // and K gives the same product, and the MX variant needs k = d - 64 dc, so
    // that each 32-element scale block is one group of 32 coordinates.  Without
    // MX the lane holds d = 64 dc + 32 half + 0..31, with MX
    // d = 64 dc + 16 half + 0..15 and 64 dc + 32 + 16 half + 0..15.
    i32x8 qf[2];
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      uint4 u0 = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
      if (qi < N) {
        const uint8_t* row = Q8 + hoff + (size_t)qi * D + 64 * dc;
        u0 = *reinterpret_cast<const uint4*>(row + (MX ? 16 * half : 32 * half));
        u1 = *reinterpret_cast<const uint4*>(row + (MX ? 32 + 16 * half : 32 * half + 16));
      }
      qf[dc] = i32x8{(int)(u0.x ^ qflip), (int)(u0.y ^ qflip), (int)(u0.z ^ qflip), (int)(u0.w ^ qflip),
                     (int)(u1.x ^ qflip), (int)(u1.y ^ qflip), (int)(u1.z ^ qflip), (int)(u1.w ^ qflip)};
    }

    // MX: this query's four E8M0 scales, shifted so that byte 2 dc holds the group of d-chunk dc
    uint32_t qsc = 0;
    if (MX) {
      const uint32_t qmx = qi < N ? *reinterpret_cast<const uint32_t*>(QMX + ((size_t)bh * N + qi) * 4) : 0x7F7F7F7Fu;
      qsc = qmx >> (8 * half);
    }
    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;

    const uint32_t nbytes = (uint32_t)N * D;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K8 + hoff), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V8 + hoff), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kmxrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(MX ? KMX + (size_t)bh * N * 4 : K8), 0, (uint32_t)N * 4, 0x00020000);
    auto issue_tile = [&](int j0, auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      const uint32_t base = (uint32_t)j0 * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int slot0 = (i * NW + wave) * 64;
        lds_dma16(krs, &smem[BUF][0][slot0], lane_off[i], base);
        lds_dma16(vrs, &smem[BUF][1][slot0], lane_off[i], base);
      }
      if (MX && wave == 0) lds_dma4(kmxrs, &kmxs[MX ? BUF : 0][0], 4 * lane, (uint32_t)j0 * 4);   // 64 keys x 4 B
    };

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    float m2 = -INFINITY, lsum = 0.0f;

    auto step = [&](int t, const BlockK& bk, auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      const int j0 = t * BC;
      __builtin_amdgcn_s_waitcnt(VMCNT(0));
      __syncthreads();
      if (t + 1 < ntiles) issue_tile(j0 + BC, IC<BUF ^ 1>{});
      FA_SYNC_POINT();
      if (CAUSAL && j0 > qw + 31) return;
      const char* kt = reinterpret_cast<const char*>(&smem[BUF][0][0]);
      const char* vt = reinterpret_cast<const char*>(&smem[BUF][1][0]);
      const uint32_t* km = &kmxs[MX ? BUF : 0][0];
      if ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw))
        tile_math<CAUSAL, true, MX>(kt, vt, koff, voff, qf, acc, m2, lsum, bk, j0, qi, N, half, km, arow, qsc);
      else
        tile_math<CAUSAL, false, MX>(kt, vt, koff, voff, qf, acc, m2, lsum, bk, j0, qi, N, half, km, arow, qsc);
    };

    issue_tile(0, IC<0>{});
    for (int t = 0; t < ntiles; t += 2) {       // tiles t and t + 1 share one 128-key scaling block
      const BlockK bk = block_consts(c_q, ksh[t / 2], vsh[t / 2] / svmax);
      step(t, bk, IC<0>{});
      if (t + 1 < ntiles) step(t + 1, bk, IC<1>{});
    }

    // epilogue: O = acc max s_v / (128 l) (then H / sqrt(d) for the Hadamard
    // variant of V), LSE = ln 2 * (m2 + log2 l)
    const float ltot = wave_halves_sum(lsum);
    if (VHAD) fwht_o(acc, half);               // every lane, before the row guard: the stage pairs lanes
    if (qi < N) {
      const float f = svmax / (P_SCALE * ltot) * (VHAD ? 0.08838834764831845f : 1.0f);   // 1 / sqrt(128)
      uint16_t* orow = O + hoff + (size_t)qi * D;
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d0 = 32 * db + 8 * a + 4 * half;
          const bf16x4_t w = {(__bf16)(acc[db][4 * a + 0] * f), (__bf16)(acc[db][4 * a + 1] * f),
                              (__bf16)(acc[db][4 * a + 2] * f), (__bf16)(acc[db][4 * a + 3] * f)};
          *reinterpret_cast<bf16x4_t*>(orow + d0) = w;
        }
      if (half == 0) LSE[(size_t)bh * N + qi] = (m2 + __log2f(ltot)) * 0.69314718055994531f;
    }
    __syncthreads();                         // every wave is done with the tile buffers before the next item's DMA
  }
}

template <bool CAUSAL, bool MX, bool VHAD>
hipError_t launch(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* qs, const float* ks,
                  const float* vs, const uint8_t* qmx, const uint8_t* kmx, void* o, float* lse, int B, int H, int N,
                  float scale, hipStream_t stream) {
  const int nqb = (N + BR - 1) / BR;
  const int BH = B * H;
  const long total = (long)nqb * BH;
  const float c0 = (float)((double)__builtin_fabsf(scale) * 1.4426950408889634);
  const uint32_t qflip = scale < 0.0f ? 0x80808080u : 0u;
  // one persistent workgroup per resident slot, never more than there are items
  const long slots = device_slots(reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<CAUSAL, MX, VHAD>), NT);
  if (slots <= 0) return hipErrorInvalidDevice;
  int grid = total < slots ? (int)total : (int)slots;
  int groups = 1;
  if (BH % 8 == 0 && grid >= 8) {            // one head set per XCD
    grid -= grid % 8;
    groups = 8;
  }
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, MX, VHAD>), dim3(grid), dim3(NT), 0, stream, q8, k8, v8, qs, ks,
                     vs, qmx, kmx, static_cast<uint16_t*>(o), lse, N, nqb, BH, groups, c0, qflip);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_c(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* qs, const float* ks,
                    const float* vs, const uint8_t* qmx, const uint8_t* kmx, bool vhad, void* o, float* lse, int B,
                    int H, int N, float scale, hipStream_t stream) {
  const bool mx = qmx != nullptr;
  if (mx) return vhad ? launch<CAUSAL, true, true>(q8, k8, v8, qs, ks, vs, qmx, kmx, o, lse, B, H, N, scale, stream)
                      : launch<CAUSAL, true, false>(q8, k8, v8, qs, ks, vs, qmx, kmx, o, lse, B, H, N, scale, stream);
  return vhad ? launch<CAUSAL, false, true>(q8, k8, v8, qs, ks, vs, qmx, kmx, o, lse, B, H, N, scale, stream)
              : launch<CAUSAL, false, false>(q8, k8, v8, qs, ks, vs, qmx, kmx, o, lse, B, H, N, scale, stream);
}

}  // namespace

hipError_t launch_attn_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* qs, const float* ks,
                           const float* vs, const uint8_t* qmx, const uint8_t* kmx, bool v_hadamard, void* o,
                           float* lse, int B, int H, int N, float scale, bool causal, hipStream_t stream) {
  return causal ? launch_c<true>(q8, k8, v8, qs, ks, vs, qmx, kmx, v_hadamard, o, lse, B, H, N, scale, stream)
                : launch_c<false>(q8, k8, v8, qs, ks, vs, qmx, kmx, v_hadamard, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
