// Fused exact attention forward, bf16 in / bf16 out, float32 softmax, gfx950:
// the streaming kernel (non-causal attention and head dimension 64; causal
// attention with head dimension 128 runs the persistent ping-pong kernel of
// attn_bf16_pp.hip, selected in launch_attn_bf16 below).
//
// Method ("Flash Attention" glossary page, second paragraph; "FlashAttention-3
// (PT)", section "FlashAttention e FlashAttention-2"): one kernel walks the
// key/value sequence tile by tile, keeps a running row maximum and row sum
// (online softmax), rescales the partial output when the maximum grows, and
// never writes the score matrix to HBM.  The work is split over query blocks,
// heads and batches (FlashAttention-2's parallelism over the sequence), and
// the 1/l normalisation is deferred to the end (its fewer non-matmul FLOPs).
//
// gfx950 mapping (the Hopper design on the pages -- WGMMA, TMA, warp
// specialisation -- is prior art, not reproduced):
//  * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
//    query rows; key/value tiles of 64 rows stream through LDS, double
//    buffered so the next tile's loads overlap this tile's math; the loads go
//    straight from HBM/L2 to LDS (buffer_load_dwordx4 ... lds: no staging
//    registers; the buffer range check returns zeros past the last token);
//  * at most 256 registers per lane, so two waves share each SIMD and the
//    hardware overlaps one wave's softmax with the other's matrix ops;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    with the 32x32 accumulator layout each lane then holds 16 keys of ONE
//    query, so the row max / row sum are in-register reductions plus a single
//    exchange between the two half-waves (v_permlane32_swap), and the running
//    statistics and the output rescale are per-lane scalars;
//  * the output is accumulated transposed too, O^T += V^T P^T: the score
//    accumulator registers, rounded to bf16, are directly the B operand, and
//    V^T comes out of the row-major LDS tile through ds_read_b64_tr_b16;
//  * Q^T stays in registers for the whole key loop;
//  * exp2 with the scale folded into one FMA (c = scale * log2 e);
//  * the reference maximum is only moved when a tile's maximum exceeds it by
//    more than 2^8 (in the exp2 domain): p = exp2(c s - m) <= 256 stays exact in
//    float32 and bf16 range, the final O / l and LSE are unchanged, and the
//    O rescale (D/2 multiplies per lane) is skipped on almost every tile.
//
// The register layouts these rely on are listed in attn_bf16_common.h.
#include "attn_bf16_common.h"

namespace fa {
namespace {

using namespace bf16k;

constexpr int BR = 128;   // query rows per workgroup
constexpr int NT = 256;   // threads per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int nqb, int total, float c,
    uint32_t qflip) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE_CHUNKS = BC * CPR;      // chunks per K (or V) tile
  constexpr int NW = NT / 64;
  constexpr int LPW = TILE_CHUNKS / NT;      // DMA instructions per wave, tensor and tile
  // Separate objects for the two K and V buffers, so the compiler never orders
  // a read of one buffer behind the DMA into the other (with one array it
  // waited for the next tile's DMA before every P V product).
  __shared__ uint4 kb0[TILE_CHUNKS], kb1[TILE_CHUNKS], vb0[TILE_CHUNKS], vb1[TILE_CHUNKS];

  const int L = xcd_logical_id(blockIdx.x, total);
  const int bh = L / nqb;
  int qb = L - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;             // longest query blocks first
  const int q0 = qb * BR;
  // wave index as a scalar: the per-wave addresses and branches stay in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int qw = q0 + 32 * wave;             // first query row of this wave
  const int qi = qw + l32;                   // this lane's query
  const size_t hoff = (size_t)bh * N * D;

  // Q^T as the B operand: lane holds query qi, dims 16*dc + 8*half + 0..7
  bf16x8 qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qi < N) u = *reinterpret_cast<const uint4*>(Q + hoff + (size_t)qi * D + 16 * dc + 8 * half);
    u.x ^= qflip; u.y ^= qflip; u.z ^= qflip; u.w ^= qflip;
    qf[dc] = __builtin_bit_cast(bf16x8, u);
  }

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

  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  // DMA: instruction i of wave w fills the 64 consecutive 16-byte LDS slots
  // starting at (i * NW + w) * 64; each lane loads the global chunk that the
  // swizzled layout keeps in its slot.  The tile's start goes in soffset.
  const uint32_t nbytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + hoff), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + hoff), 0, nbytes, 0x00020000);
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = (i * NW + wave) * 64 + lane, row = pos / CPR, slot = pos % CPR;
    lane_off[i] = (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2;
  }
  auto issue_tile = [&](int j0, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      lds_dma16(krs, (BUF ? kb1 : kb0) + slot0, lane_off[i], base);
      lds_dma16(vrs, (BUF ? vb1 : vb0) + slot0, lane_off[i], base);
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m2 = -INFINITY;   // reference maximum, exp2 domain (c * raw score)
  float lsum = 0.0f;      // this half-wave's share of the row sum

  auto step = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int j0 = t * BC;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this wave's part of tile t has landed
    __syncthreads();                         // ... and every other wave's; the other buffer is free
    if (t + 1 < ntiles) issue_tile(j0 + BC, IC<BUF ^ 1>{});
    FA_SYNC_POINT();
    if (CAUSAL && j0 > qw + 31) return;      // the whole tile is above this wave's diagonal
    const char* kt = reinterpret_cast<const char*>(BUF ? kb1 : kb0);
    const char* vt = reinterpret_cast<const char*>(BUF ? vb1 : vb0);
    if ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw))
      tile_math<D, CAUSAL, true>(kt, vt, koff, voff, qf, acc, m2, lsum, c, j0, qi, N, half);
    else
      tile_math<D, CAUSAL, false>(kt, vt, koff, voff, qf, acc, m2, lsum, c, j0, qi, N, half);
  };

  issue_tile(0, IC<0>{});
  for (int t = 0; t < ntiles; t += 2) {     // unrolled by the two LDS buffers
    step(t, IC<0>{});
    if (t + 1 < ntiles) step(t + 1, IC<1>{});
  }

  // epilogue: O = O / l, LSE = ln 2 * (m2 + log2 l)
  const float ltot = wave_halves_sum(lsum);
  if (qi < N) {
    const float inv = 1.0f / ltot;
    uint16_t* orow = O + hoff + (size_t)qi * D;
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
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                  float scale, hipStream_t stream) {
  const int nqb = (N + BR - 1) / BR;
  const int total = nqb * H * B;
  const float c = (float)((double)__builtin_fabsf(scale) * 1.4426950408889634);
  const uint32_t qflip = scale < 0.0f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, nqb, total, c, qflip);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int N, int d, float scale, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_attn_bf16_pp(q, k, v, o, lse, B, H, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
