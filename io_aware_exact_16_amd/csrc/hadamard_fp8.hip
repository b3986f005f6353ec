// Incoherent processing + per-block FP8 (E4M3) quantisation, gfx950.
//
// "FlashAttention-3 (PT)", section "Inovacoes tecnicas", item 3: before FP8
// quantisation Q and K are multiplied by an orthogonal (Hadamard) matrix,
// which spreads outlier coordinates over all coordinates; because the matrix
// is orthogonal it cancels in Q K^T.  The matrix here is the Sylvester Hadamard
// matrix of order d scaled by 1/sqrt(d), applied to every token row with a fast
// Walsh-Hadamard transform (log2 d butterfly stages).
//
// Work unit: one (batch, head, block of 128 tokens) -- the scaling
// granularity -- so the block maximum is a workgroup reduction and every byte
// is read from and written to HBM exactly once.  Arithmetic:
//  * the butterflies run in float32 (each of the log2 d stages adds at most
//    2^-24 times the row's l1 norm of rounding error); without the transform
//    y = x is exact in float32;
//  * the rounding decision is taken on the float32 quotient
//    y_u * RN32(448 / A), A = max |y_u| over the block (the 1/sqrt(d) of the
//    matrix cancels in y / s); v_cvt_pk_fp8_f32 rounds to nearest even.  The
//    result is a rounding of the exact y / s to a neighbouring E4M3 value;
//    only quotients within that float32 error of a rounding boundary can go
//    either way;
//  * the stored scale is s = A / (448 sqrt(d)) (A / 448 without the matrix),
//    rounded once from float64 to float32; s = 1 for an all-zero block.
//
// Transform kernel, streaming (meant to run at HBM bandwidth): a persistent grid
// walks the blocks of up to three tensors (Q, K and V of one attention call in
// one launch, each with its own transform flag); each workgroup DMAs the next
// block's tile HBM -> LDS (buffer_load ... lds, XOR-swizzled rows, rows past N
// read as zeros) while it transforms the current one, and holds its E4M3 bytes
// in registers until the next block's wait, so no wait ever covers a store it
// has just issued.  In the tile each thread owns 64 consecutive elements of
// one row (2 threads per row at d = 128): 6 of the 7 butterfly stages are in
// registers, the last is one DPP lane swap.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BLK = 128;   // tokens per scaling block
constexpr int EPT = 64;    // elements per thread

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset + soffset, 0, 0, 0);
}

// Up to three tensors of the same shape, quantised in one launch.
struct QuantJobs {
  const void* x[3];
  uint8_t* x8[3];
  float* s[3];
  int had[3];
  int pow2[3];   // power-of-two scale 2^ceil(log2(amax / 448)) instead of amax / 448
  uint8_t* mx[3];   // non-null: MX mode, one E8M0 scale per 32 coordinates of a row ([N, d / 32] per head)
  int njobs;
};

// 2^-E and the E8M0 code E + 127 of the power-of-two scale 2^E, E =
// ceil(log2(amax / denom)) clamped to [-127, 127], for amax > 0; the
// multiplier that forms y / 2^E from the unnormalised transform y_u also
// carries 1 / sqrt(d) (rnorm).
__device__ __forceinline__ float pow2_multiplier(float amax, double denom, double rnorm, int* e8) {
  int e;
  const double m = frexp((double)amax / denom, &e);
  int E = m == 0.5 ? e - 1 : e;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  *e8 = E + 127;
  return (float)(ldexp(1.0, -E) * rnorm);
}

template <int D, bool BF16IN>
__global__ __launch_bounds__(2 * D) void hadamard_fp8_quant_kernel(const QuantJobs jobs, int N, int nb,
                                                                   int nblocks, double denom_had) {
  constexpr int NT = 2 * D;                  // threads: 128 rows x (D / 64) threads per row
  constexpr int NW = NT / 64;
  constexpr int TPR = D / EPT;
  constexpr int ES = BF16IN ? 2 : 4;         // input element size
  constexpr int CPR = D * ES / 16;           // 16-byte chunks per input row
  constexpr int TILE = BLK * CPR;            // chunks per tile
  constexpr int LPT = TILE / NT;             // DMA instructions per thread and tile
  constexpr int CPT = EPT * ES / 16;         // chunks read per thread
  // chunk c of tile row r sits at r * CPR + (c ^ (r & 7)): conflict-free reads
  // of each thread's 64-element segment
  __shared__ uint4 tile0[TILE], tile1[TILE];
  __shared__ float wmax[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = tid / TPR, part = tid % TPR;
  const int total = nblocks * jobs.njobs;
  // job of a global block index, and its tensors (wave-uniform selects)
  auto job_of = [&](int blk) { return blk >= 2 * nblocks ? 2 : (blk >= nblocks ? 1 : 0); };

  // DMA: instruction i of wave w fills slots (i * NW + w) * 64 + lane
  uint32_t lane_off[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int slot = (i * NW + wave) * 64 + lane, r = slot / CPR, c = (slot % CPR) ^ (r & 7);
    lane_off[i] = (uint32_t)(r * D * ES + 16 * c);
  }
  auto issue = [&](int gblk, uint4* dst) {
    const int jb_all = gblk - job_of(gblk) * nblocks;
    const int bh = jb_all / nb, jb = jb_all - bh * nb;
    const int jo = job_of(gblk);
    const void* X = jo == 0 ? jobs.x[0] : (jo == 1 ? jobs.x[1] : jobs.x[2]);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const char*>(X) + (size_t)bh * N * D * ES), 0, (uint32_t)N * D * ES, 0x00020000);
    const uint32_t base = (uint32_t)(jb * BLK) * D * ES;
#pragma unroll
    for (int i = 0; i < LPT; ++i) lds_dma16(rs, dst + (i * NW + wave) * 64, lane_off[i], base);
  };

  // the previous block's results, stored once the next block's wait is done
  uint4 held[EPT / 16];
  uint8_t* held_dst = nullptr;
  float held_scale = 0.0f;
  float* held_sdst = nullptr;
  uint8_t* held_mx = nullptr;                // MX mode: this thread's two E8M0 codes
  uint32_t held_mxv = 0;
  auto flush = [&]() {
    if (held_dst) {
#pragma unroll
      for (int i = 0; i < EPT / 16; ++i) *reinterpret_cast<uint4*>(held_dst + 16 * i) = held[i];
    }
    if (held_sdst) *held_sdst = held_scale;
    if (held_mx) *reinterpret_cast<uint16_t*>(held_mx) = (uint16_t)held_mxv;
    held_mx = nullptr;
  };

  // one block: its tile is in cur (its DMA is complete after the wait below),
  // the next block's tile goes to nxt; cur and nxt are distinct arrays at every
  // call, so the compiler never orders the reads of cur behind the DMA into nxt
  auto block = [&](int gblk, const uint4* cur, uint4* nxt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this thread's part of the tile (and older stores)
    __syncthreads();                         // ... every thread's part; everyone is done with nxt
    if (gblk + (int)gridDim.x < total) issue(gblk + gridDim.x, nxt);
    FA_SYNC_POINT();
    flush();

    const int jo = job_of(gblk);
    const int jb_all = gblk - jo * nblocks;
    const int bh = jb_all / nb, jb = jb_all - bh * nb;
    const int r0 = jb * BLK;
    const bool had = (jo == 0 ? jobs.had[0] : (jo == 1 ? jobs.had[1] : jobs.had[2])) != 0;
    const bool pw2 = (jo == 0 ? jobs.pow2[0] : (jo == 1 ? jobs.pow2[1] : jobs.pow2[2])) != 0;
    float x[EPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint4 u = cur[row * CPR + ((part * CPT + i) ^ (row & 7))];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16IN) {
          x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
          x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        } else {
          x[4 * i + j] = __uint_as_float(w[j]);
        }
      }
    }

    if (had) {
#pragma unroll
      for (int s = 1; s < EPT; s <<= 1)
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (!(i & s)) {
            const float a = x[i], b = x[i + s];
            x[i] = a + b;
            x[i + s] = a - b;
          }
      if (TPR == 2) {   // stride-64 stage: partner element sits in the adjacent lane
        // part 0 keeps x + other, part 1 other - x: one FMA with a +-1 factor
        // (exact, like the add), and a lane swap that every lane sources, so
        // the DPP move needs no fallback value
        const float sgn = part == 0 ? 1.0f : -1.0f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const float other =
              __uint_as_float(__builtin_amdgcn_mov_dpp((int)__float_as_uint(x[i]), 0xB1, 0xF, 0xF, false));
          x[i] = __builtin_fmaf(x[i], sgn, other);
        }
      }
    }

    uint8_t* const MXO = jo == 0 ? jobs.mx[0] : (jo == 1 ? jobs.mx[1] : jobs.mx[2]);
    if (MXO) {   // MX mode: this thread's 64 values are two whole groups of 32
      const double rnorm = had ? 1.0 / __builtin_sqrt((double)D) : 1.0;
      uint32_t e8pair = 0;
#pragma unroll
      for (int gi = 0; gi < EPT / 32; ++gi) {
        float ga = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) ga = fmaxf(ga, fabsf(x[32 * gi + i]));
        int e8 = 0;
        const float mul = ga > 0.0f ? pow2_multiplier(ga, had ? denom_had : 448.0, rnorm, &e8) : 0.0f;
        e8pair |= (uint32_t)e8 << (8 * gi);
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
          const int e = 32 * gi + i;
          uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(x[e] * mul, x[e + 1] * mul, 0, false);
          const uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(x[e + 2] * mul, x[e + 3] * mul, p, true);
          reinterpret_cast<uint32_t*>(held)[(32 * gi + i) / 4] = wv;
        }
      }
      uint8_t* const X8 = jo == 0 ? jobs.x8[0] : (jo == 1 ? jobs.x8[1] : jobs.x8[2]);
      held_dst = r0 + row < N ? X8 + (size_t)bh * N * D + (size_t)(r0 + row) * D + part * EPT : nullptr;
      held_mx = r0 + row < N ? MXO + ((size_t)bh * N + r0 + row) * (D / 32) + part * (EPT / 32) : nullptr;
      held_mxv = e8pair;
      held_sdst = nullptr;
      return;
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) amax = fmaxf(amax, fabsf(x[i]));
    if (r0 + row >= N) amax = 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) wmax[wave] = amax;
    // the waves' maxima are in LDS; a bare barrier, so that the prefetch DMA
    // and the stores issued above stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
    float A = wmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) A = fmaxf(A, wmax[w]);

    // the multiplier that forms y / s: 448 / A, or for a power-of-two scale
    // s = 2^E, E = ceil(log2(A / denom)) (at least -126), 2^-E (times 1/sqrt(d)
    // with the transform, whose 1/sqrt(d) no longer cancels)
    const double denom = had ? denom_had : 448.0;
    float inv32 = A > 0.0f ? 448.0f / A : 0.0f;
    float scale = A > 0.0f ? (float)((double)A / denom) : 1.0f;
    if (pw2 && A > 0.0f) {
      int e;
      const double m = frexp((double)A / denom, &e);
      int E = m == 0.5 ? e - 1 : e;
      E = E < -126 ? -126 : E;
      scale = ldexpf(1.0f, E);
      inv32 = (float)(ldexp(1.0, -E) / (had ? denom_had / 448.0 : 1.0));
    }
#pragma unroll
    for (int i = 0; i < EPT / 16; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 16 * i + 4 * j;
        uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(x[e] * inv32, x[e + 1] * inv32, 0, false);
        w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(x[e + 2] * inv32, x[e + 3] * inv32, p, true);
      }
      held[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    uint8_t* const X8 = jo == 0 ? jobs.x8[0] : (jo == 1 ? jobs.x8[1] : jobs.x8[2]);
    float* const S = jo == 0 ? jobs.s[0] : (jo == 1 ? jobs.s[1] : jobs.s[2]);
    held_dst = r0 + row < N ? X8 + (size_t)bh * N * D + (size_t)(r0 + row) * D + part * EPT : nullptr;
    held_sdst = tid == 0 ? S + (size_t)bh * nb + jb : nullptr;
    held_scale = scale;
  };

  int blk = blockIdx.x;
  if (blk < total) issue(blk, tile0);
  while (blk < total) {                      // unrolled over the two tiles
    block(blk, tile0, tile1);
    blk += gridDim.x;
    if (blk >= total) break;
    block(blk, tile1, tile0);
    blk += gridDim.x;
  }
  flush();
}

// Without the transform the scale is the maximum over the whole block, so no
// thread needs a whole row: each thread quantises whole 16-byte input chunks
// (fully coalesced loads straight into registers, no LDS tile), the maximum is
// a workgroup reduction, and the codes go out as coalesced stores.  Values stay
// in float32, where bf16 and fp32 inputs are exact.  Few registers, so many
// blocks' loads are in flight per compute unit.
template <int D, bool BF16IN>
__global__ __launch_bounds__(256) void fp8_quant_plain_kernel(const void* __restrict__ X, uint8_t* __restrict__ X8,
                                                              float* __restrict__ S, int N, int nb) {
  constexpr int NT = 256, NW = NT / 64;
  constexpr int ES = BF16IN ? 2 : 4;
  constexpr int EPC = 16 / ES;                   // elements per 16-byte chunk
  constexpr int CHUNKS = BLK * D / EPC;          // chunks per block
  constexpr int CPT = CHUNKS / NT;               // chunks per thread
  __shared__ float wmax[NW];
  const int bh = blockIdx.x / nb, jb = blockIdx.x - bh * nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t e0 = ((size_t)bh * N + (size_t)jb * BLK) * D;   // first element of the block
  const size_t nvalid = (size_t)min(BLK, N - jb * BLK) * D;     // elements of the block inside the tensor
  const char* xb = static_cast<const char*>(X) + e0 * ES;

  uint4 u[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * NT + tid;                  // consecutive threads, consecutive chunks
    u[i] = (size_t)c * EPC < nvalid ? *reinterpret_cast<const uint4*>(xb + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (BF16IN) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[j] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[j] & 0xffff0000u)));
      } else {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[j])));
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  float A = wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) A = fmaxf(A, wmax[w]);

  const float inv32 = A > 0.0f ? 448.0f / A : 0.0f;
  uint8_t* dst = X8 + e0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * NT + tid;
    if ((size_t)c * EPC >= nvalid) continue;
    const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
    if (BF16IN) {                                // 8 elements -> 8 codes
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float q0 = __uint_as_float(w[2 * h] << 16) * inv32;
        const float q1 = __uint_as_float(w[2 * h] & 0xffff0000u) * inv32;
        const float q2 = __uint_as_float(w[2 * h + 1] << 16) * inv32;
        const float q3 = __uint_as_float(w[2 * h + 1] & 0xffff0000u) * inv32;
        const uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        o[h] = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, p, true);
      }
      *reinterpret_cast<uint2*>(dst + (size_t)c * EPC) = make_uint2(o[0], o[1]);
    } else {                                     // 4 elements -> 4 codes
      const float q0 = __uint_as_float(w[0]) * inv32, q1 = __uint_as_float(w[1]) * inv32;
      const float q2 = __uint_as_float(w[2]) * inv32, q3 = __uint_as_float(w[3]) * inv32;
      const uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      *reinterpret_cast<uint32_t*>(dst + (size_t)c * EPC) = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, p, true);
    }
  }
  if (tid == 0) S[(size_t)bh * nb + jb] = A > 0.0f ? (float)((double)A / 448.0) : 1.0f;
}

template <int D, bool BF16IN>
hipError_t launch(const QuantJobs& jobs, int B, int H, int N, hipStream_t stream) {
  const int nb = (N + BLK - 1) / BLK;
  const int nblocks = nb * H * B;
  const long total = (long)nblocks * jobs.njobs;
  const double denom = 448.0 * __builtin_sqrt((double)D);   // s = A / (448 sqrt(d)) with the transform
  const long slots = device_slots(reinterpret_cast<const void*>(&hadamard_fp8_quant_kernel<D, BF16IN>), 2 * D);
  if (slots <= 0) return hipErrorInvalidDevice;
  const int grid = total < slots ? (int)total : (int)slots;
  hipLaunchKernelGGL((hadamard_fp8_quant_kernel<D, BF16IN>), dim3(grid), dim3(2 * D), 0, stream, jobs, N, nb, nblocks,
                     denom);
  return hipGetLastError();
}

template <int D, bool BF16IN>
hipError_t launch_plain(const void* x, uint8_t* x8, float* s, int B, int H, int N, hipStream_t stream) {
  const int nb = (N + BLK - 1) / BLK;
  hipLaunchKernelGGL((fp8_quant_plain_kernel<D, BF16IN>), dim3(nb * H * B), dim3(256), 0, stream, x, x8, s, N, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hadamard_fp8_quant(const void* x, bool x_is_bf16, uint8_t* x8, float* scales, int B, int H,
                                     int N, int d, bool hadamard, hipStream_t stream) {
  if (hadamard) {   // d = 128 (checked by the entry point)
    QuantJobs jobs = {};
    jobs.x[0] = x;
    jobs.x8[0] = x8;
    jobs.s[0] = scales;
    jobs.had[0] = 1;
    jobs.njobs = 1;
    return x_is_bf16 ? launch<128, true>(jobs, B, H, N, stream) : launch<128, false>(jobs, B, H, N, stream);
  }
  if (d == 128)
    return x_is_bf16 ? launch_plain<128, true>(x, x8, scales, B, H, N, stream)
                     : launch_plain<128, false>(x, x8, scales, B, H, N, stream);
  return x_is_bf16 ? launch_plain<64, true>(x, x8, scales, B, H, N, stream)
                   : launch_plain<64, false>(x, x8, scales, B, H, N, stream);
}

hipError_t launch_mx_fp8_quant(const void* x, bool x_is_bf16, uint8_t* x8, uint8_t* e8m0, int B, int H, int N,
                               bool hadamard, hipStream_t stream) {
  QuantJobs jobs = {};
  jobs.x[0] = x;
  jobs.x8[0] = x8;
  jobs.mx[0] = e8m0;
  jobs.had[0] = hadamard ? 1 : 0;
  jobs.njobs = 1;
  return x_is_bf16 ? launch<128, true>(jobs, B, H, N, stream) : launch<128, false>(jobs, B, H, N, stream);
}

hipError_t launch_qkv_fp8_quant(const void* const x[3], bool x_is_bf16, uint8_t* const x8[3], float* const scales[3],
                                const int had[3], const int pow2[3], int B, int H, int N, hipStream_t stream) {
  QuantJobs jobs = {};
  for (int i = 0; i < 3; ++i) {
    jobs.x[i] = x[i];
    jobs.x8[i] = x8[i];
    jobs.s[i] = scales[i];
    jobs.had[i] = had[i];
    jobs.pow2[i] = pow2[i];
  }
  jobs.njobs = 3;
  return x_is_bf16 ? launch<128, true>(jobs, B, H, N, stream) : launch<128, false>(jobs, B, H, N, stream);
}

}  // namespace fa
