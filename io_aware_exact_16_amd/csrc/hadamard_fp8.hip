// Incoherent processing + per-block FP8 (E4M3) quantisation, gfx950.
//
// "FlashAttention-3 (PT)", section "Inovacoes tecnicas", item 3: before FP8
// quantisation Q and K are multiplied by an orthogonal (Hadamard) matrix,
// which spreads outlier coordinates over all coordinates; because the matrix
// is orthogonal it cancels in Q K^T.  The matrix here is the Sylvester Hadamard
// matrix of order d scaled by 1/sqrt(d), applied to every token row with a fast
// Walsh-Hadamard transform (log2 d butterfly stages).
//
// One workgroup per (batch, head, block of 128 tokens) -- the scaling
// granularity -- so the block maximum is a workgroup reduction and every byte
// is read from and written to HBM exactly once.  The kernel is bound by HBM
// bandwidth; arithmetic is chosen for reproducibility instead of speed:
//  * the butterflies run in float64: sums of +-bf16 (or fp32) values are then
//    exact, so the transformed values y_u = x H do not depend on the order of
//    the butterflies (on gfx950 unpacked float64 adds issue at the float32 rate);
//  * the rounding decision is taken on the float32 quotient
//    RN32(y_u) * RN32(448 / RN32(A)), A = max |y_u| over the block (the 1/sqrt(d)
//    of the matrix cancels in y / s), plus 0 so that a zero quotient is +0;
//    v_cvt_pk_fp8_f32 rounds to nearest even;
//  * the stored scale is s = A / (448 sqrt(d)) (A / 448 without the matrix),
//    rounded once from float64 to float32; s = 1 for an all-zero block.
// Coalesced 16-byte loads land in a padded LDS tile; each thread then owns 64
// consecutive elements of one row (2 threads per row at d = 128), so 6 of the
// 7 butterfly stages are in registers and the last is one DPP lane swap.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BLK = 128;   // tokens per scaling block
constexpr int EPT = 64;    // elements per thread

template <int D, bool BF16IN, bool HAD>
__global__ __launch_bounds__(2 * D) void hadamard_fp8_quant_kernel(const void* __restrict__ X,
                                                                   uint8_t* __restrict__ X8,
                                                                   float* __restrict__ S, int N, int nb,
                                                                   double denom) {
  constexpr int NT = 2 * D;                  // threads: 128 rows x (D / 64) threads per row
  constexpr int TPR = D / EPT;
  constexpr int ES = BF16IN ? 2 : 4;         // input element size
  constexpr int ROWB = D * ES + 16;          // padded LDS row stride in bytes
  constexpr int CPR = D * ES / 16;           // 16-byte chunks per input row
  constexpr int LDC = BLK * CPR / NT;        // chunks loaded per thread
  __shared__ __attribute__((aligned(16))) char tile[BLK * ROWB];
  __shared__ double wmax[NT / 64];

  const int bh = blockIdx.x / nb, jb = blockIdx.x % nb;
  const int r0 = jb * BLK, tid = threadIdx.x;
  const size_t hoff = (size_t)bh * N * D;
  const char* xb = static_cast<const char*>(X) + hoff * ES;

#pragma unroll
  for (int i = 0; i < LDC; ++i) {
    const int c = i * NT + tid, row = c / CPR, cc = c % CPR;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r0 + row < N) u = *reinterpret_cast<const uint4*>(xb + ((size_t)(r0 + row) * D) * ES + 16 * cc);
    *reinterpret_cast<uint4*>(tile + row * ROWB + 16 * cc) = u;
  }
  __syncthreads();

  const int row = tid / TPR, part = tid % TPR;
  double x[EPT];
  {
    const char* src = tile + row * ROWB + part * EPT * ES;
#pragma unroll
    for (int i = 0; i < EPT * ES / 16; ++i) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + 16 * i);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16IN) {
          x[8 * i + 2 * j] = (double)__uint_as_float(w[j] << 16);
          x[8 * i + 2 * j + 1] = (double)__uint_as_float(w[j] & 0xffff0000u);
        } else {
          x[4 * i + j] = (double)__uint_as_float(w[j]);
        }
      }
    }
  }

  if (HAD) {
#pragma unroll
    for (int s = 1; s < EPT; s <<= 1)
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (!(i & s)) {
          const double a = x[i], b = x[i + s];
          x[i] = a + b;
          x[i + s] = a - b;
        }
    if (TPR == 2) {   // stride-64 stage: partner element sits in the adjacent lane
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const uint64_t bits = __double_as_longlong(x[i]);
        const uint32_t lo = __builtin_amdgcn_update_dpp(0, (uint32_t)bits, 0xB1, 0xF, 0xF, false);
        const uint32_t hi = __builtin_amdgcn_update_dpp(0, (uint32_t)(bits >> 32), 0xB1, 0xF, 0xF, false);
        const double other = __longlong_as_double(((uint64_t)hi << 32) | lo);
        x[i] = part == 0 ? x[i] + other : other - x[i];
      }
    }
  }

  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) amax = fmax(amax, fabs(x[i]));
  if (r0 + row >= N) amax = 0.0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  double A = wmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) A = fmax(A, wmax[w]);

  const float a32 = (float)A;
  const float inv32 = a32 > 0.0f ? 448.0f / a32 : 0.0f;
  if (r0 + row < N) {
    uint8_t* dst = X8 + hoff + (size_t)(r0 + row) * D + part * EPT;
#pragma unroll
    for (int i = 0; i < EPT / 16; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 16 * i + 4 * j;
        const float q0 = (float)x[e] * inv32 + 0.0f, q1 = (float)x[e + 1] * inv32 + 0.0f;
        const float q2 = (float)x[e + 2] * inv32 + 0.0f, q3 = (float)x[e + 3] * inv32 + 0.0f;
        uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, p, true);
      }
      *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (tid == 0) S[(size_t)bh * nb + jb] = A > 0.0 ? (float)(A / denom) : 1.0f;
}

template <int D, bool BF16IN, bool HAD>
hipError_t launch(const void* x, uint8_t* x8, float* s, int B, int H, int N, hipStream_t stream) {
  const int nb = (N + BLK - 1) / BLK;
  const double denom = HAD ? 448.0 * __builtin_sqrt((double)D) : 448.0;
  hipLaunchKernelGGL((hadamard_fp8_quant_kernel<D, BF16IN, HAD>), dim3(nb * H * B), dim3(2 * D), 0, stream, x,
                     x8, s, N, nb, denom);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hadamard_fp8_quant(const void* x, bool x_is_bf16, uint8_t* x8, float* scales, int B, int H,
                                     int N, int d, bool hadamard, hipStream_t stream) {
  if (d == 128) {
    if (x_is_bf16) return hadamard ? launch<128, true, true>(x, x8, scales, B, H, N, stream)
                                   : launch<128, true, false>(x, x8, scales, B, H, N, stream);
    return hadamard ? launch<128, false, true>(x, x8, scales, B, H, N, stream)
                    : launch<128, false, false>(x, x8, scales, B, H, N, stream);
  }
  return x_is_bf16 ? launch<64, true, false>(x, x8, scales, B, H, N, stream)
                   : launch<64, false, false>(x, x8, scales, B, H, N, stream);
}

}  // namespace fa
