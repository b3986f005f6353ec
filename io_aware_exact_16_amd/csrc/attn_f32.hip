// Fused exact attention forward entirely in float32 (correctness path for
// float32 inputs; the throughput path is the bf16 kernel).
//
// Same method as the bf16 kernel ("Flash Attention" glossary page, second
// paragraph: tiles in on-chip memory, online softmax accumulating partial
// results, no N x N matrix in HBM), in the plainest gfx950 form: one lane per
// query row, key/value tiles of 32 rows staged in LDS and read as wave-wide
// broadcasts, running max / sum / output in registers, natural-exp softmax.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int ROWS = 64;   // query rows per workgroup (one wave, one row per lane)
constexpr int TK = 32;     // key rows per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(ROWS) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                            const float* __restrict__ K,
                                                            const float* __restrict__ V, float* __restrict__ O,
                                                            float* __restrict__ LSE, int N, int nqb, float scale) {
  __shared__ float qs[ROWS][D + 1];
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int q0 = qb * ROWS, tid = threadIdx.x, qi = q0 + tid;
  const size_t hoff = (size_t)bh * N * D;

  for (int i = tid; i < ROWS * D; i += ROWS) {
    const int r = i / D, col = i % D;
    qs[r][col] = (q0 + r < N) ? Q[hoff + (size_t)(q0 + r) * D + col] : 0.0f;
  }

  float o[D];
#pragma unroll
  for (int t = 0; t < D; ++t) o[t] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const int kend = CAUSAL ? min(N, q0 + ROWS) : N;

  for (int j0 = 0; j0 < kend; j0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D; i += ROWS) {
      const int r = i / D, col = i % D;
      const bool ok = j0 + r < N;
      ks[r][col] = ok ? K[hoff + (size_t)(j0 + r) * D + col] : 0.0f;
      vs[r][col] = ok ? V[hoff + (size_t)(j0 + r) * D + col] : 0.0f;
    }
    __syncthreads();

    float s[TK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < D; ++t) acc = __builtin_fmaf(qs[tid][t], ks[j][t], acc);
      acc *= scale;
      const int key = j0 + j;
      if (key >= N || (CAUSAL && key > qi)) acc = -INFINITY;
      s[j] = acc;
      tmax = fmaxf(tmax, acc);
    }
    const float mnew = fmaxf(m, tmax);
    if (mnew != -INFINITY) {             // a row with nothing visible yet keeps its state
      const float alpha = expf(m - mnew);
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] *= alpha;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        const float p = s[j] == -INFINITY ? 0.0f : expf(s[j] - mnew);
        ps += p;
#pragma unroll
        for (int t = 0; t < D; ++t) o[t] = __builtin_fmaf(p, vs[j][t], o[t]);
      }
      l = l * alpha + ps;
      m = mnew;
    }
  }

  if (qi < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int t = 0; t < D; ++t) O[hoff + (size_t)qi * D + t] = o[t] * inv;
    LSE[(size_t)bh * N + qi] = m + logf(l);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                  float scale, hipStream_t stream) {
  const int nqb = (N + ROWS - 1) / ROWS;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3(nqb * H * B), dim3(ROWS), 0, stream, q, k, v, o,
                     lse, N, nqb, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                           int N, int d, float scale, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
