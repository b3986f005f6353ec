// Device helpers shared by the bf16 attention kernels (streaming, persistent
// ping-pong and split-KV decode): register layouts of the 32x32x16 bf16 matrix
// instruction, the swizzled LDS tile layout, the buffer-to-LDS DMA and the
// half-wave reductions.  Included by HIP translation units only.
//
// Register-level layouts (lane l of 64, h = l / 32; verified on gfx950):
//   32x32x16 bf16 MFMA: A[i][k] in lane (i + 32 * (k / 8)), element k % 8;
//   B[k][j] in lane (j + 32 * (k / 8)), element k % 8; C[i][j] in lane
//   (j + 32 * ((i / 4) % 2)), register 4 * (i / 8) + i % 4.
//   ds_read_b64_tr_b16: within each 16-lane group, lane 4r + c names the 4
//   elements at [r][4c..4c+3] of a 4 x 16 tile; lane j receives column j.
#pragma once

#include "fa_internal.h"

namespace fa {
namespace bf16k {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int BC = 64;    // key rows per tile

// Position (in 16-byte chunks) of chunk `ch` of tile row `row` in LDS.  The
// XOR swizzle makes both read patterns of the kernel conflict-free: 16 lanes
// reading 16 B from 16 different rows (K operand), and 32 lanes reading
// 8 B from 4 rows x 4 chunks (transposed V operand).
template <int D>
__device__ __forceinline__ int swz(int row) {
  return (D == 128) ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

template <int D>
__device__ __forceinline__ int lds_chunk(int row, int ch) {
  return row * (D / 8) + (ch ^ swz<D>(row));
}

// Row of a 32-key block that A-operand row m must hold so that, in the
// accumulator layout, the 8 registers r = 0..7 (8..15) of half-wave h hold keys
// 8h + r (16 + 8h + r - 8): consecutive keys, ready to be the B operand of P V.
// It swaps bits 2 and 3 of m.
__device__ __forceinline__ int key_of_arow(int m) {
  return (m & 0x13) | ((m >> 1) & 0x4) | ((m << 1) & 0x8);
}

// 16 bytes per lane from a buffer straight into LDS: lane i's data lands at
// lds + 16 * i (lds must be the same for the whole wave).  The byte offset is
// voffset (per lane) + soffset (per wave), both passed in the instruction's
// per-lane offset, which the hardware checks against the buffer's byte size:
// reads past it return zeros.  (A plain device function: the builtin written
// inside a kernel template keeps the host pass from emitting the kernel's
// launch stub.)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset + soffset, 0, 0, 0);
}

__device__ __forceinline__ float wave_halves_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float wave_halves_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ bf16x4_t tr_read(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// One 64-key tile of one wave: S^T = K Q^T, (mask), online softmax, O^T += V^T P^T.
// kt / vt are the LDS K and V tiles; koff / voff are this lane's byte offsets
// into them (first 32-key block, first 16-key chunk); MASK marks tiles that
// cross the causal diagonal or the end of the sequence.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void tile_math(const char* kt, const char* vt, const uint32_t (&koff)[D / 16],
                                          const uint32_t (&voff)[D / 32][2], const bf16x8 (&qf)[D / 16],
                                          f32x16 (&acc)[D / 32], float& m2, float& lsum, float c, int j0, int qi,
                                          int N, int half) {
  constexpr int KB_BYTES = 32 * D * 2;   // one 32-key block of the tile
  constexpr int KC_BYTES = 16 * D * 2;   // one 16-key chunk of the tile
  f32x16 s[BC / 32];
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

  __builtin_amdgcn_sched_barrier(0);
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
        if (key >= N || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
      }
  }

  // p = exp2(c s - m2), rounded to bf16 as the B operand of P V; the row sum
  // uses the float32 p (summing the bf16-rounded values would cost up to 2^-9
  // relative in l, i.e. in LSE, on rows with few keys).
  bf16x8 pb[BC / 16];
  auto pchunk = [&](int kc) -> float {
    float r[2] = {0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float s0 = s[kc >> 1][8 * (kc & 1) + e], s1 = s[kc >> 1][8 * (kc & 1) + e + 1];
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -m2));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -m2));
      if (MASK) {                        // exact zeros for masked keys, also when c = 0
        p0 = s0 == -INFINITY ? 0.0f : p0;
        p1 = s1 == -INFINITY ? 0.0f : p1;
      }
      r[(e >> 1) & 1] += p0 + p1;
      pb[kc][e] = (__bf16)p0;
      pb[kc][e + 1] = (__bf16)p1;
    }
    return r[0] + r[1];
  };
  // The reference maximum m2 only has to keep every p finite and in range, so
  // the tile maximum is not formed on the common path.  A tile whose lane sum
  // of p is at most 2^8 has every p at most 2^8; a larger or non-finite sum
  // (the first tile, where m2 = -inf) moves m2 to the tile maximum, rescales O
  // and l, and computes P again.
  auto move_reference = [&]() {
    float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // 4 independent chains
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pm[(kb * 2 + (r >> 3)) & 3] = fmaxf(pm[(kb * 2 + (r >> 3)) & 3], s[kb][r]);
    const float tm2 = wave_halves_max(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]))) * c;
    if (tm2 > m2) {
      const float alpha = __builtin_amdgcn_exp2f(m2 - tm2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m2 = tm2;
    }
  };
  // all four chunks of P first, one range check for the tile, then P V
  float cs = (pchunk(0) + pchunk(1)) + (pchunk(2) + pchunk(3));
  if (__any(!(cs <= 256.0f))) {
    move_reference();
    cs = (pchunk(0) + pchunk(1)) + (pchunk(2) + pchunk(3));
  }
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
  constexpr int NPV = (D / 32) * (BC / 16);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < NPV - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  lsum += cs;
}

}  // namespace bf16k
}  // namespace fa
