// Device helpers shared by the two bf16 attention kernels (streaming and
// persistent ping-pong): register layouts of the 32x32x16 bf16 matrix
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
constexpr float RESCALE_THRESHOLD = 8.0f;   // log2 of the allowed growth of p

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
// voffset (per lane) + soffset (per wave); reads past the buffer's byte size
// return zeros.  (A plain device function: the builtin written inside a kernel
// template keeps the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0, 0);
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

}  // namespace bf16k
}  // namespace fa
