// Internal declarations shared by the HIP translation units of libfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Shapes are validated by the C entry points before these are called.
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, float scale, bool causal, hipStream_t stream);

// Causal attention, head dimension 128: the persistent ping-pong kernel.
hipError_t launch_attn_bf16_pp(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, float scale, hipStream_t stream);

// Split-KV decode: how the Nk keys are cut into S chunks of `chunk` keys (a
// pure function of the sizes, shared by the launcher and the workspace query).
void decode_split(int B, int H, int Nq, int Nk, int* S, int* chunk);

// Partial results of every chunk: op [S, B*H, Nq, d] float32, lp [S, B*H, Nq].
hipError_t launch_attn_decode_bf16(const void* q, const void* k, const void* v, float* op, float* lp, int B, int H,
                                   int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream);

// Size of the library-owned device scratch of fa_fwd_decode_noalloc, and its
// address on the current device (looked up once per device, thread-safe).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

// Merge P parts [P, rows, d] / [P, rows] into o [rows, d] (bf16 or float32) and lse [rows].
hipError_t launch_lse_merge(const float* op, const float* lp, void* o, bool bf16_out, float* lse, int P, long rows,
                            int d, hipStream_t stream);

// Backward pass, bf16: workspace of attn_bwd_workspace_bytes(B, H, N, d) bytes
// (LSE log2 e and Delta, float32 [B*H*N] each, 256-byte aligned; the dQ pass
// writes them, the dK/dV pass reads them).
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
                                int d, float scale, bool causal, hipStream_t stream);

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int N, int d, float scale, bool causal, hipStream_t stream);

// qmx / kmx: both null, or MX-style E8M0 scales [B*H, N, 4]; v_hadamard: V's
// codes hold V H / sqrt(d) and O is transformed back in the epilogue.
hipError_t launch_attn_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           const float* qs, const float* ks, const float* vs, const uint8_t* qmx,
                           const uint8_t* kmx, bool v_hadamard, void* o, float* lse,
                           int B, int H, int N, float scale, bool causal, hipStream_t stream);

hipError_t launch_hadamard_fp8_quant(const void* x, bool x_is_bf16, uint8_t* x8, float* scales,
                                     int B, int H, int N, int d, bool hadamard, hipStream_t stream);

// MX-style quantisation (d = 128): one E8M0 scale per 32 coordinates of a row.
hipError_t launch_mx_fp8_quant(const void* x, bool x_is_bf16, uint8_t* x8, uint8_t* e8m0, int B, int H, int N,
                               bool hadamard, hipStream_t stream);

// Q, K and V (d = 128, one shape) in one launch, each with its own transform
// and power-of-two-scale flags.
hipError_t launch_qkv_fp8_quant(const void* const x[3], bool x_is_bf16, uint8_t* const x8[3], float* const scales[3],
                                const int had[3], const int pow2[3], int B, int H, int N, hipStream_t stream);

// Resident workgroup slots of `kernel` at `block_threads` threads on the
// current device: compute units x workgroups per compute unit.  Queried once
// per (device, kernel, block size) and cached; thread-safe.  0 on a HIP error.
long device_slots(const void* kernel, int block_threads);

// Workgroups are handed to the 8 XCDs round-robin by workgroup id.  This maps
// the hardware id to a logical id so that each XCD receives one contiguous
// range of logical ids (neighbouring query blocks of the same heads share the
// XCD's L2).  A bijection on [0, total) for any total.
__device__ __forceinline__ int xcd_logical_id(int lin, int total) {
  const int xcd = lin & 7, idx = lin >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Race check.  Built with FA_DEBUG_SYNC defined (libfa_debugsync.so), every
// FA_SYNC_POINT waits for all of the wave's outstanding memory operations
// (the DMAs it has just issued included) and then for every wave of the
// workgroup, so each LDS buffer hand-off becomes fully serial: no DMA is in
// flight while any wave computes.  The kernels place these points only where
// every wave of the workgroup passes.  Both builds must give bitwise-equal
// results; a difference means a kernel reads an LDS buffer before its data
// has landed, or overwrites one that is still being read.  In the regular
// build the points are empty.
#ifdef FA_DEBUG_SYNC
#define FA_SYNC_POINT()               \
  do {                                \
    __builtin_amdgcn_s_waitcnt(0);    \
    __syncthreads();                  \
  } while (0)
#else
#define FA_SYNC_POINT() \
  do {                  \
  } while (0)
#endif

}  // namespace fa
