// Split-KV attention forward for a few queries against a long key sequence
// (a decode step), and the merge of partial attentions through their
// log-sum-exps, bf16 in, gfx950.
//
// "Flash Attention" glossary page, second paragraph: the online softmax
// accumulates partial results block by block; fourth paragraph: ring attention
// spreads that tiling over devices, and long-context inference runs on it.
// Both rest on one identity: for disjoint key parts s with partial results
// O_s (normalised by their own sum) and LSE_s,
//     LSE = ln sum_s exp(LSE_s),    O = sum_s exp(LSE_s - LSE) O_s.
//
// Decode: the Nq queries are the last Nq of the Nk tokens (query i has
// position Nk - Nq + i; causal: it sees keys 0 .. Nk - Nq + i).  With few
// queries the work is bound by reading K and V once from HBM, so the keys
// are split into S chunks and every (chunk, 32-query group, head) is one
// single-wave workgroup: enough workgroups to keep HBM busy even for one
// head.  Each workgroup streams its chunk's 64-key tiles through LDS by DMA
// (double buffered) and runs the same per-tile math as the streaming prefill
// kernel (S^T = K Q^T on bf16 MFMA, online softmax, O^T += V^T P^T); it writes
// its partial O_s (float32, normalised) and LSE_s (-inf when the chunk holds
// no key the query sees) to the caller's workspace.  A second kernel merges
// the S parts per query row with the identity above.
#include <mutex>

#include "attn_bf16_common.h"

namespace fa {
namespace {

// Library-owned scratch of the entry point that allocates nothing
// (fa_fwd_decode_noalloc): the partial results of the split-KV kernel.  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device (decode_scratch below).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

using namespace bf16k;

constexpr int DEC_NT = 64;        // one wave per workgroup: 32 queries
constexpr int DEC_QG = 32;        // queries per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DEC_NT) void attn_decode_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ OP, float* __restrict__ LP, int BH, int Nq, int Nk, int nqg, int S, int chunk, float c,
    uint32_t qflip) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE_CHUNKS = BC * CPR;
  constexpr int LPW = TILE_CHUNKS / DEC_NT;  // DMA instructions per tensor and tile
  __shared__ uint4 kbuf0[TILE_CHUNKS], kbuf1[TILE_CHUNKS], vbuf0[TILE_CHUNKS], vbuf1[TILE_CHUNKS];

  const int lin = blockIdx.x;
  const int s = lin % S, rest = lin / S;
  const int g = rest % nqg, bh = rest / nqg;
  const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
  const int qr = DEC_QG * g + l32;           // this lane's query row
  const int pos0 = Nk - Nq;                  // position of query row 0
  const int qi = pos0 + qr;                  // this lane's query position
  const int k0 = s * chunk;
  int kend = min(Nk, k0 + chunk);
  if (CAUSAL) kend = min(kend, pos0 + min(Nq - 1, DEC_QG * g + DEC_QG - 1) + 1);   // keys any row here sees
  const int ntiles = kend > k0 ? (kend - k0 + BC - 1) / BC : 0;
  const int qmin = pos0 + DEC_QG * g;        // smallest query position of the group

  // Q^T as the B operand: lane holds query qr, dims 16*dc + 8*half + 0..7 (zeros past Nq)
  bf16x8 qf[D / 16];
  {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Q + (size_t)bh * Nq * D), 0, (uint32_t)Nq * D * 2, 0x00020000);
    const uint32_t off = (uint32_t)(qr * D + 8 * half) * 2;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 32 * dc, 0));
      u.x ^= qflip; u.y ^= qflip; u.z ^= qflip; u.w ^= qflip;
      qf[dc] = __builtin_bit_cast(bf16x8, u);
    }
  }

  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) koff[dc] = 16 * lds_chunk<D>(key_of_arow(l32), 2 * dc + half);
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

  // K/V tile DMA: instruction i fills slots i * 64 + lane with the global
  // chunks that the swizzled layout keeps there; keys past Nk read as zeros
  const uint32_t nbytes = (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + (size_t)bh * Nk * D), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + (size_t)bh * Nk * D), 0, nbytes, 0x00020000);
  uint32_t lane_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int pos = i * 64 + lane, row = pos / CPR, slot = pos % CPR;
    lane_off[i] = (uint32_t)(row * D + 8 * (slot ^ swz<D>(row))) * 2;
  }
  auto issue_tile = [&](int j0, uint4* kd, uint4* vd) {
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(krs, kd + i * 64, lane_off[i], base);
      lds_dma16(vrs, vd + i * 64, lane_off[i], base);
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m2 = -INFINITY, lsum = 0.0f;

  // one tile: its DMA is complete after the wait; the next tile's goes to the
  // other buffer pair (distinct arrays, so reads are never ordered behind it)
  auto step = [&](int t, const uint4* kc, const uint4* vc, uint4* kn, uint4* vn) {
    const int j0 = k0 + t * BC;
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    if (t + 1 < ntiles) issue_tile(j0 + BC, kn, vn);
    FA_SYNC_POINT();
    const char* kt = reinterpret_cast<const char*>(kc);
    const char* vt = reinterpret_cast<const char*>(vc);
    if ((j0 + BC > kend) || (CAUSAL && j0 + BC - 1 > qmin))
      tile_math<D, CAUSAL, true>(kt, vt, koff, voff, qf, acc, m2, lsum, c, j0, qi, kend, half);
    else
      tile_math<D, CAUSAL, false>(kt, vt, koff, voff, qf, acc, m2, lsum, c, j0, qi, kend, half);
  };
  if (ntiles > 0) issue_tile(k0, kbuf0, vbuf0);
  for (int t = 0; t < ntiles; t += 2) {
    step(t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 < ntiles) step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }

  // partial result, normalised by its own sum; a row that saw no key of the
  // chunk has weight zero in the merge: LSE_s = -inf, O_s = 0
  const float ltot = wave_halves_sum(lsum);
  if (qr < Nq) {
    const size_t row = ((size_t)s * BH + bh) * Nq + qr;
    const bool any = ltot > 0.0f;
    const float inv = any ? 1.0f / ltot : 0.0f;
    float* orow = OP + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * half;
        *reinterpret_cast<float4*>(orow + d0) = make_float4(acc[db][4 * a + 0] * inv, acc[db][4 * a + 1] * inv,
                                                            acc[db][4 * a + 2] * inv, acc[db][4 * a + 3] * inv);
      }
    if (half == 0) LP[row] = any ? (m2 + __log2f(ltot)) * 0.69314718055994531f : -INFINITY;
  }
}

// Merge P partial results per row: parts [P][rows][D] (float32, normalised),
// LSEs [P][rows]; one workgroup of D threads per row, thread t owns column t.
template <int D, bool BF16OUT>
__global__ __launch_bounds__(D) void lse_merge_kernel(const float* __restrict__ OP, const float* __restrict__ LP,
                                                      void* __restrict__ O, float* __restrict__ LSE, int P,
                                                      long rows) {
  const long row = blockIdx.x;
  const int t = threadIdx.x;
  // two passes (maximum, then weighted sums), each unrolled so that one
  // thread's loads of several parts are in flight together
  float m = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < P; ++p) m = fmaxf(m, LP[(long)p * rows + row]);
  float num = 0.0f, den = 0.0f;
  if (m > -INFINITY) {
#pragma unroll 8
    for (int p = 0; p < P; ++p) {
      const float l = LP[(long)p * rows + row];
      const float op = OP[((long)p * rows + row) * D + t];
      if (l == -INFINITY) continue;          // a part with no visible key: weight 0, its O ignored
      const float w = __expf(l - m);
      den += w;
      num += w * op;
    }
  }
  const float o = den > 0.0f ? num / den : 0.0f;
  if (BF16OUT) static_cast<__bf16*>(O)[row * D + t] = (__bf16)o;
  else static_cast<float*>(O)[row * D + t] = o;
  if (t == 0) LSE[row] = den > 0.0f ? m + __logf(den) : -INFINITY;
}

template <int D, bool BF16OUT>
hipError_t launch_merge_d(const float* op, const float* lp, void* o, float* lse, int P, long rows,
                          hipStream_t stream) {
  hipLaunchKernelGGL((lse_merge_kernel<D, BF16OUT>), dim3(rows), dim3(D), 0, stream, op, lp, o, lse, P, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_decode_d(const void* q, const void* k, const void* v, float* op, float* lp, int BH, int Nq,
                           int Nk, int S, int chunk, float scale, hipStream_t stream) {
  const int nqg = (Nq + DEC_QG - 1) / DEC_QG;
  const float c = (float)((double)__builtin_fabsf(scale) * 1.4426950408889634);
  const uint32_t qflip = scale < 0.0f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((attn_decode_bf16_kernel<D, CAUSAL>), dim3((long)S * nqg * BH), dim3(DEC_NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), op, lp, BH, Nq, Nk, nqg, S, chunk, c, qflip);
  return hipGetLastError();
}

}  // namespace

void decode_split(int B, int H, int Nq, int Nk, int* S, int* chunk) {
  // about 2048 single-wave workgroups in total, chunks of at least 256 keys
  // (a multiple of the 64-key tile)
  const long units = (long)B * H * ((Nq + DEC_QG - 1) / DEC_QG);
  long want = (2048 + units - 1) / units;
  const long max_s = ((long)Nk + 255) / 256;
  if (want > max_s) want = max_s;
  if (want < 1) want = 1;
  long ch = ((long)Nk + want - 1) / want;
  ch = (ch + BC - 1) / BC * BC;
  *chunk = (int)ch;
  *S = (int)(((long)Nk + ch - 1) / ch);
}

hipError_t launch_attn_decode_bf16(const void* q, const void* k, const void* v, float* op, float* lp, int B, int H,
                                   int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream) {
  int S, chunk;
  decode_split(B, H, Nq, Nk, &S, &chunk);
  const int BH = B * H;
  if (d == 128) return causal ? launch_decode_d<128, true>(q, k, v, op, lp, BH, Nq, Nk, S, chunk, scale, stream)
                              : launch_decode_d<128, false>(q, k, v, op, lp, BH, Nq, Nk, S, chunk, scale, stream);
  return causal ? launch_decode_d<64, true>(q, k, v, op, lp, BH, Nq, Nk, S, chunk, scale, stream)
                : launch_decode_d<64, false>(q, k, v, op, lp, BH, Nq, Nk, S, chunk, scale, stream);
}

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_lse_merge(const float* op, const float* lp, void* o, bool bf16_out, float* lse, int P, long rows,
                            int d, hipStream_t stream) {
  if (d == 128) return bf16_out ? launch_merge_d<128, true>(op, lp, o, lse, P, rows, stream)
                                : launch_merge_d<128, false>(op, lp, o, lse, P, rows, stream);
  return bf16_out ? launch_merge_d<64, true>(op, lp, o, lse, P, rows, stream)
                  : launch_merge_d<64, false>(op, lp, o, lse, P, rows, stream);
}

}  // namespace fa
