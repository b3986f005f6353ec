// C entry points of libfa.so: argument checks, kernel-instance dispatch, launch
// on the caller's stream.  Declared and documented in include/fa.h.
#include <math.h>
#include <stddef.h>

#include <map>
#include <mutex>
#include <tuple>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr long long kMaxGrid = 2147483647LL;
static_assert(fa::kDecodeScratchBytes == FA_DECODE_SCRATCH_BYTES, "the header states the scratch size");

bool sizes_ok(int B, int H, int N, int d, int rows_per_block) {
  if (B < 1 || H < 1 || N < 1) return false;
  const long long heads = (long long)B * H;
  const long long blocks = heads * ((N + (long long)rows_per_block - 1) / rows_per_block);
  if (blocks > kMaxGrid) return false;
  // element offsets are computed in 64 bits; keep the tensor far from overflow
  const long double elems = (long double)heads * N * d;
  return elems < 9.0e18L;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

namespace fa {

long device_slots(const void* kernel, int block_threads) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int>, long> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(dev, kernel, block_threads);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess) return 0;
  const long slots = (long)cus * (per_cu > 0 ? per_cu : 1);
  std::lock_guard<std::mutex> g(mu);
  cache[key] = slots;
  return slots;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;   // FP8 goes through fa_fwd_fp8
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 64)) return FA_ERR_SHAPE;
  if ((long long)N * d * 4 >= (1LL << 32)) return FA_ERR_SHAPE;   // one head's K or V must stay below 4 GiB
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (o == q || o == k || o == v || (const void*)lse == q || (const void*)lse == k || (const void*)lse == v ||
      (void*)lse == o)
    return FA_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16) return launch_status(fa::launch_attn_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, s));
  return launch_status(fa::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), static_cast<float*>(o), lse, B, H, N, d,
                                           scale, causal, s));
}

int fa_fwd_fp8_ex(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                  const float* k_scale, const float* v_scale, const uint8_t* q_mx, const uint8_t* k_mx, void* o,
                  float* lse, int B, int H, int N, int d, float scale, int causal, int flags, void* stream) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 64)) return FA_ERR_SHAPE;
  if ((long long)N * d * 4 >= (1LL << 32)) return FA_ERR_SHAPE;   // same per-head limit as fa_fwd
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if ((q_mx == nullptr) != (k_mx == nullptr)) return FA_ERR_ARG;   // MX scales for both Q and K, or neither
  if (flags & ~FA_FP8_V_HADAMARD) return FA_ERR_ARG;
  const void* ins[8] = {q8, k8, v8, q_scale, k_scale, v_scale, q_mx, k_mx};
  for (const void* p : ins)
    if (p && (p == o || p == (const void*)lse)) return FA_ERR_ARG;
  if ((void*)lse == o) return FA_ERR_ARG;
  return launch_status(fa::launch_attn_fp8(q8, k8, v8, q_scale, k_scale, v_scale, q_mx, k_mx,
                                           (flags & FA_FP8_V_HADAMARD) != 0, o, lse, B, H, N, scale, causal,
                                           static_cast<hipStream_t>(stream)));
}

int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  return fa_fwd_fp8_ex(q8, k8, v8, q_scale, k_scale, v_scale, nullptr, nullptr, o, lse, B, H, N, d, scale, causal,
                       0, stream);
}

int fa_hadamard_fp8_quant(const void* x, int in_dtype, uint8_t* x8, float* scales, int B, int H, int N, int d,
                          int hadamard, void* stream) {
  if (!x || !x8 || !scales) return FA_ERR_NULL;
  if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_DTYPE;
  if (hadamard != 0 && hadamard != 1) return FA_ERR_ARG;
  if (d != 128 && !(d == 64 && !hadamard)) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 128)) return FA_ERR_SHAPE;
  // one head of the input is addressed with 32-bit byte offsets
  if ((long long)N * d * (in_dtype == FA_F32 ? 4 : 2) >= (1LL << 32)) return FA_ERR_SHAPE;
  if ((const void*)x8 == x || (const void*)scales == x || (void*)scales == (void*)x8) return FA_ERR_ARG;
  return launch_status(fa::launch_hadamard_fp8_quant(x, in_dtype == FA_BF16, x8, scales, B, H, N, d, hadamard != 0,
                                                     static_cast<hipStream_t>(stream)));
}

int fa_mx_fp8_quant(const void* x, int in_dtype, uint8_t* x8, uint8_t* e8m0, int B, int H, int N, int d,
                    int hadamard, void* stream) {
  if (!x || !x8 || !e8m0) return FA_ERR_NULL;
  if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_DTYPE;
  if (hadamard != 0 && hadamard != 1) return FA_ERR_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 128)) return FA_ERR_SHAPE;
  if ((long long)N * d * (in_dtype == FA_F32 ? 4 : 2) >= (1LL << 32)) return FA_ERR_SHAPE;
  if ((const void*)x8 == x || (const void*)e8m0 == x || (void*)e8m0 == (void*)x8) return FA_ERR_ARG;
  return launch_status(fa::launch_mx_fp8_quant(x, in_dtype == FA_BF16, x8, e8m0, B, H, N, hadamard != 0,
                                               static_cast<hipStream_t>(stream)));
}

int fa_qkv_fp8_quant(const void* q, const void* k, const void* v, int in_dtype, uint8_t* q8, uint8_t* k8,
                     uint8_t* v8, float* q_scale, float* k_scale, float* v_scale, int B, int H, int N, int d,
                     int flags, void* stream) {
  if (!q || !k || !v || !q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale) return FA_ERR_NULL;
  if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_DTYPE;
  if (flags & ~(FA_QUANT_HADAMARD_QK | FA_QUANT_HADAMARD_V | FA_QUANT_POW2_SCALE_V)) return FA_ERR_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 128)) return FA_ERR_SHAPE;
  if ((long long)N * d * (in_dtype == FA_F32 ? 4 : 2) >= (1LL << 32)) return FA_ERR_SHAPE;
  if ((long long)B * H * ((N + 127) / 128) * 3 > kMaxGrid) return FA_ERR_SHAPE;
  const void* ins[3] = {q, k, v};
  void* outs[6] = {q8, k8, v8, q_scale, k_scale, v_scale};
  for (void* o : outs)
    for (const void* p : ins)
      if (o == p) return FA_ERR_ARG;
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (outs[i] == outs[j]) return FA_ERR_ARG;
  uint8_t* const x8[3] = {q8, k8, v8};
  float* const sc[3] = {q_scale, k_scale, v_scale};
  const int hqk = (flags & FA_QUANT_HADAMARD_QK) ? 1 : 0;
  const int had[3] = {hqk, hqk, (flags & FA_QUANT_HADAMARD_V) ? 1 : 0};
  const int pow2[3] = {0, 0, (flags & FA_QUANT_POW2_SCALE_V) ? 1 : 0};
  return launch_status(fa::launch_qkv_fp8_quant(ins, in_dtype == FA_BF16, x8, sc, had, pow2, B, H, N,
                                                static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  if (!sizes_ok(B, H, Nq, d, 1) || !sizes_ok(B, H, Nk, d, 1)) return 0;
  int S = 0, chunk = 0;
  fa::decode_split(B, H, Nq, Nk, &S, &chunk);
  return (size_t)S * B * H * Nq * (size_t)(d + 1) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points; the workspace size they need
// goes to *need.
int decode_checks(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int Nq,
                  int Nk, int d, float scale, int causal, size_t* need) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, Nq, d, 32) || !sizes_ok(B, H, Nk, d, 64)) return FA_ERR_SHAPE;
  if ((long long)Nk * d * 4 >= (1LL << 32) || (long long)Nq * d * 4 >= (1LL << 32)) return FA_ERR_SHAPE;
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;   // the queries are the last Nq of the Nk tokens
  int S = 0, chunk = 0;
  fa::decode_split(B, H, Nq, Nk, &S, &chunk);
  const long long units = (long long)S * B * H * ((Nq + 31) / 32);
  if (units > kMaxGrid || (long long)B * H * Nq > kMaxGrid) return FA_ERR_SHAPE;
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (p == o || p == (const void*)lse) return FA_ERR_ARG;
  if ((const void*)lse == o) return FA_ERR_ARG;
  *need = (size_t)S * B * H * Nq * (size_t)(d + 1) * sizeof(float);
  return FA_OK;
}

int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, void* workspace, hipStream_t s) {
  int S = 0, chunk = 0;
  fa::decode_split(B, H, Nq, Nk, &S, &chunk);
  float* op = static_cast<float*>(workspace);
  float* lp = op + (size_t)S * B * H * Nq * d;
  hipError_t e = fa::launch_attn_decode_bf16(q, k, v, op, lp, B, H, Nq, Nk, d, scale, causal != 0, s);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  return launch_status(fa::launch_lse_merge(op, lp, o, true, lse, S, (long)B * H * Nq, d, s));
}

}  // namespace

extern "C" {

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const int st = decode_checks(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, &need);
  if (st != FA_OK) return st;
  if (!workspace) return FA_ERR_NULL;
  if (workspace_bytes < need) return FA_ERR_ARG;
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (p == (const void*)workspace) return FA_ERR_ARG;
  if (workspace == o || workspace == (void*)lse) return FA_ERR_ARG;
  return decode_launch(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, workspace, static_cast<hipStream_t>(stream));
}

int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                          int Nk, int d, float scale, int causal, void* stream) {
  size_t need = 0;
  const int st = decode_checks(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, &need);
  if (st != FA_OK) return st;
  if (need > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  return decode_launch(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, ws, static_cast<hipStream_t>(stream));
}

int fa_lse_merge(const float* o_parts, const float* lse_parts, int P, int B, int H, int N, int d, void* o,
                 int o_dtype, float* lse, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (P < 1 || !sizes_ok(B, H, N, d, 1)) return FA_ERR_SHAPE;
  if ((long double)P * B * H * N * d >= 9.0e18L) return FA_ERR_SHAPE;
  const void* ins[2] = {o_parts, lse_parts};
  for (const void* p : ins)
    if (p == o || p == (const void*)lse) return FA_ERR_ARG;
  if ((void*)lse == o) return FA_ERR_ARG;
  return launch_status(fa::launch_lse_merge(o_parts, lse_parts, o, o_dtype == FA_BF16, lse, P, (long)B * H * N, d,
                                            static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if ((d != 64 && d != 128) || !sizes_ok(B, H, N, d, 1)) return 0;
  return fa::attn_bwd_workspace_bytes(B, H, N, d);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!sizes_ok(B, H, N, d, 128)) return FA_ERR_SHAPE;   // the dK/dV pass: 128 keys per workgroup (dQ: 256 queries)
  if ((long long)N * d * 4 >= (1LL << 32)) return FA_ERR_SHAPE;   // same per-head limit as fa_fwd
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (workspace_bytes < fa::attn_bwd_workspace_bytes(B, H, N, d)) return FA_ERR_ARG;
  const void* ins[6] = {q, k, v, o, lse, dout};
  void* outs[4] = {dq, dk, dv, workspace};
  for (void* w : outs)
    for (const void* p : ins)
      if (w == p) return FA_ERR_ARG;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (outs[i] == outs[j]) return FA_ERR_ARG;
  return launch_status(fa::launch_attn_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale,
                                                causal != 0, static_cast<hipStream_t>(stream)));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N below 1, or the sizes exceed the supported range";
    case FA_ERR_DTYPE: return "unknown or unsupported dtype for this entry point";
    case FA_ERR_UNSUPPORTED: return "head dimension not supported for this entry point";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ARG:
      return "invalid argument: non-finite scale, flag not 0/1, an output aliasing an input, or a workspace too small";
    case FA_ERR_SCRATCH: return "the sizes need more scratch than the library's static device array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
