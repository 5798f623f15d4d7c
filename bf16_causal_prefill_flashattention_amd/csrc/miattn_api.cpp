// C ABI of libmiattn.so: host-side argument validation and dispatch to the
// gfx950 kernels.  Declarations and the contract of every entry point are in
// include/miattn.h.
#include "../../include/miattn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "kernels.h"

static_assert(MIATTN_P_LEAN == miattn::kPLean && MIATTN_P_LEAN_BLOCK == miattn::kPLeanBlock &&
                  MIATTN_P_EXACT == miattn::kPExact && MIATTN_P_EXACT_BLOCK == miattn::kPExactBlock &&
                  MIATTN_P_LEAN_TILE == miattn::kPLeanTile && MIATTN_P_EXACT_TILE == miattn::kPExactTile,
              "the ABI's probability modes are the kernels' modes");

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dims(int d_qk, int d_v) { return d_v == 128 && (d_qk == 128 || d_qk == 192); }

// Validation touches no device state, so a rejected call enqueues nothing.
int validate_attn_fwd(const void* q, const void* k, const void* v, void* out, const float* lse, int B, int Hq,
                      int Hkv, int Nq, int Nk, int d_qk, int d_v, int dtype, const float* qs, const float* ks,
                      const float* vs) {
  if (dtype != MIATTN_DTYPE_BF16 && dtype != MIATTN_DTYPE_FP8_E4M3) return MIATTN_ERR_DTYPE;
  if (B < 0 || Nq < 0 || Nk < Nq || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return MIATTN_ERR_SIZE;
  if (!supported_dims(d_qk, d_v)) return MIATTN_ERR_SHAPE;
  if (B == 0 || Nq == 0) return MIATTN_OK;  // empty: pointers are not dereferenced
  if (!q || !k || !v || !out) return MIATTN_ERR_NULL;
  if (dtype == MIATTN_DTYPE_FP8_E4M3 && (!qs || !ks || !vs)) return MIATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return MIATTN_ERR_ALIGN;
  if (dtype == MIATTN_DTYPE_FP8_E4M3 && (!aligned(qs, 4) || !aligned(ks, 4) || !aligned(vs, 4)))
    return MIATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return MIATTN_ERR_ALIGN;
  // every element offset must fit in 63 bits and the grid in a 31-bit count
  const double dmax = (double)(d_qk > d_v ? d_qk : d_v);
  if ((double)B * (double)Nk * (double)Hq * dmax > 9.0e18) return MIATTN_ERR_SIZE;
  if ((double)B * Hq > 2147483647.0) return MIATTN_ERR_SIZE;
  // kernels address one 128-key tile of K or V with 32-bit offsets
  if ((double)Hkv * dmax * 2.0 * 128.0 > 2147483647.0) return MIATTN_ERR_SIZE;
  const long long units = miattn::attn_fwd_units(B, Hq, Nq);
  if (units <= 0 || units > 0x7fffffffLL) return MIATTN_ERR_SIZE;
  return MIATTN_OK;
}

miattn::AttnParams shape_params(int B, int Hq, int Hkv, int Nq, int Nk, int dtype, bool block64, int p_mode) {
  miattn::AttnParams p{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.block64 = block64 ? 1 : 0;
  p.p_mode = dtype == MIATTN_DTYPE_FP8_E4M3 ? p_mode : miattn::kPLean;  // BF16 has one mode
  return p;
}

// ws == nullptr: no key split.  Otherwise the launch splits its keys when the
// plan for the current device says so, with the workspace at ws.
int run_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                 const float* v_scale, double tau, void* stream, bool block64 = false,
                 int p_mode = MIATTN_P_DEFAULT, void* ws = nullptr, size_t ws_bytes = 0) {
  miattn::AttnParams p = shape_params(B, Hq, Hkv, Nq, Nk, dtype, block64, p_mode);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.sm_scale_log2 = (float)(1.4426950408889634 * tau);  // log2-domain softmax scale
  if (ws != nullptr) {
    miattn::SplitPlan plan;
    if (miattn::attn_split_plan(p, dtype, d_qk, d_v, &plan) != hipSuccess) return MIATTN_ERR_HIP;
    if (plan.tiles > 0) {
      if (ws_bytes < plan.bytes) return MIATTN_ERR_SIZE;
      p.split_tiles = plan.tiles;
      p.split_units = plan.units;
      p.ws_o = static_cast<float*>(ws);
      p.ws_lse = p.ws_o + (size_t)B * Hq * plan.units * miattn::kQueryTile * d_v;
    }
  }
  const hipError_t e = miattn::launch_attn_fwd(p, dtype, d_qk, d_v, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

int validate_quantize(const void* x, int x_dtype, void* y, float* scale, int B, int H, int N, int d,
                      int hadamard) {
  if (x_dtype != MIATTN_SRC_FP32 && x_dtype != MIATTN_SRC_BF16) return MIATTN_ERR_DTYPE;
  if (hadamard != 0 && hadamard != 1) return MIATTN_ERR_DTYPE;
  if (B < 0 || N < 0 || H < 1) return MIATTN_ERR_SIZE;
  if (d != 128 && d != 192) return MIATTN_ERR_SHAPE;
  if (B == 0) return MIATTN_OK;
  if (!scale) return MIATTN_ERR_NULL;
  if (N > 0 && (!x || !y)) return MIATTN_ERR_NULL;
  if (!aligned(scale, 4)) return MIATTN_ERR_ALIGN;
  if (N > 0 && (!aligned(x, 16) || !aligned(y, 16))) return MIATTN_ERR_ALIGN;
  if ((double)B * H > 2147483647.0 / 1024.0) return MIATTN_ERR_SIZE;
  const double blocks = (double)B * H * ((N + 255) / 256);
  if (blocks > 2147483647.0) return MIATTN_ERR_SIZE;
  if ((double)B * N * H * d > 9.0e18) return MIATTN_ERR_SIZE;
  return MIATTN_OK;
}

}  // namespace

extern "C" {

int attn_version(void) { return MIATTN_ABI_VERSION; }

const char* attn_status_string(int status) {
  switch (status) {
    case MIATTN_OK: return "success";
    case MIATTN_ERR_NULL: return "a required pointer is NULL";
    case MIATTN_ERR_SIZE: return "invalid size (negative, zero head count, Hq not a multiple of Hkv, Nq > Nk, or too large)";
    case MIATTN_ERR_SHAPE: return "unsupported head dimensions (need (128,128) or (192,128); the quantizer needs d in {128, 192})";
    case MIATTN_ERR_DTYPE: return "unknown dtype, source type or flag value";
    case MIATTN_ERR_HIP: return "the HIP runtime reported an error while enqueuing";
    case MIATTN_ERR_ALIGN: return "misaligned pointer (tensors need 16-byte, scales and lse 4-byte alignment)";
    case MIATTN_ERR_VALUE: return "invalid scalar argument (softmax scale must be finite and positive, or 0)";
    case MIATTN_ERR_SCRATCH: return "the launch needs more workspace than the static scratch of attn_fwd_noalloc holds";
    default: return "unknown status code";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d_qk,
             int d_v, int dtype, const float* q_scale, const float* k_scale, const float* v_scale, void* stream) {
  const int st =
      validate_attn_fwd(q, k, v, out, nullptr, B, Hq, Hkv, N, N, d_qk, d_v, dtype, q_scale, k_scale, v_scale);
  if (st != MIATTN_OK || B == 0 || N == 0) return st;
  return run_attn_fwd(q, k, v, out, nullptr, B, Hq, Hkv, N, N, d_qk, d_v, dtype, q_scale, k_scale, v_scale,
                      1.0 / std::sqrt((double)d_qk), stream);
}

int attn_fwd_chunk(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                   const float* v_scale, float softmax_scale, void* stream) {
  if (!(softmax_scale == 0.0f || (std::isfinite(softmax_scale) && softmax_scale > 0.0f))) return MIATTN_ERR_VALUE;
  const int st =
      validate_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, q_scale, k_scale, v_scale);
  if (st != MIATTN_OK || B == 0 || Nq == 0) return st;
  const double tau = softmax_scale == 0.0f ? 1.0 / std::sqrt((double)d_qk) : (double)softmax_scale;
  return run_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, q_scale, k_scale, v_scale, tau,
                      stream);
}

int attn_quantize_fp8(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N, int d,
                      int hadamard, void* stream) {
  const int st = validate_quantize(x, x_dtype, x_fp8, scale, B, H, N, d, hadamard);
  if (st != MIATTN_OK || B == 0) return st;
  const hipError_t e =
      miattn::launch_quantize_fp8(x, x_dtype, x_fp8, scale, B, H, N, d, hadamard != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

int attn_fwd_block64(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d_qk, int d_v, const float* q_scale, const float* k_scale,
                     const float* v_scale, float softmax_scale, int p_block_scale, void* stream) {
  if (p_block_scale != 0 && p_block_scale != 1) return MIATTN_ERR_DTYPE;
  if (!(softmax_scale == 0.0f || (std::isfinite(softmax_scale) && softmax_scale > 0.0f))) return MIATTN_ERR_VALUE;
  const int st = validate_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, MIATTN_DTYPE_FP8_E4M3, q_scale,
                                   k_scale, v_scale);
  if (st != MIATTN_OK) return st;
  if (Nk > miattn::kBlock64MaxKeys) return MIATTN_ERR_SIZE;
  if (B == 0 || Nq == 0) return MIATTN_OK;
  const double tau = softmax_scale == 0.0f ? 1.0 / std::sqrt((double)d_qk) : (double)softmax_scale;
  return run_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, MIATTN_DTYPE_FP8_E4M3, q_scale, k_scale,
                      v_scale, tau, stream, true, p_block_scale != 0 ? MIATTN_P_LEAN_BLOCK : MIATTN_P_LEAN);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d_qk, int d_v, const float* q_scale, const float* k_scale, const float* v_scale,
                 float softmax_scale, int scales, int p_mode, void* stream) {
  if (scales != MIATTN_SCALES_HEAD && scales != MIATTN_SCALES_BLOCK64) return MIATTN_ERR_DTYPE;
  if (p_mode < MIATTN_P_LEAN || p_mode > MIATTN_P_EXACT_TILE) return MIATTN_ERR_DTYPE;
  if (!(softmax_scale == 0.0f || (std::isfinite(softmax_scale) && softmax_scale > 0.0f))) return MIATTN_ERR_VALUE;
  const int st = validate_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, MIATTN_DTYPE_FP8_E4M3, q_scale,
                                   k_scale, v_scale);
  if (st != MIATTN_OK) return st;
  if (scales == MIATTN_SCALES_BLOCK64 && Nk > miattn::kBlock64MaxKeys) return MIATTN_ERR_SIZE;
  if (B == 0 || Nq == 0) return MIATTN_OK;
  const double tau = softmax_scale == 0.0f ? 1.0 / std::sqrt((double)d_qk) : (double)softmax_scale;
  return run_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, MIATTN_DTYPE_FP8_E4M3, q_scale, k_scale,
                      v_scale, tau, stream, scales == MIATTN_SCALES_BLOCK64, p_mode);
}

int attn_fwd_ws_size(int B, int Hq, int Hkv, int Nq, int Nk, int d_qk, int d_v, int dtype, int scales, int p_mode,
                     size_t* bytes) {
  if (!bytes) return MIATTN_ERR_NULL;
  *bytes = 0;
  if (dtype != MIATTN_DTYPE_BF16 && dtype != MIATTN_DTYPE_FP8_E4M3) return MIATTN_ERR_DTYPE;
  if (scales != MIATTN_SCALES_HEAD && scales != MIATTN_SCALES_BLOCK64) return MIATTN_ERR_DTYPE;
  if (p_mode < MIATTN_P_LEAN || p_mode > MIATTN_P_EXACT_TILE) return MIATTN_ERR_DTYPE;
  if (B < 0 || Nq < 0 || Nk < Nq || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return MIATTN_ERR_SIZE;
  if (!supported_dims(d_qk, d_v)) return MIATTN_ERR_SHAPE;
  if (B == 0 || Nq == 0) return MIATTN_OK;
  const bool block64 = dtype == MIATTN_DTYPE_FP8_E4M3 && scales == MIATTN_SCALES_BLOCK64;
  const miattn::AttnParams p = shape_params(B, Hq, Hkv, Nq, Nk, dtype, block64, p_mode);
  miattn::SplitPlan plan;
  if (miattn::attn_split_plan(p, dtype, d_qk, d_v, &plan) != hipSuccess) return MIATTN_ERR_HIP;
  *bytes = plan.bytes;
  return MIATTN_OK;
}

int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Nq,
                int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                const float* v_scale, float softmax_scale, int scales, int p_mode, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (scales != MIATTN_SCALES_HEAD && scales != MIATTN_SCALES_BLOCK64) return MIATTN_ERR_DTYPE;
  if (p_mode < MIATTN_P_LEAN || p_mode > MIATTN_P_EXACT_TILE) return MIATTN_ERR_DTYPE;
  if (!(softmax_scale == 0.0f || (std::isfinite(softmax_scale) && softmax_scale > 0.0f))) return MIATTN_ERR_VALUE;
  const int st =
      validate_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, q_scale, k_scale, v_scale);
  if (st != MIATTN_OK) return st;
  const bool block64 = dtype == MIATTN_DTYPE_FP8_E4M3 && scales == MIATTN_SCALES_BLOCK64;
  if (block64 && Nk > miattn::kBlock64MaxKeys) return MIATTN_ERR_SIZE;
  if (B == 0 || Nq == 0) return MIATTN_OK;
  size_t need = 0;
  const int sst = attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, scales, p_mode, &need);
  if (sst != MIATTN_OK) return sst;
  if (need > 0) {
    if (!workspace) return MIATTN_ERR_NULL;
    if (!aligned(workspace, 16)) return MIATTN_ERR_ALIGN;
    if (workspace_bytes < need) return MIATTN_ERR_SIZE;
  }
  const double tau = softmax_scale == 0.0f ? 1.0 / std::sqrt((double)d_qk) : (double)softmax_scale;
  return run_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, q_scale, k_scale, v_scale, tau,
                      stream, block64, dtype == MIATTN_DTYPE_FP8_E4M3 ? p_mode : MIATTN_P_LEAN,
                      need > 0 ? workspace : nullptr, workspace_bytes);
}

int attn_quantize_fp8_block64(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N, int d,
                              int hadamard, void* stream) {
  const int st = validate_quantize(x, x_dtype, x_fp8, scale, B, H, N, d, hadamard);
  if (st != MIATTN_OK || B == 0 || N == 0) return st;
  if ((double)B * H * ((N + 63) / 64) > 2147483647.0) return MIATTN_ERR_SIZE;  // one workgroup per block
  const hipError_t e = miattn::launch_quantize_fp8_block64(x, x_dtype, x_fp8, scale, B, H, N, d, hadamard != 0,
                                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

}  // extern "C"
