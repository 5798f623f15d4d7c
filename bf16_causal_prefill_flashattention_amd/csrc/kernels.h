// Internal (C++) interface between the C ABI layer and the HIP kernels.
// Not exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>

namespace miattn {

// The Nq queries are the last Nq positions of a sequence whose first Nk
// positions of keys and values are given (Nq <= Nk): query row i sits at
// position i + Nk - Nq and sees keys j <= i + Nk - Nq.  Nq == Nk is plain
// causal prefill.
struct AttnParams {
  const void* q;  // [B, Nq, Hq, d_qk]
  const void* k;  // [B, Nk, Hkv, d_qk]
  const void* v;  // [B, Nk, Hkv, d_v]
  void* out;      // [B, Nq, Hq, d_v] bf16
  float* lse;     // [B, Hq, Nq] fp32 natural-log sum of exp of the scaled scores, or null
  const float* q_scale;  // [B, Hq]  (FP8 only)
  const float* k_scale;  // [B, Hkv] (FP8 only)
  const float* v_scale;  // [B, Hkv] (FP8 only)
  int B, Hq, Hkv, Nq, Nk;
  float sm_scale_log2;  // softmax scale times log2(e)
};

// Work units of one attention launch (pairs of query tiles of one batch and
// head); the launch runs min(units, CUs) persistent workgroups.
long long attn_fwd_units(int B, int Hq, int Nq);
// Query tiles (work items) of one launch.
long long attn_fwd_tiles(int B, int Hq, int Nq);

// dtype: 0 = bf16, 1 = fp8 e4m3fn.  (d_qk, d_v) in {(128,128), (192,128)}.
hipError_t launch_attn_fwd(const AttnParams& p, int dtype, int d_qk, int d_v, hipStream_t stream);

// x: [B, N, H, d] fp32 (x_dtype 0) or bf16 (x_dtype 1); x_fp8 same shape, u8;
// scale: [B, H] fp32, also used as the amax accumulator while the call runs.
hipError_t launch_quantize_fp8(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N,
                               int d, bool hadamard, hipStream_t stream);

}  // namespace miattn
