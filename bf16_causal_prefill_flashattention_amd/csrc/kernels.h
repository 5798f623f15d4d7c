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
  // FP8 scales.  Per head (block64 == 0): q [B, Hq], k and v [B, Hkv].
  // Per 64 positions (block64 != 0): q [B, Hq, ceil(Nq/64)], k and v
  // [B, Hkv, ceil(Nk/64)]; the k and v scales are powers of two, applied by the
  // scaled MFMAs as their E8M0 exponents.
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int B, Hq, Hkv, Nq, Nk;
  float sm_scale_log2;  // softmax scale times log2(e)
  int block64;
  // FP8 probability mode (PMode): how the probabilities are rounded to e4m3
  // for the P.V product
  int p_mode;
};

// FP8 probability modes.  Lean: the e4m3 code of 2^x written from one FMA on
// the log2-domain score; exact: exp2 and the hardware e4m3 conversion.  Both
// scale the probabilities by a fixed 2^6 before rounding; the block modes also
// shift each query's probabilities of every 64-key step by 2^k, k the octaves
// their max lies below the running max, and the tile modes do the same once
// per key tile; the scaled MFMAs undo the shift.
enum PMode { kPLean = 0, kPLeanBlock = 1, kPExact = 2, kPExactBlock = 3, kPLeanTile = 4, kPExactTile = 5 };

// Largest key count of a block-scaled launch: the exponents of all key tiles of
// a work item are staged in LDS (one 32-bit word per 128-key tile).
constexpr int kBlock64MaxKeys = 1 << 20;

// Work units of one attention launch (pairs of query tiles of one batch and
// head); the launch runs min(units, CUs) persistent workgroups.
long long attn_fwd_units(int B, int Hq, int Nq);
// Query tiles (work items) of one launch.
long long attn_fwd_tiles(int B, int Hq, int Nq);

// dtype: 0 = bf16, 1 = fp8 e4m3fn (p.block64 selects the scale granularity,
// p.p_mode the probability mode).  (d_qk, d_v) in {(128,128), (192,128)}.
hipError_t launch_attn_fwd(const AttnParams& p, int dtype, int d_qk, int d_v, hipStream_t stream);

// Per-family launchers (one translation unit each), called by launch_attn_fwd
// with the grid it chose.
hipError_t launch_attn_bf16(const AttnParams& p, int d_qk, dim3 grid, hipStream_t stream);
hipError_t launch_attn_fp8_head_d128(const AttnParams& p, dim3 grid, hipStream_t stream);
hipError_t launch_attn_fp8_head_d192(const AttnParams& p, dim3 grid, hipStream_t stream);
hipError_t launch_attn_fp8_block64_d128(const AttnParams& p, dim3 grid, hipStream_t stream);
hipError_t launch_attn_fp8_block64_d192(const AttnParams& p, dim3 grid, hipStream_t stream);

// x: [B, N, H, d] fp32 (x_dtype 0) or bf16 (x_dtype 1); x_fp8 same shape, u8;
// scale: [B, H] fp32, also used as the amax accumulator while the call runs.
hipError_t launch_quantize_fp8(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N,
                               int d, bool hadamard, hipStream_t stream);

// Same source and code layout; scale: [B, H, ceil(N/64)] fp32 powers of two.
hipError_t launch_quantize_fp8_block64(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N,
                                       int d, bool hadamard, hipStream_t stream);

}  // namespace miattn
