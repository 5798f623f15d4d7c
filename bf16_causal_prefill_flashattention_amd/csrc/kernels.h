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
  // Key split (split_tiles > 0, chosen by attn_split_plan): query tile qt of a
  // (batch, head) is cut into ceil(T / split_tiles) work items over consecutive
  // ranges of split_tiles key tiles (T = the key tiles it needs); the
  // split_units items of a (batch, head) are its query tiles' ranges in order.
  // Items of a query tile with more than one range write their output rows
  // normalised, in fp32, to ws_o [B*Hq*split_units, kQueryTile, d_v] and their
  // log2-domain sums of exp to ws_lse [B*Hq*split_units, kQueryTile] (slot
  // bh * split_units + item), and attn_merge_kernel combines the ranges.
  int split_tiles;
  int split_units;
  // set by launch_attn_fwd: 1 runs 128-query items on 4-wave workgroups (see kSoloQueryTile)
  int solo;
  // set by launch_attn_fwd: 1 deals the query tiles to the persistent
  // workgroups in snake order of cost instead of as heavy/light pairs (when
  // the pairs do not split evenly over the workgroups)
  int snake;
  float* ws_o;
  float* ws_lse;
};

// Queries per work item (one workgroup of 8 waves x 32 queries).
constexpr int kQueryTile = 256;
// Queries per work item of the 4-wave mode, used by unsplit launches of at
// most kSoloMaxKeys keys whose 256-query items leave CUs idle while their
// 128-query items fit one per CU: each wave then does its own matrix and
// vector work of every step (one wave per SIMD), and twice as many CUs share
// the launch.  The longest item still walks every key tile, one step per tile
// as before, and a step of one wave doing both halves takes a little longer
// than a ping-pong step; what the mode saves is per item (half the queries to
// load and rows to store), so it pays on short key ranges only.
constexpr int kSoloQueryTile = 128;
constexpr int kSoloMaxKeys = 1536;

// Launches with at most this many keys use 128-key FP8 tiles where the kernel
// would otherwise use 192: a short sequence's last query tile wastes less of
// its final key tile (measured on MI355X: 1K tokens 7% and 4K 6% faster with
// 128, 16K and 32K 2-4% slower).
constexpr int kShortKeys = 4096;

// Keys per tile of a kernel variant: FP8 at d_qk = 128 without the per-64-key
// probability shift streams 192-key tiles (128 when the launch has at most
// kShortKeys keys), the other FP8 variants 128; BF16 128 at d_qk = 128 and 64
// at d_qk = 192.  (block64: the scale granularity, which does not change it.)
constexpr int tile_keys_of(bool fp8, int d_qk, bool block64, bool shift_step, bool short_keys = false) {
  (void)block64;
  return fp8 ? ((d_qk == 128 && !shift_step && !short_keys) ? 192 : 128) : (d_qk == 128 ? 128 : 64);
}

// Key tiles query tile qt needs: keys up to the position of its last query.
__host__ __device__ inline int qtile_key_tiles(int qt, int Nq, int Nk, int bn) {
  const long long last = (long long)(qt + 1) * kQueryTile < Nq ? (long long)(qt + 1) * kQueryTile : Nq;
  return (int)((last + (Nk - Nq) - 1) / bn + 1);
}

// Key split of one launch on the current device: tiles = key tiles per work
// item (0: no split), units = work items per (batch, head), bytes = workspace,
// first_qt = the first query tile with more than one range.
struct SplitPlan {
  int tiles, units, first_qt;
  size_t bytes;
};
hipError_t attn_split_plan(const AttnParams& p, int dtype, int d_qk, int d_v, SplitPlan* plan);

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
