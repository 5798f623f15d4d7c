// Launch of the causal forward attention: grid size, the key split of short
// launches, the choice of kernel variant (dtype, head dimensions, FP8 scale
// granularity and probability mode) and the merge of split key ranges.
// The kernel template is in attn_fwd_impl.hpp; its variants are instantiated in
// attn_fwd_bf16.hip and attn_fwd_fp8_{head,block64}_d{128,192}.hip.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <atomic>

#include "device_common.hpp"
#include "kernels.h"

namespace miattn {

namespace {
constexpr int kBM = kQueryTile;
constexpr int kMergeRows = 8;  // query rows per merge workgroup (32 lanes per row, 4 channels each)

// CU count per device, filled on first use (atomic: concurrent callers may
// both fill it, with the same value)
hipError_t device_cus(int* cus) {
  static std::atomic<int> cu_count[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    n = n > 0 ? n : 1;
    cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
}

int variant_tile_keys(const AttnParams& p, int dtype, int d_qk) {
  return tile_keys_of(dtype != 0, d_qk, p.block64 != 0, p.p_mode == kPLeanBlock || p.p_mode == kPExactBlock,
                      p.Nk <= kShortKeys);
}

// Key ranges of query tile qt with ranges of L tiles.
__host__ __device__ inline int qtile_ranges(int qt, int Nq, int Nk, int bn, int L) {
  return (qtile_key_tiles(qt, Nq, Nk, bn) + L - 1) / L;
}

// Merge of the key ranges of the split query tiles: workgroup = kMergeRows
// query rows of one (batch, head) and query tile >= first_qt; lane group of 32
// = one row, 4 channels per lane.  With r the ranges of the row's query tile
// and (o_s, e_s) range s's normalised output and log2 sum of exp:
//   E = max_s e_s,  w_s = 2^(e_s - E),  out = sum_s w_s o_s / sum_s w_s,
//   lse = ln 2 * (E + log2 sum_s w_s),
// summed in range order (deterministic).  Range 0 holds key 0, which every
// query sees, so E is finite.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p, int bn, int first_qt) {
  const int nqt = (p.Nq + kBM - 1) / kBM;
  const int per_bh = (nqt - first_qt) * (kBM / kMergeRows);
  const int bh = blockIdx.x / per_bh, rem = blockIdx.x % per_bh;
  const int qt = first_qt + rem / (kBM / kMergeRows);
  const int row = (rem % (kBM / kMergeRows)) * kMergeRows + threadIdx.x / 32;
  const int q = qt * kBM + row;
  if (q >= p.Nq) return;
  const int L = p.split_tiles, U = p.split_units;
  int u0 = 0;  // the tile's first unit within its (batch, head)
  for (int j = 0; j < qt; ++j) u0 += qtile_ranges(j, p.Nq, p.Nk, bn, L);
  const int nr = qtile_ranges(qt, p.Nq, p.Nk, bn, L);
  const size_t slot0 = (size_t)bh * U + u0;
  float e_max = -INFINITY;
  for (int s = 0; s < nr; ++s) e_max = fmaxf(e_max, p.ws_lse[(slot0 + s) * kBM + row]);
  const int c = 4 * (threadIdx.x % 32);
  float den = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nr; ++s) {
    const size_t r = (slot0 + s) * kBM + row;
    const float w = exp2f(p.ws_lse[r] - e_max);
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.ws_o + r * 128 + c);
    den += w;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, o[i], acc[i]);
  }
  const float inv = 1.f / den;
  const int b = bh / p.Hq, h = bh % p.Hq;
  __bf16* out = static_cast<__bf16*>(p.out) + (((size_t)b * p.Nq + q) * p.Hq + h) * 128 + c;
  const i32x2 v2 = {(int)pack_bf16x2(acc[0] * inv, acc[1] * inv), (int)pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<i32x2*>(out) = v2;
  if (p.lse != nullptr && c == 0) p.lse[(size_t)bh * p.Nq + q] = (e_max + log2f(den)) * 0.69314718055994531f;
}
}  // namespace

long long attn_fwd_units(int B, int Hq, int Nq) {
  const long long nqt = (Nq + kBM - 1) / kBM;
  return (long long)B * Hq * ((nqt + 1) / 2);
}

long long attn_fwd_tiles(int B, int Hq, int Nq) {
  return (long long)B * Hq * ((Nq + kBM - 1) / kBM);
}

// A launch whose query tiles leave CUs idle (one tile per workgroup) is bound
// by its longest query tile, the last one, which walks every key tile.  The
// split cuts every query tile into ranges of at most L key tiles, so the
// longest item walks L tiles, at the price of writing the ranges' fp32 rows
// and reading them back in the merge.  The plan takes the L (among the
// smallest that gives every range a CU of its own, and its doublings) with the
// least modelled time, and splits only when that beats the unsplit launch.
// Time model, fitted to MI355X measurements of split and unsplit launches
// (1K and 4K tokens at 8 and 32 heads, 16K at 2 heads, 512- and 1024-query
// chunks against 32K keys): a key tile of the longest item costs ~1 us at
// full occupancy for 24576 MFMA-cycles' worth of work (192 FP8 or 96 BF16 keys
// at d = 128), partial rows ~0.55 us per MB written and read back, plus 2 us
// for the merge.  (At 1K tokens and 32 heads, or 4K tokens and 8 heads, the
// partial rows cost about what the shorter critical path saves, so such
// launches stay unsplit; a short chunk against a long prefix splits.)
hipError_t attn_split_plan(const AttnParams& p, int dtype, int d_qk, int d_v, SplitPlan* plan) {
  *plan = SplitPlan{0, 0, 0, 0};
  if (p.B < 1 || p.Nq < 1 || d_v != 128) return hipSuccess;
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const long long nbh = (long long)p.B * p.Hq;
  const int nqt = (p.Nq + kBM - 1) / kBM;
  if (nbh * nqt > cus) return hipSuccess;  // no idle CUs
  const int bn = variant_tile_keys(p, dtype, d_qk);
  const int tmax = qtile_key_tiles(nqt - 1, p.Nq, p.Nk, bn);
  auto units = [&](int L) {
    long long u = 0;
    for (int j = 0; j < nqt; ++j) u += qtile_ranges(j, p.Nq, p.Nk, bn, L);
    return u;
  };
  // smallest L with nbh * units(L) <= cus (units is non-increasing in L)
  int lo = 1, hi = tmax;  // units(tmax) = nqt fits
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (nbh * units(mid) <= cus) hi = mid; else lo = mid + 1;
  }
  const double tile_us = bn * (d_qk + d_v) / (dtype != 0 ? 2.0 : 1.0) / 24576.0;
  auto split_us = [&](int L) {
    double rows = 0;  // partial rows: the rows of the query tiles with more than one range, per range
    for (int j = 0; j < nqt; ++j) {
      const int r = qtile_ranges(j, p.Nq, p.Nk, bn, L);
      if (r > 1) rows += (double)r * std::min(kBM, p.Nq - j * kBM);
    }
    const double bytes = (double)nbh * rows * (d_v + 1) * sizeof(float);
    return L * tile_us + bytes * 0.55e-6 + 2.0;
  };
  int best = 0;
  double best_us = tmax * tile_us;
  for (int L = std::max(lo, 2); L <= tmax - 2; L *= 2) {
    const double t = split_us(L);
    if (t < best_us) {
      best = L;
      best_us = t;
    }
  }
  if (best == 0) return hipSuccess;
  int first = 0;
  while (qtile_ranges(first, p.Nq, p.Nk, bn, best) == 1) ++first;
  plan->tiles = best;
  plan->units = (int)units(best);
  plan->first_qt = first;
  plan->bytes = (size_t)nbh * plan->units * kBM * (d_v + 1) * sizeof(float);
  return hipSuccess;
}

hipError_t launch_attn_fwd(const AttnParams& p, int dtype, int d_qk, int d_v, hipStream_t stream) {
  if (p.Nq < 1 || p.Nk < p.Nq) return hipErrorInvalidValue;
  if (d_v != 128 || (d_qk != 128 && d_qk != 192)) return hipErrorInvalidValue;
  if (p.p_mode < kPLean || p.p_mode > kPExactTile) return hipErrorInvalidValue;
  if (dtype == 0 && (p.block64 || p.p_mode != kPLean)) return hipErrorInvalidValue;
  if (p.block64 && p.Nk > kBlock64MaxKeys) return hipErrorInvalidValue;
  const long long units = attn_fwd_units(p.B, p.Hq, p.Nq);
  if (units <= 0 || units > 0x7fffffffLL) return hipErrorInvalidValue;
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const long long tiles = attn_fwd_tiles(p.B, p.Hq, p.Nq);
  AttnParams lp = p;
  lp.solo = 0;
  lp.snake = 0;
  dim3 grid;
  int first_qt = 0;
  if (p.split_tiles > 0) {
    // the plan must be attn_split_plan's for these arguments
    SplitPlan plan;
    e = attn_split_plan(p, dtype, d_qk, d_v, &plan);
    if (e != hipSuccess) return e;
    if (plan.tiles != p.split_tiles || plan.units != p.split_units || !p.ws_o || !p.ws_lse)
      return hipErrorInvalidValue;
    grid = dim3((unsigned)((long long)p.B * p.Hq * p.split_units));
    first_qt = plan.first_qt;
  } else {
    const long long solo_items = (long long)p.B * p.Hq * ((p.Nq + kSoloQueryTile - 1) / kSoloQueryTile);
    if (tiles < cus && solo_items <= cus && p.Nk <= kSoloMaxKeys && variant_tile_keys(p, dtype, d_qk) <= 128) {
      // 256-query items leave CUs idle and 128-query items fit one per CU:
      // one 4-wave workgroup per 128-query item (the 4-wave kernels exist for
      // tiles of at most 128 keys)
      lp.solo = 1;
      grid = dim3((unsigned)solo_items);
    } else {
      // as many workgroups as CUs, or one per tile when the tiles do not fill
      // the CUs (the kernel derives the same choice from gridDim)
      grid = dim3(tiles <= cus ? (int)tiles : (int)std::min<long long>(units, cus));
      // Pairs of equal cost balance the CUs when they split evenly over them;
      // otherwise (e.g. 384 pairs, or 192, on 256 CUs) a round of pairs runs
      // on part of the CUs only, and dealing single tiles in snake order of
      // cost over all CUs evens the load out.
      // (per-head scales and BF16; tile positions stay in int)
      if (tiles > cus && units % cus != 0 && !p.block64 && tiles < (1LL << 30)) {
        lp.snake = 1;
        grid = dim3(cus);
      }
    }
  }
  if (dtype == 0) e = launch_attn_bf16(lp, d_qk, grid, stream);
  else if (p.block64) e = d_qk == 128 ? launch_attn_fp8_block64_d128(lp, grid, stream)
                                      : launch_attn_fp8_block64_d192(lp, grid, stream);
  else e = d_qk == 128 ? launch_attn_fp8_head_d128(lp, grid, stream) : launch_attn_fp8_head_d192(lp, grid, stream);
  if (e != hipSuccess || p.split_tiles == 0) return e;
  const int nqt = (p.Nq + kBM - 1) / kBM;
  const long long mblocks = (long long)p.B * p.Hq * (nqt - first_qt) * (kBM / kMergeRows);
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)mblocks), dim3(256), 0, stream, p,
                     variant_tile_keys(p, dtype, d_qk), first_qt);
  return hipGetLastError();
}

}  // namespace miattn
