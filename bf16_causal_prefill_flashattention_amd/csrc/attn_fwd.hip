// Launch of the causal forward attention: grid size and the choice of kernel
// variant (dtype, head dimensions, FP8 scale granularity and probability mode).
// The kernel template is in attn_fwd_impl.hpp; its variants are instantiated in
// attn_fwd_bf16.hip and attn_fwd_fp8_{head,block64}_d{128,192}.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "kernels.h"

namespace miattn {

namespace {
constexpr int kBM = 256;  // queries per work item (one workgroup of 8 waves x 32)
}  // namespace

long long attn_fwd_units(int B, int Hq, int Nq) {
  const long long nqt = (Nq + kBM - 1) / kBM;
  return (long long)B * Hq * ((nqt + 1) / 2);
}

long long attn_fwd_tiles(int B, int Hq, int Nq) {
  return (long long)B * Hq * ((Nq + kBM - 1) / kBM);
}

hipError_t launch_attn_fwd(const AttnParams& p, int dtype, int d_qk, int d_v, hipStream_t stream) {
  if (p.Nq < 1 || p.Nk < p.Nq) return hipErrorInvalidValue;
  if (d_v != 128 || (d_qk != 128 && d_qk != 192)) return hipErrorInvalidValue;
  if (p.p_mode < kPLean || p.p_mode > kPExactTile) return hipErrorInvalidValue;
  if (dtype == 0 && (p.block64 || p.p_mode != kPLean)) return hipErrorInvalidValue;
  if (p.block64 && p.Nk > kBlock64MaxKeys) return hipErrorInvalidValue;
  const long long units = attn_fwd_units(p.B, p.Hq, p.Nq);
  if (units <= 0 || units > 0x7fffffffLL) return hipErrorInvalidValue;
  // CU count per device, filled on first use (atomic: concurrent callers may
  // both fill it, with the same value)
  static std::atomic<int> cu_count[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int cus = cu_count[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 1;
    cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  const long long tiles = attn_fwd_tiles(p.B, p.Hq, p.Nq);
  // as many workgroups as CUs, or one per tile when the tiles do not fill the
  // CUs (the kernel derives the same choice from gridDim)
  const dim3 grid(tiles <= cus ? (int)tiles : (int)std::min<long long>(units, cus));
  if (dtype == 0) return launch_attn_bf16(p, d_qk, grid, stream);
  if (p.block64) return d_qk == 128 ? launch_attn_fp8_block64_d128(p, grid, stream)
                                    : launch_attn_fp8_block64_d192(p, grid, stream);
  return d_qk == 128 ? launch_attn_fp8_head_d128(p, grid, stream) : launch_attn_fp8_head_d192(p, grid, stream);
}

}  // namespace miattn
