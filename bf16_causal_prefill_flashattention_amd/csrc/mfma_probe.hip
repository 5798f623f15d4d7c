// Matrix-core throughput under the board power limit: back-to-back MFMAs and
// nothing else, for bench.py --mfma-probe (a measurement aid built into
// libmiattn_probe.so; the attention path does not use it).
//
// Every wave holds NSETS operand sets for A and B, loaded once from a buffer
// the caller fills (e.g. with the attention inputs' value distribution), and
// issues iters x 4 MFMAs into 4 independent accumulators, stepping to another
// A and B set at every MFMA so the inputs switch the way a real product's do
// (power depends on the operand bits).  With two waves per SIMD the matrix pipe
// stays busy; the clock the power limit then allows, times the MFMA rate, is
// the ceiling an attention kernel on such data cannot exceed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace {

using namespace miattn;

constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr int kSets = 4;       // operand sets per wave for each of A and B

template <bool FP8>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(const int* operands, float* out, int iters) {
  constexpr int W = FP8 ? 8 : 4;  // 32-bit words per lane of one operand
  const int tid = threadIdx.x;
  // operand words of this thread: 2 * kSets * W consecutive ints
  const int* src = operands + (size_t)(blockIdx.x * kThreads + tid) * (2 * kSets * W);
  int a[kSets][W], b[kSets][W];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int w = 0; w < W; ++w) {
      a[s][w] = src[s * W + w];
      b[s][w] = src[(kSets + s) * W + w];
    }
  f32x16 acc[4] = {zero16(), zero16(), zero16(), zero16()};
  for (int it = 0; it < iters; it += kSets) {  // (iters: a multiple of kSets)
#pragma unroll
    for (int c = 0; c < 4 * kSets; ++c) {
      // a new pair at every MFMA (indices known at compile time: no selects)
      const int sa = c & (kSets - 1), sb = (c / kSets + 3 * c) & (kSets - 1);
      if constexpr (FP8) {
        const i32x8 av = {a[sa][0], a[sa][1], a[sa][2], a[sa][3], a[sa][4], a[sa][5], a[sa][6], a[sa][7]};
        const i32x8 bv = {b[sb][0], b[sb][1], b[sb][2], b[sb][3], b[sb][4], b[sb][5], b[sb][6], b[sb][7]};
        acc[c & 3] = mfma_fp8_32x32x64(av, bv, acc[c & 3]);
      } else {
        const i32x4 av = {a[sa][0], a[sa][1], a[sa][2], a[sa][3]};
        const i32x4 bv = {b[sb][0], b[sb][1], b[sb][2], b[sb][3]};
        acc[c & 3] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc[c & 3]);
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  out[blockIdx.x * kThreads + tid] = sum;
}

}  // namespace

extern "C" {

// Threads per workgroup and operand ints per thread of mfma_probe_run.
int mfma_probe_threads(void) { return kThreads; }
int mfma_probe_words(int fp8) { return 2 * kSets * (fp8 ? 8 : 4); }

// `blocks` workgroups; each thread reads mfma_probe_words(fp8) ints of
// `operands` (bf16 pairs, or e4m3 quadruples, as raw bits) and writes one
// float of out; every wave issues 4 * iters MFMAs (bf16 32x32x16, or fp8
// 32x32x64; iters a positive multiple of 4).  Returns 0, -1 for invalid
// sizes, -5 when the launch failed.
int mfma_probe_run(int fp8, int blocks, int iters, const int* operands, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || iters % kSets != 0 || !operands || !out || (fp8 != 0 && fp8 != 1)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL((mfma_probe_kernel<true>), dim3(blocks), dim3(kThreads), 0, s, operands, out, iters);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<false>), dim3(blocks), dim3(kThreads), 0, s, operands, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
