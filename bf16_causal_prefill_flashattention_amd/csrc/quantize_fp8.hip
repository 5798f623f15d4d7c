// FP8 e4m3 front end for gfx950: per-(batch, head) amax/448 scaling, or
// per-(batch, head, 64 positions) power-of-two scaling, with an optional
// Hadamard rotation of the head dimension.
//
// Page legend: [P1] "Zyphra ZYFA: 1.76x FP8 FlashAttention Speedup on AMD
// MI355X"; [P2] "Zyphra Says Its AMD MI355X Attention Kernel Is 1.76x Faster";
// [P3] "Zyphra 开源 ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速 1.76 倍".
//
// FP8 attention needs per-tensor or per-head scale factors to bring values
// into the e4m3 range ([P1] "ZYFA's performance and accuracy data"); here one
// fp32 scale per (batch, head) equals amax/448.  Rotating Q and K by a
// Hadamard matrix first roughly halves the input-quantization error ([P3]
// "ZYFA 的 FP8 注意力有多准确？", [P2] "Accuracy and Code"); the rotation used is
// the Sylvester H_128 at head dimension 128 and three Sylvester H_64 blocks at
// 192 (the pages show the rotation at 128 only), unnormalised in the values,
// with the normalisation (2^-3.5 or 2^-3) folded into the stored scale.
//
// Finer granularity ([P1] "ZYFA's performance and accuracy data" names scaling
// granularity as a lever on accuracy): one power-of-two scale 2^e per 64
// positions of a (batch, head), e the smallest integer with amax <= 448 * 2^e
// (at least -126), codes = e4m3(z * 2^-e) with no clamp needed.  Powers of two
// are what the scaled matrix instructions apply to K and V for free.  With the
// rotation, z = fp32(x H * norm) carries the normalisation in the values.
//
// The codes are integers decided by fp32 arithmetic, so every rounding step
// is pinned: the transform is the radix-2 butterfly with stage widths 1, 2,
// ..., 64, each butterfly (a, b) -> (a + b, a - b) in fp32; then
// inv = 448 / amax and y = x * inv (each correctly rounded), a clamp to
// [-448, 448] and the hardware round-to-nearest-even conversion to e4m3.
//
// HBM-bound: the amax pass reads x once, the quantize pass reads x again and
// writes one byte per element.  Passes run in stream order:
//   init (amax <- 0) -> amax (atomic max of the fp32 bit patterns, which order
//   non-negative floats like integers; max is order-free, so the result is
//   deterministic) -> quantize -> finalize (amax -> scale, in place).
#include "device_common.hpp"
#include "kernels.h"

namespace miattn {

namespace {

constexpr int kQThreads = 256;
constexpr int kRowsPerBlock = 256;
constexpr float kInvSqrt128 = 0.08838834764831845f;  // fp32(2^-3.5)

template <typename T>
__device__ __forceinline__ void load8(const T* src, bool valid, float v[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* src, bool valid, float v[8]) {
  // whole-vector bit casts only (see the note on bit casts in device_common.hpp)
  const f32x4 a = __builtin_bit_cast(f32x4, gload16(src, valid));
  const f32x4 b = __builtin_bit_cast(f32x4, gload16(src + 4, valid));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* src, bool valid, float v[8]) {
  i32x4 a = gload16(src, valid);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = static_cast<uint32_t>(static_cast<int>(a[i]));
    v[2 * i] = __builtin_bit_cast(float, w << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
}

// Unnormalised NPT-point Walsh-Hadamard transform of each group of NPT
// channels of a row held by consecutive lanes, 8 consecutive channels per lane
// (lane cc holds channels 8cc .. 8cc+7; a group is NPT/8 lanes, aligned in the
// wave).  Stage widths 1, 2, 4 are inside a lane; widths 8..NPT/2 pair lane cc
// with lane cc ^ (width / 8).
template <int NPT>
__device__ __forceinline__ void fwht_row(float v[8], int cc) {
#pragma unroll
  for (int wd = 1; wd < 8; wd <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & wd)) {
        const float a = v[i], b = v[i + wd];
        v[i] = a + b;
        v[i + wd] = a - b;
      }
    }
  }
#pragma unroll
  for (int dl = 1; dl < NPT / 8; dl <<= 1) {
    const bool upper = (cc & dl) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float o = __shfl_xor(v[i], dl, kWave);
      v[i] = upper ? (o - v[i]) : (v[i] + o);
    }
  }
}

__global__ void amax_init_kernel(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// Grid: one workgroup per (b*H + h, chunk of kRowsPerBlock sequence rows).
template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQThreads) void amax_kernel(const T* x, uint32_t* amax_bits, int N, int H,
                                                         int nchunks) {
  constexpr int TPR = D / 8;              // threads per row
  constexpr int RPP = kQThreads / TPR;    // rows per pass
  const int bh = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const bool active = rr < RPP;
  const int r0 = chunk * kRowsPerBlock;
  const int r1 = min(r0 + kRowsPerBlock, N);
  float m = 0.f;
  for (int base = r0; base < r1; base += RPP) {  // uniform trip count over the block
    const int r = base + rr;
    const bool valid = active && r < r1;
    float v[8];
    load8<T>(x + (((size_t)b * N + (valid ? r : 0)) * H + h) * D + cc * 8, valid, v);
    if constexpr (HAD) fwht_row<(D == 128 ? 128 : 64)>(v, cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  __shared__ float wmax[kQThreads / kWave];
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float mm = wmax[0];
#pragma unroll
    for (int i = 1; i < kQThreads / kWave; ++i) mm = fmaxf(mm, wmax[i]);
    atomicMax(amax_bits + bh, __builtin_bit_cast(uint32_t, mm));
  }
}

template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const T* x, uint8_t* y, const uint32_t* amax_bits,
                                                             int N, int H, int nchunks) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kQThreads / TPR;
  const int bh = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const bool active = rr < RPP;
  const float amax = __builtin_bit_cast(float, amax_bits[bh]);
  const float inv = amax == 0.f ? 1.f : 448.f / amax;
  const int r0 = chunk * kRowsPerBlock;
  const int r1 = min(r0 + kRowsPerBlock, N);
  for (int base = r0; base < r1; base += RPP) {
    const int r = base + rr;
    const bool valid = active && r < r1;
    const size_t off = (((size_t)b * N + (valid ? r : 0)) * H + h) * D + cc * 8;
    float v[8];
    load8<T>(x + off, valid, v);
    if constexpr (HAD) fwht_row<(D == 128 ? 128 : 64)>(v, cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i] * inv, -448.f), 448.f);
    if (valid) {
      i32x2 codes = {(int)pack_fp8x4(v[0], v[1], v[2], v[3]), (int)pack_fp8x4(v[4], v[5], v[6], v[7])};
      *reinterpret_cast<i32x2*>(y + off) = codes;
    }
  }
}

__global__ void finalize_scale_kernel(float* scale, int n, float norm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float amax = scale[i];  // holds the amax bit pattern written by the passes above
    float s = amax == 0.f ? 1.f : amax / 448.f;
    if (norm != 1.f) s = s * norm;
    scale[i] = s;
  }
}

// Exponent e of the power-of-two block scale: the smallest integer with
// amax <= 448 * 2^e = 1.75 * 2^(e+8), at least -126; 0 for amax == 0.  With
// amax = 1.m * 2^k that is k - 8, plus one when the significand exceeds 1.75.
__device__ __forceinline__ int block_exponent(float amax) {
  const uint32_t a = __builtin_bit_cast(uint32_t, amax);
  if (a == 0u) return 0;
  const int ef = (int)(a >> 23);
  if (ef == 0) return -126;  // subnormal amax: far below the clamp
  const int e = ef - 127 - 8 + ((a & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : e;
}

// One workgroup per (b*H + h, 64-position block): the block is read once into
// registers, its amax reduced in the workgroup, then quantized and written.
template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQThreads) void quantize_block64_kernel(const T* x, uint8_t* y, float* scale, int N,
                                                                     int H, int nblk) {
  constexpr int TPR = D / 8;                      // threads per row
  constexpr int RPP = kQThreads / TPR;            // rows per pass
  constexpr int PASSES = (64 + RPP - 1) / RPP;    // passes over the 64 rows
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const int r0 = blk * 64, r1 = min(r0 + 64, N);
  float v[PASSES][8];
  float m = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int r = r0 + ps * RPP + rr;
    const bool valid = rr < RPP && ps * RPP + rr < 64 && r < r1;
    load8<T>(x + (((size_t)b * N + (valid ? r : 0)) * H + h) * D + cc * 8, valid, v[ps]);
    if constexpr (HAD) {
      fwht_row<(D == 128 ? 128 : 64)>(v[ps], cc);
      const float norm = D == 128 ? kInvSqrt128 : 0.125f;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[ps][i] = v[ps][i] * norm;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[ps][i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  __shared__ float wmax[kQThreads / kWave];
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  float amax = wmax[0];
#pragma unroll
  for (int i = 1; i < kQThreads / kWave; ++i) amax = fmaxf(amax, wmax[i]);
  const int e = block_exponent(amax);
  // 2^-e is a normal fp32 number: e lies in [-126, 121]
  const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
  if (tid == 0) scale[(size_t)bh * nblk + blk] = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int r = r0 + ps * RPP + rr;
    const bool valid = rr < RPP && ps * RPP + rr < 64 && r < r1;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[ps][i] * inv;  // exact: |w| <= 448
    if (valid) {
      i32x2 codes = {(int)pack_fp8x4(w[0], w[1], w[2], w[3]), (int)pack_fp8x4(w[4], w[5], w[6], w[7])};
      *reinterpret_cast<i32x2*>(y + (((size_t)b * N + r) * H + h) * D + cc * 8) = codes;
    }
  }
}

template <typename T, int D, bool HAD>
void launch_passes(const void* x, void* y, float* scale, int B, int H, int N, hipStream_t stream) {
  const int nchunks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  const int grid = B * H * nchunks;
  if (grid == 0) return;
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(scale);
  hipLaunchKernelGGL((amax_kernel<T, D, HAD>), dim3(grid), dim3(kQThreads), 0, stream, static_cast<const T*>(x),
                     amax_bits, N, H, nchunks);
  hipLaunchKernelGGL((quantize_kernel<T, D, HAD>), dim3(grid), dim3(kQThreads), 0, stream,
                     static_cast<const T*>(x), static_cast<uint8_t*>(y), amax_bits, N, H, nchunks);
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N,
                               int d, bool hadamard, hipStream_t stream) {
  const int n = B * H;
  if (n == 0) return hipSuccess;
  const int small = (n + 255) / 256;
  hipLaunchKernelGGL(amax_init_kernel, dim3(small), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(scale), n);
  if (x_dtype == 0) {
    if (d == 128 && hadamard) launch_passes<float, 128, true>(x, x_fp8, scale, B, H, N, stream);
    else if (d == 128) launch_passes<float, 128, false>(x, x_fp8, scale, B, H, N, stream);
    else if (hadamard) launch_passes<float, 192, true>(x, x_fp8, scale, B, H, N, stream);
    else launch_passes<float, 192, false>(x, x_fp8, scale, B, H, N, stream);
  } else {
    if (d == 128 && hadamard) launch_passes<__bf16, 128, true>(x, x_fp8, scale, B, H, N, stream);
    else if (d == 128) launch_passes<__bf16, 128, false>(x, x_fp8, scale, B, H, N, stream);
    else if (hadamard) launch_passes<__bf16, 192, true>(x, x_fp8, scale, B, H, N, stream);
    else launch_passes<__bf16, 192, false>(x, x_fp8, scale, B, H, N, stream);
  }
  const float norm = !hadamard ? 1.f : (d == 128 ? kInvSqrt128 : 0.125f);
  hipLaunchKernelGGL(finalize_scale_kernel, dim3(small), dim3(256), 0, stream, scale, n, norm);
  return hipGetLastError();
}

namespace {
template <typename T, int D, bool HAD>
void launch_block64(const void* x, void* y, float* scale, int B, int H, int N, hipStream_t stream) {
  const int nblk = (N + 63) / 64;
  const long long grid = (long long)B * H * nblk;
  if (grid == 0) return;
  hipLaunchKernelGGL((quantize_block64_kernel<T, D, HAD>), dim3((unsigned)grid), dim3(kQThreads), 0, stream,
                     static_cast<const T*>(x), static_cast<uint8_t*>(y), scale, N, H, nblk);
}
}  // namespace

hipError_t launch_quantize_fp8_block64(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N,
                                       int d, bool hadamard, hipStream_t stream) {
  if (x_dtype == 0) {
    if (d == 128) {
      if (hadamard) launch_block64<float, 128, true>(x, x_fp8, scale, B, H, N, stream);
      else launch_block64<float, 128, false>(x, x_fp8, scale, B, H, N, stream);
    } else {
      if (hadamard) launch_block64<float, 192, true>(x, x_fp8, scale, B, H, N, stream);
      else launch_block64<float, 192, false>(x, x_fp8, scale, B, H, N, stream);
    }
  } else {
    if (d == 128) {
      if (hadamard) launch_block64<__bf16, 128, true>(x, x_fp8, scale, B, H, N, stream);
      else launch_block64<__bf16, 128, false>(x, x_fp8, scale, B, H, N, stream);
    } else {
      if (hadamard) launch_block64<__bf16, 192, true>(x, x_fp8, scale, B, H, N, stream);
      else launch_block64<__bf16, 192, false>(x, x_fp8, scale, B, H, N, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace miattn
