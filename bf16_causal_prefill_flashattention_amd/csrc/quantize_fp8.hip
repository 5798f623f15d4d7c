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

// One cross-lane butterfly stage of width DL lanes (DL in {1, 2, 4, 8}, within
// a 16-lane DPP row): lane l pairs with lane l ^ DL; the lower lane of the pair
// (bit DL clear) becomes a + b, the upper a - b, where a is the lower lane's
// value and b the upper's -- the same fp32 operations as the butterfly
// (b + a = a + b, and a + (-b) = a - b exactly).  DPP reads operands of other
// lanes inside the vector instruction, so no LDS round trip is needed.
//   DL = 4, 8: banks (groups of 4 lanes) are wholly lower or upper, so a
//   bank-masked add (lower banks, reading lane l + DL) and a bank-masked
//   subtract (upper banks, reading lane l - DL) write the two halves.
//   DL = 1, 2: lower and upper lanes share banks, so the upper lanes' own value
//   is negated first (sign-bit XOR, `sgn` = 0x80000000 on upper lanes) and one
//   quad-permuted add forms partner + own for all lanes.
// The s_nop 1 gives the two wait states a DPP read needs after the vector
// write of its source (the compiler does not see into the assembly).
template <int DL>
__device__ __forceinline__ void fwht_xlane(float v[8], uint32_t sgn) {
  float r[8];
  if constexpr (DL == 4 || DL == 8) {
#define MIATTN_BFLY(LO, HI)                                                     \
  "v_add_f32_dpp %" #LO ", %" #HI ", %" #HI " row_shl:" DLS " row_mask:0xf bank_mask:" LOB "\n\t" \
  "v_sub_f32_dpp %" #LO ", %" #HI ", %" #HI " row_shr:" DLS " row_mask:0xf bank_mask:" HIB "\n\t"
    if constexpr (DL == 4) {
#define DLS "4"
#define LOB "0x5"
#define HIB "0xa"
      asm("s_nop 1\n\t" MIATTN_BFLY(0, 8) MIATTN_BFLY(1, 9) MIATTN_BFLY(2, 10) MIATTN_BFLY(3, 11)
              MIATTN_BFLY(4, 12) MIATTN_BFLY(5, 13) MIATTN_BFLY(6, 14) MIATTN_BFLY(7, 15)
          : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
          : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
#undef DLS
#undef LOB
#undef HIB
    } else {
#define DLS "8"
#define LOB "0x3"
#define HIB "0xc"
      asm("s_nop 1\n\t" MIATTN_BFLY(0, 8) MIATTN_BFLY(1, 9) MIATTN_BFLY(2, 10) MIATTN_BFLY(3, 11)
              MIATTN_BFLY(4, 12) MIATTN_BFLY(5, 13) MIATTN_BFLY(6, 14) MIATTN_BFLY(7, 15)
          : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
          : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
#undef DLS
#undef LOB
#undef HIB
    }
#undef MIATTN_BFLY
  } else {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[i]) ^ sgn);
#define MIATTN_QADD(R, S, T) "v_add_f32_dpp %" #R ", %" #S ", %" #T " quad_perm:" QP " row_mask:0xf bank_mask:0xf\n\t"
#define MIATTN_QSTAGE                                                                                            \
  asm("s_nop 1\n\t" MIATTN_QADD(0, 8, 16) MIATTN_QADD(1, 9, 17) MIATTN_QADD(2, 10, 18) MIATTN_QADD(3, 11, 19)      \
          MIATTN_QADD(4, 12, 20) MIATTN_QADD(5, 13, 21) MIATTN_QADD(6, 14, 22) MIATTN_QADD(7, 15, 23)            \
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]) \
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(t[0]),    \
        "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(t[4]), "v"(t[5]), "v"(t[6]), "v"(t[7]))
    if constexpr (DL == 1) {
#define QP "[1,0,3,2]"
      MIATTN_QSTAGE;
#undef QP
    } else {
#define QP "[2,3,0,1]"
      MIATTN_QSTAGE;
#undef QP
    }
#undef MIATTN_QSTAGE
#undef MIATTN_QADD
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = r[i];
}

// Row layout of the quantizer kernels: TPR lanes per row; lane c (0..TPR-1)
// holds, for each i < NI, the 8 consecutive channels 8 (TPR i + c) .. +7 in
// v[i][0..7], so each of a row's NI loads reads contiguous bytes over its TPR
// lanes.  Without the rotation a lane holds one group (TPR = D / 8: a load
// instruction covers whole rows); with it, 4 lanes per row (NI = D / 32), so
// that all but two butterfly stages run inside a lane.
template <int D, bool HAD>
struct Row {
  static constexpr int TPR = HAD ? 4 : D / 8;  // lanes per row
  static constexpr int NI = D / (8 * TPR);     // 8-channel groups per lane
  static constexpr int RPP = kQThreads / TPR;  // rows per pass of a workgroup
  static __device__ __forceinline__ int ch(int c, int i) { return 8 * (TPR * i + c); }
};

// Butterfly stage of width 32 or 64 channels, inside a lane: groups i and
// i + G (G = 1 or 2, i with bit G clear) -> (a + b, a - b).
template <int NI, int G>
__device__ __forceinline__ void fwht_groups(float (&v)[NI][8]) {
  static_assert(NI % (2 * G) == 0, "groups pair up");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (!(i & G)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = v[i][j], b = v[i + G][j];
        v[i][j] = a + b;
        v[i + G][j] = a - b;
      }
    }
  }
}

// Unnormalised Walsh-Hadamard transform of each row (4 lanes per row): one
// H_128 at D = 128,
// H_64 on each of the three groups of 64 channels at D = 192, as butterfly
// stages of widths 1, 2, 4 (inside each 8-channel group), 8 and 16 (lane c
// with c ^ 1, c ^ 2), 32 (groups i, i ^ 1) and, at D = 128, 64 (groups i,
// i ^ 2).  With LAST = false the final stage is left out (see amax_kernel).
// sgn1 / sgn2: 0x80000000 on lanes whose bit 0 / bit 1 is set, else 0.
template <int D, bool LAST>
__device__ __forceinline__ void fwht_row(float (&v)[D / 32][8], uint32_t sgn1, uint32_t sgn2) {
  constexpr int NI = D / 32;
  static_assert(Row<D, true>::NI == NI, "4 lanes per row");
#pragma unroll
  for (int g = 0; g < NI; ++g) {
#pragma unroll
    for (int wd = 1; wd < 8; wd <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!(i & wd)) {
          const float a = v[g][i], b = v[g][i + wd];
          v[g][i] = a + b;
          v[g][i + wd] = a - b;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < NI; ++g) fwht_xlane<1>(v[g], sgn1);
#pragma unroll
  for (int g = 0; g < NI; ++g) fwht_xlane<2>(v[g], sgn2);
  if constexpr (D == 128) {
    fwht_groups<NI, 1>(v);
    if constexpr (LAST) fwht_groups<NI, 2>(v);
  } else {
    if constexpr (LAST) fwht_groups<NI, 1>(v);
  }
}

__global__ void amax_init_kernel(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// Grid: one workgroup per (b*H + h, chunk of kRowsPerBlock sequence rows).
// With the rotation the last butterfly stage is not formed: the larger
// magnitude of its two outputs, max(|a + b|, |a - b|), equals |a| + |b|, and
// in fp32 max(|fl(a + b)|, |fl(a - b)|) = fl(|a| + |b|) exactly (one of the two
// is +-(|a| + |b|) before rounding, the other no larger, and round-to-nearest
// is monotone and symmetric), so the amax is the same bits.
template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQThreads) void amax_kernel(const T* x, uint32_t* amax_bits, int N, int H,
                                                         int nchunks) {
  using L = Row<D, HAD>;
  constexpr int TPR = L::TPR, RPP = L::RPP, NI = L::NI;
  const int bh = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const uint32_t sgn1 = (tid & 1) ? 0x80000000u : 0u, sgn2 = (tid & 2) ? 0x80000000u : 0u;
  const bool active = rr < RPP;  // D = 192 without the rotation: 240 of the 256 lanes
  const int r0 = chunk * kRowsPerBlock;
  const int r1 = min(r0 + kRowsPerBlock, N);
  float m = 0.f;
  // Without the rotation, U = 4 passes per round with their loads issued
  // together: a lane with no row in a pass (past the block's end, or idle)
  // reads row r0 again instead of reading nothing -- a repeated row leaves the
  // max unchanged, and the loads then need no branch between them.  With the
  // rotation (four loads per pass already) a lane with no row loads nothing.
  constexpr int U = HAD ? 1 : 4;
  for (int base = r0; base < r1; base += U * RPP) {  // uniform trip count over the block
    float vu[U][NI][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + u * RPP + rr;
      const bool valid = active && r < r1;
      const T* row = x + (((size_t)b * N + (valid ? r : (HAD ? 0 : r0))) * H + h) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i) load8<T>(row + L::ch(cc, i), HAD ? valid : true, vu[u][i]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
    float (&v)[NI][8] = vu[u];
    if constexpr (HAD) {
      fwht_row<D, false>(v, sgn1, sgn2);
      constexpr int G = D == 128 ? 2 : 1;  // the last stage pairs groups i and i + G
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (!(i & G)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]) + fabsf(v[i + G][j]));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
    }
    }
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
  using L = Row<D, HAD>;
  constexpr int TPR = L::TPR, RPP = L::RPP, NI = L::NI;
  const int bh = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const uint32_t sgn1 = (tid & 1) ? 0x80000000u : 0u, sgn2 = (tid & 2) ? 0x80000000u : 0u;
  const bool active = rr < RPP;
  const float amax = __builtin_bit_cast(float, amax_bits[bh]);
  const float inv = amax == 0.f ? 1.f : 448.f / amax;
  const int r0 = chunk * kRowsPerBlock;
  const int r1 = min(r0 + kRowsPerBlock, N);
  if constexpr (HAD) {
    for (int base = r0; base < r1; base += RPP) {
      const int r = base + rr;
      const bool valid = active && r < r1;
      const size_t off = (((size_t)b * N + (valid ? r : 0)) * H + h) * D;
      float v[NI][8];
#pragma unroll
      for (int i = 0; i < NI; ++i) load8<T>(x + off + L::ch(cc, i), valid, v[i]);
      fwht_row<D, true>(v, sgn1, sgn2);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = fminf(fmaxf(v[i][j] * inv, -448.f), 448.f);
        if (valid) {
          i32x2 codes = {(int)pack_fp8x4(v[i][0], v[i][1], v[i][2], v[i][3]),
                         (int)pack_fp8x4(v[i][4], v[i][5], v[i][6], v[i][7])};
          *reinterpret_cast<i32x2*>(y + off + L::ch(cc, i)) = codes;
        }
      }
    }
  } else {
    // U = 4 passes per round: their loads issued together (a lane with no row
    // in a pass reads row r0 and stores nothing), then their conversions and
    // stores
    constexpr int U = 4;
    for (int base = r0; base < r1; base += U * RPP) {
      float vu[U][NI][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = base + u * RPP + rr;
        const size_t off = (((size_t)b * N + (active && r < r1 ? r : r0)) * H + h) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) load8<T>(x + off + L::ch(cc, i), true, vu[u][i]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = base + u * RPP + rr;
        const bool valid = active && r < r1;
        const size_t off = (((size_t)b * N + (valid ? r : r0)) * H + h) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
          for (int j = 0; j < 8; ++j) vu[u][i][j] = fminf(fmaxf(vu[u][i][j] * inv, -448.f), 448.f);
          if (valid) {
            i32x2 codes = {(int)pack_fp8x4(vu[u][i][0], vu[u][i][1], vu[u][i][2], vu[u][i][3]),
                           (int)pack_fp8x4(vu[u][i][4], vu[u][i][5], vu[u][i][6], vu[u][i][7])};
            *reinterpret_cast<i32x2*>(y + off + L::ch(cc, i)) = codes;
          }
        }
      }
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
// registers (PASSES passes of RPP rows), its amax reduced in the workgroup,
// then quantized and written.
template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQThreads) void quantize_block64_kernel(const T* x, uint8_t* y, float* scale, int N,
                                                                     int H, int nblk) {
  using L = Row<D, HAD>;
  constexpr int TPR = L::TPR, RPP = L::RPP, NI = L::NI;
  constexpr int PASSES = (64 + RPP - 1) / RPP;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, rr = tid / TPR, cc = tid % TPR;
  const uint32_t sgn1 = (tid & 1) ? 0x80000000u : 0u, sgn2 = (tid & 2) ? 0x80000000u : 0u;
  const int r0 = blk * 64, r1 = min(r0 + 64, N);
  float v[PASSES][NI][8];
  float m = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int r = r0 + ps * RPP + rr;
    const bool valid = rr < RPP && ps * RPP + rr < 64 && r < r1;
    const size_t off = (((size_t)b * N + (valid ? r : 0)) * H + h) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) load8<T>(x + off + L::ch(cc, i), valid, v[ps][i]);
    if constexpr (HAD) {
      fwht_row<D, true>(v[ps], sgn1, sgn2);
      const float norm = D == 128 ? kInvSqrt128 : 0.125f;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[ps][i][j] = v[ps][i][j] * norm;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[ps][i][j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
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
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = v[ps][i][j] * inv;  // exact: |w| <= 448
      if (valid) {
        i32x2 codes = {(int)pack_fp8x4(w[0], w[1], w[2], w[3]), (int)pack_fp8x4(w[4], w[5], w[6], w[7])};
        *reinterpret_cast<i32x2*>(y + (((size_t)b * N + r) * H + h) * D + L::ch(cc, i)) = codes;
      }
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
