// Device-side helpers shared by the gfx950 (CDNA4) kernels of miattn.
//
// Vector types for the MFMA operands, thin wrappers around the matrix-core
// builtins, LDS/global vector accesses and byte/half-word transposes.  Only
// gfx950 is targeted; nothing here has a second code path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Note on bit casts: with this toolchain, __builtin_bit_cast applied to an
// element of an ext_vector_type value (bit_cast<float>(v[i])) has been seen to
// fold every element to v[0].  Bit-cast whole vectors, or copy the element to a
// scalar first.

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Lane l supplies A row (l % 32) and B column (l % 32), 8 consecutive k-slots
// each; the k-slots of a lane are the same for A and B.  D: lane l holds column
// (l % 32), rows 8*i + 4*(l / 32) + j in register 4*i + j.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 fp32) += A(32x64 e4m3) * B(64x32 e4m3), unit block scales
// (E8M0 127 = 2^0).  Lane l supplies 32 k-slots of A row / B column (l % 32);
// same D layout as above.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// As mfma_fp8_32x32x64 with the A operand scaled by 2^(E - 127), E = byte SEL
// of scale_a (an E8M0 exponent).  Each lane's byte scales the 32 k-slots of A
// it supplies; with the same word in every lane the whole A block gets one
// power-of-two scale, applied exactly inside the instruction.
template <int SEL>
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64_sa(i32x8 a, i32x8 b, f32x16 c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, scale_a, 0, 127);
}

// As mfma_fp8_32x32x64 with A scaled by byte SELA of scale_a and B by byte SELB
// of scale_b (E8M0 exponents).  B's scale is per lane: lane l's byte scales the
// 32 k-slots of column l % 32 it supplies.
template <int SELA, int SELB>
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64_sab(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SELA, scale_a, SELB, scale_b);
}

// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3), unit block scales.  Lane l
// supplies 32 k-slots of A row / B column (l % 16); lane group l / 16 selects
// which quarter of the 128 k-slots.  D: lane l holds column (l % 16), rows
// 4*(l / 16) + j in register j.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// As mfma_fp8_16x16x128 with B scaled per lane by byte SELB of scale_b (E8M0):
// lane l's byte scales the 32 k-slots it supplies.
template <int SELB>
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128_sb(i32x8 a, i32x8 b, f32x4 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, SELB, scale_b);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies 8 k-slots of
// A row / B column (l % 16); lane group l / 16 selects which quarter of the 32
// k-slots.  D: lane l holds column (l % 16), rows 4*(l / 16) + j in register j.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 16-byte global load that yields zeros when `valid` is false (no access).
__device__ __forceinline__ i32x4 gload16(const void* p, bool valid) {
  i32x4 r = {0, 0, 0, 0};
  if (valid) r = *reinterpret_cast<const i32x4*>(p);
  return r;
}

// Raw buffer resource over [base, base + bytes): 16-byte loads whose offset is
// at or beyond `bytes` return zeros without touching memory, so ragged tiles
// need no branches.  Offsets are 32-bit, so callers rebase per tile.
// The base and size must be wave-uniform; readfirstlane states that to the
// compiler (a descriptor it believes divergent is built in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, 0);
}

__device__ __forceinline__ i32x4 lds_load16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ void lds_store16(void* p, i32x4 v) {
  *reinterpret_cast<i32x4*>(p) = v;
}
__device__ __forceinline__ void lds_store8(void* p, i32x2 v) {
  *reinterpret_cast<i32x2*>(p) = v;
}
__device__ __forceinline__ void lds_store4(void* p, int v) {
  *reinterpret_cast<int*>(p) = v;
}

// Byte permute: result byte i = byte sel.byte[i] of the 8-byte value {hi:lo}
// (selectors 0-3 pick from lo, 4-7 from hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round two fp32 to bf16 (nearest-even) and pack them, first value low: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Round four fp32 to OCP e4m3 (hardware conversion, nearest-even) and pack
// them, first value in the low byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  // the first conversion writes the low half only; start from an undefined
  // register (the high half is overwritten next) instead of materialising 0
  int w;
  asm("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Swap with the lane 32 positions away (lane l <-> lane l ^ 32).
__device__ __forceinline__ float xor32(float v) {
  return __shfl_xor(v, 32, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace miattn
