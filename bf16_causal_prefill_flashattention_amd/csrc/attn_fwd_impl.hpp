// Kernel template of the causal forward attention (included by the
// translation units that instantiate its variants).
#pragma once

// Causal forward (prefill) attention for gfx950: O = softmax(Q K^T tau + mask) V.
//
// Page legend: [P1] "Zyphra ZYFA: 1.76x FP8 FlashAttention Speedup on AMD
// MI355X"; [P3] "Zyphra 开源 ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速
// 1.76 倍".
//
// What is computed: exact causal softmax attention, evaluated tile by tile with
// an online softmax so the N x N score matrix never reaches HBM ([P1] "Why
// prefill attention deserves dedicated optimization").  FP8 e4m3 inputs carry
// per-(batch, head) fp32 scales folded in before the softmax; both matrix
// products accumulate in FP32 ([P1] "ZYFA's performance and accuracy data";
// [P3] "为什么 FP8 注意力在 MI355X 上表现不佳？").  Output is BF16.
//
// Queries may be the last Nq positions of a longer key sequence (Nq <= Nk: one
// chunk of a chunked prefill against the keys and values before it); query row
// i then sits at position i + Nk - Nq.  Optionally the natural-log sum of exp
// of each query's scaled scores (LSE) is written, which is what combining the
// results of separate key ranges needs.
//
// Work decomposition.  One workgroup = 8 waves = 256 consecutive queries of one
// (batch, query head); each wave owns 32 queries.  Key tiles hold 192 keys (FP8
// at d_qk = 128 with per-head scales and no per-64-key shift, launches of more
// than 4096 keys), 128 (the other FP8 variants and launches, and BF16 at
// d_qk = 128) or 64 (BF16, d_qk = 192); a wave skips
// the tiles wholly above its queries and masks only the tiles that cross its
// diagonal.  A split launch gives each workgroup one range of a query tile's
// key tiles instead (the kernel's SPLIT instantiation): ranges of a query tile
// with more than one write normalised fp32 rows and their log2 sum of exp, and
// a merge kernel combines them.  Short launches that leave CUs idle may run
// 4-wave workgroups over 128 queries instead (NW = 4, one wave per SIMD doing
// the matrix and the vector work of each step; kSoloQueryTile).
//
// Matrix layout.  A wave computes S^T = K_tile * Q^T (keys on MFMA rows,
// queries on MFMA columns), so lane l owns query (l % 32) and holds half of the
// tile's scores for it; the other half sits in lane l ^ 32.  The output is
// accumulated transposed, O^T += V^T * P^T: the probabilities leave the S^T
// accumulator straight into the MFMA B operand, in an order of keys that the
// V^T operand reproduces when it is read from LDS.
//
// Two-group ping-pong.  A tile's softmax depends on that tile's S = K Q^T
// MFMAs, and its P.V product on the softmax, so within one wave the two kinds
// of work of a tile follow each other.  (Independent vector instructions do
// issue while the wave's own MFMAs execute: on gfx950, 128 independent FMAs
// interleaved with 16 FP8 32x32x64 MFMAs took the MFMAs' 980 cycles.)  Here the
// 8 waves form two groups (waves 0-3 and 4-7, one wave of each per SIMD) that
// run the same loop one phase apart, separated by workgroup barriers, so one
// wave's softmax runs beside the other's matrix work:
//   phase 2p   : group A matrix work  | group B vector work
//   phase 2p+1 : group A vector work  | group B matrix work
// where "matrix work" of step p is P_{p-1} V_{p-1} followed by S_p = K_p Q^T,
// and "vector work" of step p is the online softmax of S_p.  This is the
// two-wave overlap the pages describe ([P3] "ZYFA 如何工作？"), ordered here by
// barriers instead of per-instruction scheduling.
//
// Data movement.  K and V tiles go from HBM/L2 straight into LDS with buffer
// loads that write LDS (no register staging).  K and V rows are stored with an
// XOR swizzle of their 16-byte chunks so that the rows one operand read
// touches fall in distinct LDS banks; the V^T operand is read with the
// transposing LDS reads of gfx950.  Two LDS buffers each for K and V; the loads
// of step p (issued in phase 2p, or early in phase 2p+1) are waited for at the
// end of phase 2p+1.  Rows at or beyond Nq
// (queries) or Nk (keys), and whole tiles past the last one a workgroup needs,
// load as zeros (buffer bounds), so ragged tiles and the loads of the final
// steps need no branches; keys >= Nk lie above the diagonal of every valid
// query and are masked.  At the end of a work item each wave stages its output
// rows in LDS and stores them from there, four whole rows per instruction.
//
// FP8 scale granularity.  Either one fp32 scale per (batch, head) for each of
// Q, K, V, folded into the score multiplier and the output, or one scale per
// 64 positions: Q's per-wave block scale (a wave's 32 queries lie in one block)
// goes into the score multiplier, and the power-of-two K and V block scales are
// applied by the scaled MFMAs as E8M0 exponents (a 32-key QK block and a 64-key
// P.V k-step each lie in one 64-key block), at no vector cost.  The exponents of
// a work item's key tiles are staged in LDS, one word per 128-key tile.
//
// FP8 probabilities.  Lean P writes the e4m3 code of 2^x straight from one FMA
// on the log2-domain score x; the exact mode uses exp2 and the hardware
// conversion ([P3] "ZYFA 如何工作？" weighs the two).  Both multiply the
// probabilities by a fixed 2^6 first.  Lean codes reach about 13 octaves below
// that (the exact conversion's subnormals about 2.5 further), so key blocks
// whose scores lie far below the running max would round to zero; a shift
// keeps them: each query's probabilities of a key tile (tile mode, the
// default) or of a 64-key P.V step (block mode, the pages' per-64-key
// power-of-two scaling of P undone by the scaled MFMA) are shifted up by k
// octaves, k = floor(running max - their max), and the P.V MFMA scales them
// back by the E8M0 exponent 2^-k.  The scaled MFMAs read the exponent of a
// 32-key block of column j from lane j + 32 b, while each lane holds half of
// both blocks of its k-step, so both lanes of a query use one exponent (the
// pair's max).  The row sum of a shifted step: block mode sums it in a
// 32x32x64 MFMA against an all-ones A with the same exponents; tile mode sums
// the step's codes on their own and scales the sum back on the vector side.
//
// Probabilities.  The running max is only raised when a tile's max exceeds it
// by more than a small threshold, so most tiles skip the rescale of the output
// accumulator.  The row sum is taken from the rounded probabilities that feed
// the P.V product ([P3] "ZYFA 如何工作？", rounded row sums), with one extra
// small MFMA per P.V k-step against a 0/1 selector matrix (16x16x128 for FP8,
// 16x16x32 for BF16).  It runs on the matrix core with the other MFMAs of the
// wave: the vector-side dot-product instructions share the matrix pipeline and
// stall behind the other wave's MFMAs.  FP8 probabilities are scaled by a fixed
// power of two before rounding to e4m3, which the row sum cancels.
#include "device_common.hpp"
#include "kernels.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace miattn {

namespace {

constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kWaves = kThreads / kWave;
constexpr int kBM = kQueryTile;  // queries per workgroup (8 waves x 32)

// Keys per tile.  A phase carries a roughly fixed cost (barriers, the first
// operand reads), so larger tiles amortise it.  FP8 at d = 128 streams
// 192-key tiles, with one scale per head or per 64 positions (128 in launches
// of at most kShortKeys keys, whose last query tiles would waste more of a
// final 192-key tile); 128 where the per-64-key probability shift (its four
// max chains) assumes it, and at d = 192 (192-byte K rows do not split 192
// keys into whole 1 KB load blocks per wave).  BF16 at d = 128 streams 128
// keys (its two 32 KB buffers of K and of V fill 128 KB of LDS, and 192 would
// not fit it); BF16 at d = 192 stays at 64 (its 384-byte K rows would not
// split into whole blocks at 96, and 128 would take all 160 KB).  SHORT:
// the variant for launches of at most kShortKeys keys (128-key tiles where the
// tiles would otherwise hold 192).
template <bool FP8, int DQK, bool BS, int PSH, bool SHORT = false>
constexpr int tile_keys() {
  return tile_keys_of(FP8, DQK, BS, PSH == 1, SHORT);
}

template <bool FP8, int DQK, int DV, int BN_, int NW = 8>
struct Cfg {
  static constexpr int EB = FP8 ? 1 : 2;     // bytes per element
  static constexpr int BN = BN_;             // keys per tile
  static constexpr int NBLK = BN / 32;       // 32-key MFMA blocks per tile
  static constexpr int KROW = DQK * EB;      // bytes of one K row
  static constexpr int VROW = DV * EB;       // bytes of one V row
  static constexpr int KCH = KROW / 16;      // 16-byte chunks per K row
  static constexpr int VCH = VROW / 16;      // 16-byte chunks per V row
  // K rows are stored unpadded with their 16-byte chunks XOR-swizzled inside
  // groups of KG chunks (k_swizzle), V rows likewise (v_swizzle)
  static constexpr int KG = KCH % 16 == 0 ? 16 : (KCH % 8 == 0 ? 8 : 4);
  static constexpr int K_TILE = BN * KROW;
  static constexpr int V_TILE = BN * VROW;
  static constexpr int K_BLOCKS = BN * KCH / 64;  // 1 KB LDS-load blocks per K tile
  static constexpr int V_BLOCKS = BN * VCH / 64;
  static constexpr int K_PER_WAVE = K_BLOCKS / NW;
  static constexpr int V_PER_WAVE = V_BLOCKS / NW;
  // A wave's consecutive 1 KB load blocks lie kWaves blocks apart.  Where that
  // is a whole number of rows and a multiple of the swizzle period (16 rows),
  // every block of a wave has the same in-tile offset pattern, so one per-lane
  // offset serves all of them and the buffer descriptor moves instead
  // (K: FP8 and BF16 at d = 128; V: always).
  static constexpr int K_ROWS_STEP = (NW * 64) % KCH == 0 ? NW * 64 / KCH : 0;
  static constexpr int V_ROWS_STEP = (NW * 64) % VCH == 0 ? NW * 64 / VCH : 0;
  static constexpr bool K_UNI = K_ROWS_STEP > 0 && K_ROWS_STEP % 16 == 0;
  static constexpr bool V_UNI = V_ROWS_STEP > 0 && V_ROWS_STEP % 16 == 0;
  static constexpr int QK_STEPS = FP8 ? DQK / 64 : DQK / 16;
  static constexpr int LDS_BYTES = 2 * V_TILE + 2 * K_TILE;
  // log2-domain growth of the running max tolerated before rescaling, and the
  // power-of-two shift applied to FP8 probabilities: p <= 2^(THRESH + SHIFT),
  // whose lean-P code round(8 (THRESH + SHIFT) + C0) = 126 is e4m3's largest
  // finite value (448) for THRESH + SHIFT < 8.855
  static constexpr float THRESH = FP8 ? 2.75f : 8.0f;
  static constexpr float SHIFT = FP8 ? 6.0f : 0.0f;
  static_assert(K_BLOCKS % NW == 0 && V_BLOCKS % NW == 0, "tiles split into whole 1 KB blocks per wave");
  static_assert(2 * K_TILE <= 65536 && 2 * V_TILE <= 65536, "LDS offsets of a buffer pair fit the 16-bit immediate");
};

// XOR applied to the 16-byte chunk index of V row `key` in LDS.  It spreads the
// rows that one transposing read touches over distinct banks: FP8 reads 8 keys
// {0-3, 8-11} + base per lane group (key bits 1 and 3 vary), BF16 reads 4
// consecutive keys (bits 0 and 1 vary).
template <bool FP8>
__device__ __forceinline__ int v_swizzle(int key) {
  if constexpr (FP8)
    return (((key >> 1) & 1) << 1) | (((key >> 3) & 1) << 2);
  else
    return (key & 3) << 2;
}

// XOR applied inside a group of KG 16-byte chunks of K row `row` in LDS.  The
// 16 lanes that one quarter of a 16-byte operand read serves (rows r..r+15, one
// chunk) then fall in 16 distinct groups of four banks: 128-byte rows (FP8,
// d=128) alternate two 8-chunk bank halves, so the swizzle takes rows in
// pairs; 256-byte rows (BF16) start in the same bank, so every row gets its
// own; 192-byte rows (FP8 MLA) cycle four 4-chunk groups; 384-byte rows (BF16
// MLA) alternate halves like 128-byte ones.
template <class C>
__device__ __forceinline__ int k_swizzle(int row) {
  if constexpr (C::KROW == 256)
    return row & 15;
  else if constexpr (C::KROW == 192)
    return (row >> 2) & 3;
  else
    return (row >> 1) & 7;
}
// LDS position (chunk index within the row) of logical chunk `ch` of K row `row`
// (an involution: it also maps a position back to its logical chunk)
template <class C>
__device__ __forceinline__ int k_chunk_pos(int row, int ch) {
  return (ch & ~(C::KG - 1)) | ((ch ^ k_swizzle<C>(row)) & (C::KG - 1));
}

typedef __attribute__((address_space(3))) void lds_void;

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, I1).
template <int I0, int I1, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

// Buffer load of 16 bytes per lane written straight to LDS: lane i's bytes land
// at lds_block + 16 i (lds_block is wave-uniform).  Offsets at or beyond the
// buffer size load zeros.
//
// Issued as inline assembly: the compiler then does not track these loads, so
// it does not make the LDS reads of the current tile wait for the loads of the
// next one (it cannot prove they touch different buffers).  The explicit
// "s_waitcnt vmcnt(0)" before the barrier that ends the next phase is what
// orders them.  The LDS address goes in M0 through an operand constraint, so
// the compiler itself writes M0 and knows what it holds.
//
// Hazards the compiler does not resolve for inline assembly: an LDS-writing
// buffer load must not follow an SALU write of M0 directly (one wait state,
// the s_nop 0 here), and must not read an SGPR written by a VALU instruction
// (v_readfirstlane) within five wait states -- rsrc_words ends with those.
__device__ __forceinline__ void load_to_lds(const i32x4& rsrc, uint32_t voffset, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}
// The destination as a generic pointer into the LDS: converted (and
// null-checked, on its 64 bits) at every load.  The key-split and 4-wave
// kernels use the 32-bit form above: with the pointers, the compiler keeps their
// high words and spills them inside its main loop (each reload then waits for
// every tile load in flight).  The unsplit 8-wave kernels keep this form, with
// which their main loops compile without spills (with the 32-bit form they gain
// some).
__device__ __forceinline__ void load_to_lds(const i32x4& rsrc, uint32_t voffset, const uint8_t* lds_block) {
  load_to_lds(rsrc, voffset, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_block));
}

// Buffer resource words for raw 16-byte loads over [base, base + bytes): 32-bit
// offsets, out-of-range offsets read zeros.  Wave-uniform.  The words come out
// of v_readfirstlane (VALU writes of SGPRs); the empty-bodied s_nop 4 that
// takes them as operands puts five wait states between those writes and any
// buffer load that reads them.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r = {(int)__builtin_amdgcn_readfirstlane((uint32_t)a),
             (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  asm volatile("s_nop 4" : "+s"(r));
  return r;
}

// The descriptor of the same buffer moved `delta` bytes on: base + delta and
// max(size - delta, 0) bytes, so each offset is range-checked exactly as it
// was against the unmoved descriptor.  On the scalar unit (no vector-written
// SGPRs, so no wait states are needed before a load reads it).
__device__ __forceinline__ i32x4 rsrc_advance(const i32x4& r, uint32_t delta) {
  int w0, w1, w2;
  asm("s_add_u32 %0, %3, %6\n\t"
      "s_addc_u32 %1, %4, 0\n\t"
      "s_sub_i32 %2, %5, %6\n\t"
      "s_max_i32 %2, %2, 0"
      : "=&s"(w0), "=&s"(w1), "=&s"(w2)
      : "s"(r[0]), "s"(r[1]), "s"(r[2]), "s"(delta)
      : "scc");
  return i32x4{w0, w1, w2, r[3]};
}

// Bytes of rows [kb, min(kb + BN, end)) of a tile at pitch `pitch`, on the
// scalar unit (left to itself the compiler clamps with a vector med3 and a
// vector multiply, then moves the result back to a scalar register: a chain of
// dependent instructions in front of every tile load).
__device__ __forceinline__ uint32_t tile_bytes(int end, int kb, int bn, uint32_t pitch) {
  int r;
  asm("s_sub_i32 %0, %1, %2\n\t"
      "s_min_i32 %0, %0, %3\n\t"
      "s_max_i32 %0, %0, 0\n\t"
      "s_mul_i32 %0, %0, %4"
      : "=&s"(r)
      : "s"(end), "s"(kb), "s"(bn), "s"(pitch)
      : "scc");
  return (uint32_t)r;
}

// Workgroup barrier that also orders every memory access around it in the
// compiler; with wait_loads the wave first waits for its own outstanding
// global/buffer loads (including the LDS-writing ones).
__device__ __forceinline__ void barrier(bool wait_loads) {
  if (wait_loads)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ float lane_xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const uint32_t a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS reads (gfx950).  Within each group of 16 lanes, tr8: lane i
// byte j = byte (i % 8) of the 8 bytes addressed by lane 2j + i/8; tr16: lane i
// element j = element (i % 4) of the 4 halves addressed by lane 4j + i/4.
// Operand reads take an LDS byte address.  The K reads' per-lane register
// already holds the LDS address of the K region, so what is added to it is a
// compile-time offset below 64 KB that fits the instruction's immediate field
// (with the region base left in the constant, a 96 KB layout puts the K
// buffers out of the immediate's reach and every read needs a vector add).
// The V buffers come first in LDS, so their reads fit as they are.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}
__device__ __forceinline__ i32x2v lds_tr8(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2v*)(size_t)a);
}
__device__ __forceinline__ i16x4 lds_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(size_t)a);
}
__device__ __forceinline__ i32x4 lds_load16_at(uint32_t a) {
  return *(const __attribute__((address_space(3))) i32x4*)(size_t)a;
}

template <bool FP8>
struct QOp;
template <>
struct QOp<true> {
  using T = i32x8;
};
template <>
struct QOp<false> {
  using T = bf16x8;
};

template <int DV>
struct RowState {
  f32x16 o[DV / 32];  // O^T accumulator: lane owns query l % 32, channels 32d + 8i + 4hl + j
  float m;            // running max, log2 domain
  f32x4 l4;           // the full row sum (every entry)
  f32x16 l16;         // the same, from the all-ones row-sum MFMA (shift per 64-key step)
  float lrun;         // shift per tile: the row sum, each step's part scaled back by its 2^-k
  float kc;           // lean P: integer code offset K = 8 (SHIFT - m) + C0 (m kept on that grid)
};

// Probability shifts of the FP8 kernels: none (a fixed 2^SHIFT), one power of
// two per query and 64-key P.V step, or one per query and key tile.
enum PShift { kShiftNone = 0, kShiftStep = 1, kShiftTile = 2 };

// Lean P.  The e4m3 code of 2^x (x in [-6, 8]) is 8x + 56 at integer x and
// linear in between, so a probability's code is round(8 x + C0) with x = s c -
// m + SHIFT.  One FMA computes MAGIC + 8 s c + K (K = 8 (SHIFT - m) + C0, an
// integer because m is kept on that grid): with MAGIC = 1.5 * 2^23 the float's
// low mantissa byte is the rounded code.  One max against MAGIC clamps codes below 0
// (the float then equals MAGIC: code 0, also for masked -inf scores) and writes
// that low byte into the packed probability word (SDWA byte select).  C0 centres
// the error of the linear mantissa: 55.66 minimises the largest log error over
// an octave.
constexpr float kLeanC0 = 55.66f;
constexpr float kLeanMagic = 12582912.0f;  // 1.5 * 2^23

// Lean-P byte inserts of NBLK score blocks (their FMAs already applied):
// byte j of word 4 blk + i is the code of score 4 i + j of block blk.
template <int NBLK>
__device__ __forceinline__ void lean_insert_bytes(uint32_t* pk, const f32x16 (&t)[NBLK], float magic) {
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = t[blk][4 * i];
      asm("v_max_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
          : "=v"(pk[4 * blk + i]) : "v"(x), "v"(magic));
    }
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = t[blk][4 * i + 1];
      asm("v_max_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
          : "+v"(pk[4 * blk + i]) : "v"(x), "v"(magic));
    }
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = t[blk][4 * i + 2];
      asm("v_max_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
          : "+v"(pk[4 * blk + i]) : "v"(x), "v"(magic));
    }
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = t[blk][4 * i + 3];
      asm("v_max_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
          : "+v"(pk[4 * blk + i]) : "v"(x), "v"(magic));
    }
}

template <class C, bool FP8, int DQK, int DV>
struct Wave {
  static constexpr int NBLK = C::NBLK;
  // per-lane LDS byte offsets (relative to a buffer)
  uint32_t k_lane[C::KG];   // K operand: LDS address of K buffer 0 + row l % 32, chunk group position (k-half folded in)
  uint32_t v_lane[DV / 32]; // V^T operand per 32-channel block: the lane's offset in a V buffer (V buffers lie
                            // in the first 64 KB of the workgroup's LDS, within reach of the immediate)
  uint32_t k_dma[C::K_UNI ? 1 : C::K_PER_WAVE];
  uint32_t v_dma[C::V_UNI ? 1 : C::V_PER_WAVE];
  typename QOp<FP8>::T q[C::QK_STEPS];
  f32x16 s[NBLK];
  uint32_t pk[FP8 ? C::BN / 8 : C::BN / 4];  // this lane's probabilities of the tile (half its keys), MFMA B-operand order
  uint32_t pscale;  // probability shift: E8M0 exponent of this query's P (k-step ks in byte ks, or byte 0 per tile)
  RowState<DV> st;
};

}  // namespace

// One work item: the kBM queries of query tile qt of (batch, head) bh, against
// all keys up to the last of them.  Key tiles are visited in increasing order,
// or from the last one down when `rev` is set (the softmax is the same in any
// key order; the order only decides which tiles the workgroups of an XCD read
// at the same time).  Called by every thread of the workgroup; leaves no load
// in flight and no wave reading LDS when it returns.
template <int DQK, int DV, bool FP8, bool BS, int PSH, bool LEAN, bool SPLIT, bool SHORT, int NW>
__device__ __forceinline__ void attn_item(const AttnParams& p, uint8_t* smem, uint32_t* ebuf, int bh, int qt,
                                          bool rev, int ta, int tb, int slot) {
  static_assert(!BS || FP8, "block scales are an FP8 feature");
  static_assert(PSH == kShiftNone || FP8, "probability shifts are an FP8 feature");
  constexpr bool PS = PSH == kShiftStep, PT = PSH == kShiftTile;
  static_assert(kShiftStep == 1, "tile_keys names the per-64-key shift by its value");

  static_assert(!LEAN || FP8, "lean-P codes are e4m3 codes");
  // NW = 8: two wave groups in ping-pong, 256 queries; NW = 4: one wave per
  // SIMD doing both halves of every step, 128 queries (unsplit launches only)
  static_assert(NW == 8 || (NW == 4 && !SPLIT), "the key split runs 8-wave workgroups");
  constexpr bool SOLO = NW == 4;
  constexpr int kWaves = NW, kThreads = 64 * NW, kBM = 32 * NW;
  using C = Cfg<FP8, DQK, DV, tile_keys<FP8, DQK, BS, PSH, SHORT>(), NW>;
  constexpr int NBLK = C::NBLK;
  constexpr int BN = C::BN;
  static_assert(!PS || BN == 128, "the per-64-key shift's four max chains cover two 64-key steps");
  static_assert(!BS || BN == 128 || BN == 192, "block-scale exponents are staged per 128- or 192-key tile");
  // block scales: ebuf words per tile (128 keys: one word, K and V exponents
  // of its two 64-key blocks; 192 keys: a K word and a V word, three blocks
  // each), and the byte of a V word that holds the exponent of P.V k-step 0
  constexpr int EW = BS && BN == 192 ? 2 : 1;
  constexpr int VSEL = BS && BN == 192 ? 0 : 2;
  constexpr bool V3 = BS && BN == 192;  // a third P.V k-step reads V byte 2
  static_assert(C::V_TILE % (16 * kThreads) == 0, "the zero-filled V buffer splits into whole stores");
  uint8_t* const Vs = smem;                 // V buffers 0, 1
  uint8_t* const Ks = smem + 2 * C::V_TILE;  // K buffers 0, 1
  // the tile loads' destinations (LDS byte addresses in the key-split and
  // 4-wave kernels, generic pointers otherwise; see load_to_lds)
  const uint32_t vs_lds = __builtin_amdgcn_readfirstlane(lds_addr(Vs));
  auto k_dst = [&](int buf, int blk) __attribute__((always_inline)) {
    if constexpr (SPLIT || SOLO) return vs_lds + 2 * C::V_TILE + buf * C::K_TILE + 1024 * blk;
    else return Ks + buf * C::K_TILE + 1024 * blk;
  };
  auto v_dst = [&](int buf, int blk) __attribute__((always_inline)) {
    if constexpr (SPLIT || SOLO) return vs_lds + buf * C::V_TILE + 1024 * blk;
    else return Vs + buf * C::V_TILE + 1024 * blk;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int grp = SOLO ? 0 : w >> 2;  // 0: matrix work on even phases, 1: on odd phases
  const int Nq = p.Nq, Nk = p.Nk;
  const int off = Nk - Nq;  // position of query row 0 in the key sequence
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / (p.Hq / p.Hkv);
  const int q0 = qt * kBM;
  // SIMD s runs waves s (group 0) and s + 4 (group 1); they own query blocks
  // 2s and 2s + 1, so both groups have work on the diagonal tiles.
  const int qblk = SOLO ? w : 2 * (w & 3) + grp;
  const int qw0 = q0 + 32 * qblk;  // first query of this wave
  const int my_q = qw0 + l32;      // query row owned by this lane (position my_q + off)

  const uint32_t q_pitch = (uint32_t)p.Hq * C::KROW;  // bytes between consecutive positions
  const uint32_t k_pitch = (uint32_t)p.Hkv * C::KROW;
  const uint32_t v_pitch = (uint32_t)p.Hkv * C::VROW;
  const uint8_t* Q = static_cast<const uint8_t*>(p.q) + ((size_t)b * Nq * p.Hq + h) * C::KROW;
  const uint8_t* K = static_cast<const uint8_t*>(p.k) + ((size_t)b * Nk * p.Hkv + g) * C::KROW;
  const uint8_t* V = static_cast<const uint8_t*>(p.v) + ((size_t)b * Nk * p.Hkv + g) * C::VROW;

  float c = p.sm_scale_log2;  // log2-domain score scale (dequantisation folded in for FP8)
  float sv = 1.f;
  if constexpr (FP8 && BS) {
    const int nbq = (Nq + 63) / 64;
    c *= p.q_scale[((size_t)b * p.Hq + h) * nbq + min(qw0, Nq - 1) / 64];
  } else if constexpr (FP8) {
    c *= p.q_scale[b * p.Hq + h] * p.k_scale[b * p.Hkv + g];
    sv = p.v_scale[b * p.Hkv + g];
  }

  Wave<C, FP8, DQK, DV> wv;

  // ---- per-lane LDS offsets of the operand reads
  // chunk ct of a K-operand read is logical chunk ct + (2 or 1) * hl of the
  // lane's row l % 32 (the rows of block blk are l % 32 + 32 blk, same swizzle)
#pragma unroll
  for (int ct = 0; ct < C::KG; ++ct)
    wv.k_lane[ct] = lds_addr(Ks) + l32 * C::KROW + 16 * ((ct ^ (hl * (FP8 ? 2 : 1)) ^ k_swizzle<C>(l32)) & (C::KG - 1));
  {
    const int grp16 = lane >> 4, s16 = lane & 15;
    const int lhl = grp16 >> 1, gc = grp16 & 1;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
      if constexpr (FP8) {
        // source lane s16 = 2j + hh reads 8 bytes: key 8(j/4) + 4hl + j%4,
        // channels 32db + 16gc + 8hh .. +8
        const int j = s16 >> 1, hh = s16 & 1;
        const int key = 8 * (j >> 2) + 4 * lhl + (j & 3);
        const int ch = 2 * db + gc;
        wv.v_lane[db] = key * C::VROW + 16 * (ch ^ v_swizzle<true>(key)) + 8 * hh;
      } else {
        // source lane s16 = 4j + qq reads 4 halves: key 4hl + j, channels
        // 32db + 16gc + 4qq .. +4
        const int j = s16 >> 2, qq = s16 & 3;
        const int key = 4 * lhl + j;
        const int ch = 4 * db + 2 * gc + (qq >> 1);
        wv.v_lane[db] = key * C::VROW + 16 * (ch ^ v_swizzle<false>(key)) + 8 * (qq & 1);
      }
    }
  }
  // (opaque from here on: the region bases stay in the registers; only the
  // chunk positions the K reads use, chunks 4kk + {0, 1} (FP8) or 2kk (BF16))
#pragma unroll
  for (int ct = 0; ct < C::KG; ++ct) {
    const bool used = FP8 ? ((ct & 3) < 2 && ct < 4 * C::QK_STEPS) : ((ct & 1) == 0 && ct < 2 * C::QK_STEPS);
    if (used) asm volatile("" : "+v"(wv.k_lane[ct]));
  }
  // ---- per-lane global offsets of the tile loads (tile-relative, the same for every tile)
#pragma unroll
  for (int i = 0; i < (C::K_UNI ? 1 : C::K_PER_WAVE); ++i) {
    const int blk = w + kWaves * i;
    const int pos = 64 * blk + lane, row = pos / C::KCH, slot = pos % C::KCH;
    wv.k_dma[i] = (uint32_t)row * k_pitch + 16u * k_chunk_pos<C>(row, slot);
  }
#pragma unroll
  for (int i = 0; i < (C::V_UNI ? 1 : C::V_PER_WAVE); ++i) {
    const int blk = w + kWaves * i;
    const int pos = 64 * blk + lane, key = pos / C::VCH, slot = pos % C::VCH;
    wv.v_dma[i] = (uint32_t)key * v_pitch + 16u * (slot ^ v_swizzle<FP8>(key));
  }
  // bytes between a wave's consecutive load blocks, where they share one offset
  const uint32_t k_blk_bytes = __builtin_amdgcn_readfirstlane(C::K_ROWS_STEP * k_pitch);
  const uint32_t v_blk_bytes = __builtin_amdgcn_readfirstlane(C::V_ROWS_STEP * v_pitch);

  const int kend = min(q0 + kBM, Nq) + off;  // keys visible to the workgroup's last query, plus one
  // key tiles of the item: [ta, T), a key range of the query tile (key split) or
  // all of it (ta = 0).  (Without the split the expressions below are kept
  // free of the range: the unsplit kernel's register allocation is sensitive
  // to them.)
  const int T = SPLIT ? min((kend + BN - 1) / BN, tb) : (kend + BN - 1) / BN;
  const int NT = SPLIT ? T - ta : T;  // steps 0..NT (step NT only drains the last P.V product)
  // tiles this wave needs: keys up to the position of its last valid query
  const int Tw = qw0 < Nq ? (SPLIT ? max(0, min((min(qw0 + 31, Nq - 1) + off) / BN + 1, T) - ta)
                                   : ((min(qw0 + 31, Nq - 1) + off) / BN + 1))
                          : 0;
  // steps [s_lo, s_hi) carry the wave's tiles; step s visits tile tile_of(s),
  // and steps at or beyond NT map to tile T (an empty load range).  A reversed
  // walk covers a whole query tile.
  const int s_lo = rev ? NT - Tw : 0, s_hi = rev ? NT : Tw;
  const int t_base = rev ? T - 1 : (SPLIT ? ta : 0), t_dir = rev ? -1 : 1;
  // (unsigned min: the -1 of a downward walk past tile 0 also maps to T)
  auto tile_of = [&](int s) __attribute__((always_inline)) {
    return (int)min((uint32_t)(t_base + t_dir * s), (uint32_t)T);
  };

  // tiles at or beyond T load with an empty range (zeros, no memory access), so
  // the loads need no branches
  // (read-first-lane: keeps the load-range arithmetic on the scalar unit)
  const int krows_end = __builtin_amdgcn_readfirstlane(min(Nk, T * BN));
  auto issue_k = [&](int t, int buf) __attribute__((always_inline)) {
    const int kb = t * BN;
    const i32x4 rk = rsrc_words(K + (size_t)min(kb, krows_end) * k_pitch, tile_bytes(krows_end, kb, BN, k_pitch));
#pragma unroll
    for (int i = 0; i < C::K_PER_WAVE; ++i) {
      const int blk = w + kWaves * i;
      if constexpr (C::K_UNI)
        load_to_lds(i == 0 ? rk : rsrc_advance(rk, i * k_blk_bytes), wv.k_dma[0], k_dst(buf, blk));
      else
        load_to_lds(rk, wv.k_dma[i], k_dst(buf, blk));
    }
  };
  auto issue_v = [&](int t, int buf) __attribute__((always_inline)) {
    const int kb = t * BN;
    const i32x4 rv = rsrc_words(V + (size_t)min(kb, krows_end) * v_pitch, tile_bytes(krows_end, kb, BN, v_pitch));
#pragma unroll
    for (int i = 0; i < C::V_PER_WAVE; ++i) {
      const int blk = w + kWaves * i;
      if constexpr (C::V_UNI)
        load_to_lds(i == 0 ? rv : rsrc_advance(rv, i * v_blk_bytes), wv.v_dma[0], v_dst(buf, blk));
      else
        load_to_lds(rv, wv.v_dma[i], v_dst(buf, blk));
    }
  };
  // loads of step p: K tile p+1 and V tile p
  auto issue_step = [&](int pstep) __attribute__((always_inline)) {
    issue_k(tile_of(pstep + 1), (pstep + 1) & 1);
    issue_v(tile_of(pstep), pstep & 1);
  };

  // ---- Q^T operand in registers.  BF16: k-step kk = channels [16kk, 16kk+16),
  // lane half hl holds 8 of them; FP8: k-step kk = channels [64kk, 64kk+64), 32 each.
  {
    const uint32_t rows = (uint32_t)max(0, min(32, Nq - qw0));
    const auto rq = make_rsrc(Q + (size_t)min(qw0, Nq) * q_pitch, rows * q_pitch);
#pragma unroll
    for (int kk = 0; kk < C::QK_STEPS; ++kk) {
      if constexpr (FP8) {
        const uint32_t off = (uint32_t)l32 * q_pitch + kk * 64 + hl * 32;
        const i32x4 lo = bload16(rq, off), hi = bload16(rq, off + 16);
        wv.q[kk] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        wv.q[kk] = __builtin_bit_cast(bf16x8, bload16(rq, (uint32_t)l32 * q_pitch + kk * 32 + hl * 16));
      }
    }
    // Pass the Q registers through an empty asm so the compiler waits for these
    // loads here, once, instead of at their first use inside the loop (where
    // the wait would also stall on the tile loads in flight).
#pragma unroll
    for (int kk = 0; kk < C::QK_STEPS; ++kk) asm volatile("" : "+v"(wv.q[kk]));
  }

#pragma unroll
  for (int d = 0; d < DV / 32; ++d) wv.st.o[d] = zero16();
  wv.st.m = -1e30f;
  wv.st.l4 = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (PS) wv.st.l16 = zero16();
  if constexpr (PT) wv.st.lrun = 0.f;
  wv.st.kc = 0.f;
  // Row-sum selector (A operand of the 16x16 row-sum MFMA): 1.0 where the lane
  // group's parity matches its row group's parity, else 0.  Lane l then finds
  // the sum over the k-step's keys for its own query l % 32 in every entry of
  // its D registers.
  // The eight operand registers are rebuilt where a step's first row-sum MFMA
  // needs them, instead of being held through the softmax, where registers are
  // scarcest: one select against the constant lane mask of the pattern (bit l
  // set where ((l >> 4) & 1) == ((l >> 2) & 1)), one AND, seven copies.  (The
  // matrix wave's vector instructions share the SIMD's vector unit with the
  // other wave's softmax, so the rebuild is kept this short.)
  auto selector = []() __attribute__((always_inline)) {
    int w;  // volatile: rebuilt in every step, not hoisted out of the loop
    asm volatile("v_cndmask_b32_e64 %0, 0, -1, %1\n\tv_and_b32_e32 %0, %2, %0"
                 : "=v"(w)
                 : "s"(0xf0f00f0ff0f00f0full), "i"(FP8 ? 0x38383838 : 0x3f803f80));  // e4m3 / bf16 ones
    return i32x8{w, w, w, w, w, w, w, w};
  };
  i32x8 sel;
  f32x4 rs;  // shift per tile: row sum of one step's codes (every entry), inside a matrix phase
  // With probability block scaling the row sum is a 32x32x64 MFMA against an
  // all-ones A: its B exponents are read per (column, 32-key block) as in the
  // P.V product (the 16x16x128 form reads one column's exponents from the lanes
  // of a single query, but that column also holds another query's keys).
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0

  // E8M0 exponents of the K tile (bytes 0, 1: its two 64-key blocks) and V tile
  // (bytes 2, 3) of the current matrix phase (block scales only)
  // (unit exponents 127 without block scales: only the probability scale applies)
  uint32_t kexp = 0, vexp = BS ? 0u : 0x7f7f7f7fu;

  // ---- matrix work of step pstep: P_{pstep-1} V_{pstep-1}, then S_pstep = K_pstep Q^T.
  // The products form one list of MFMAs (PV first, then QK with the k-steps
  // outermost so consecutive MFMAs are independent); the LDS operand of MFMA
  // i+1 is read while MFMA i runs.
  constexpr int PV_OPS = FP8 ? (BN / 64) * (DV / 32) : (BN / 16) * (DV / 32);
  constexpr int QK_OPS = NBLK * C::QK_STEPS;
  using AOp = typename std::conditional<FP8, i32x8, i32x4>::type;
  auto fetch = [&](int i, const uint8_t* vb, const uint8_t* kb) __attribute__((always_inline)) -> AOp {
    AOp a;
    if (i < PV_OPS) {
      if constexpr (FP8) {
        const int ks = i / (DV / 32), db = i % (DV / 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2v t = lds_tr8(lds_addr(vb) + wv.v_lane[db] + (64 * ks + 32 * (r >> 1) + 16 * (r & 1)) * C::VROW);
          a[2 * r] = t[0];
          a[2 * r + 1] = t[1];
        }
      } else {
        const int chunk = i / (DV / 32), db = i % (DV / 32);
        const i16x4 t0 = lds_tr16(lds_addr(vb) + wv.v_lane[db] + (16 * chunk) * C::VROW);
        const i16x4 t1 = lds_tr16(lds_addr(vb) + wv.v_lane[db] + (16 * chunk + 8) * C::VROW);
        const i32x2v u0 = __builtin_bit_cast(i32x2v, t0), u1 = __builtin_bit_cast(i32x2v, t1);
        a = i32x4{u0[0], u0[1], u1[0], u1[1]};
      }
    } else {
      const int j = i - PV_OPS, kk = j / NBLK, blk = j % NBLK;
      const uint32_t row = (uint32_t)(kb - Ks) + blk * 32 * C::KROW;  // a compile-time offset
      if constexpr (FP8) {
        // logical chunks 4kk + 2hl + {0, 1}
        const int c0 = 4 * kk, c1 = 4 * kk + 1;
        const i32x4 lo = lds_load16_at(wv.k_lane[c0 & (C::KG - 1)] + row + 16 * (c0 & ~(C::KG - 1)));
        const i32x4 hi = lds_load16_at(wv.k_lane[c1 & (C::KG - 1)] + row + 16 * (c1 & ~(C::KG - 1)));
        a = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const int c0 = 2 * kk;  // logical chunk 2kk + hl
        a = lds_load16_at(wv.k_lane[c0 & (C::KG - 1)] + row + 16 * (c0 & ~(C::KG - 1)));
      }
    }
    return a;
  };
  auto mma = [&](int i, const AOp& a) __attribute__((always_inline)) {
    if (i < PV_OPS) {
      if constexpr (FP8) {
        const int ks = i / (DV / 32), db = i % (DV / 32);
        const i32x8 pb = {(int)wv.pk[8 * ks + 0], (int)wv.pk[8 * ks + 1], (int)wv.pk[8 * ks + 2],
                          (int)wv.pk[8 * ks + 3], (int)wv.pk[8 * ks + 4], (int)wv.pk[8 * ks + 5],
                          (int)wv.pk[8 * ks + 6], (int)wv.pk[8 * ks + 7]};
        if constexpr (PS) {
          if (db == 0)
            wv.st.l16 = ks == 0 ? mfma_fp8_32x32x64_sab<0, 0>(ones, pb, wv.st.l16, 127, (int)wv.pscale)
                                : mfma_fp8_32x32x64_sab<0, 1>(ones, pb, wv.st.l16, 127, (int)wv.pscale);
          wv.st.o[db] = ks == 0 ? mfma_fp8_32x32x64_sab<2, 0>(a, pb, wv.st.o[db], (int)vexp, (int)wv.pscale)
                                : mfma_fp8_32x32x64_sab<3, 1>(a, pb, wv.st.o[db], (int)vexp, (int)wv.pscale);
        } else if constexpr (PT) {
          // the step's row sum on its own (scaled back when the phase ends)
          if (db == 0) rs = mfma_fp8_16x16x128(sel, pb, ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : rs);
          wv.st.o[db] = ks == 0 ? mfma_fp8_32x32x64_sab<VSEL, 0>(a, pb, wv.st.o[db], (int)vexp, (int)wv.pscale)
                        : (V3 && ks == 2) ? mfma_fp8_32x32x64_sab<2, 0>(a, pb, wv.st.o[db], (int)vexp, (int)wv.pscale)
                                                  : mfma_fp8_32x32x64_sab<VSEL + 1, 0>(a, pb, wv.st.o[db], (int)vexp,
                                                                                      (int)wv.pscale);
        } else {
          if (db == 0) wv.st.l4 = mfma_fp8_16x16x128(sel, pb, wv.st.l4);
          if constexpr (BS)
            wv.st.o[db] = ks == 0 ? mfma_fp8_32x32x64_sa<VSEL>(a, pb, wv.st.o[db], (int)vexp)
                          : (V3 && ks == 2) ? mfma_fp8_32x32x64_sa<2>(a, pb, wv.st.o[db], (int)vexp)
                                                    : mfma_fp8_32x32x64_sa<VSEL + 1>(a, pb, wv.st.o[db], (int)vexp);
          else
            wv.st.o[db] = mfma_fp8_32x32x64(a, pb, wv.st.o[db]);
        }
      } else {
        const int chunk = i / (DV / 32), db = i % (DV / 32);
        const i32x4 pw = {(int)wv.pk[4 * chunk], (int)wv.pk[4 * chunk + 1], (int)wv.pk[4 * chunk + 2],
                          (int)wv.pk[4 * chunk + 3]};
        if (db == 0)
          wv.st.l4 = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(sel, sel, 0, 1, 2, 3)),
                                        __builtin_bit_cast(bf16x8, pw), wv.st.l4);
        wv.st.o[db] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pw), wv.st.o[db]);
      }
    } else {
      const int j = i - PV_OPS, kk = j / NBLK, blk = j % NBLK;
      const f32x16 acc = kk == 0 ? zero16() : wv.s[blk];
      if constexpr (FP8 && BS)
        wv.s[blk] = blk < 2 ? mfma_fp8_32x32x64_sa<0>(a, wv.q[kk], acc, (int)kexp)
                    : blk < 4 ? mfma_fp8_32x32x64_sa<1>(a, wv.q[kk], acc, (int)kexp)
                              : mfma_fp8_32x32x64_sa<2>(a, wv.q[kk], acc, (int)kexp);
      else if constexpr (FP8)
        wv.s[blk] = mfma_fp8_32x32x64(a, wv.q[kk], acc);
      else
        wv.s[blk] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), wv.q[kk], acc);
    }
  };
  // LDS reads of the operand of list entry i, and MFMAs it issues
  auto n_reads = [](int i) constexpr { return i < PV_OPS ? (FP8 ? 4 : 2) : (FP8 ? 2 : 1); };
  auto n_mfma = [](int i) constexpr { return (i < PV_OPS && i % (DV / 32) == 0) ? 2 : 1; };
  // MFMAs [i0, i1) of the list; the operand of MFMA i+2 is read before MFMA i
  // issues (three operand buffers), an order pinned with scheduling groups.
  auto run_ops = [&](auto i0_tag, auto i1_tag, const uint8_t* vb, const uint8_t* kb) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0_tag)::value, I1 = decltype(i1_tag)::value;
    AOp buf[3];
    buf[0] = fetch(I0, vb, kb);
    __builtin_amdgcn_sched_group_barrier(0x100, n_reads(I0), 0);
    if constexpr (I0 + 1 < I1) {
      buf[1] = fetch(I0 + 1, vb, kb);
      __builtin_amdgcn_sched_group_barrier(0x100, n_reads(I0 + 1), 0);
    }
    static_for<I0, I1>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + 2 < I1) {
        buf[(i + 2 - I0) % 3] = fetch(i + 2, vb, kb);
        __builtin_amdgcn_sched_group_barrier(0x100, n_reads(i + 2), 0);
      }
      mma(i, buf[(i - I0) % 3]);
      __builtin_amdgcn_sched_group_barrier(0x008, n_mfma(i), 0);
    });
  };
  auto matrix_work = [&](int pstep, auto parity) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parity)::value;  // pstep & 1
    const uint8_t* vb = Vs + (1 - PAR) * C::V_TILE;       // V tile pstep-1
    const uint8_t* kb = Ks + PAR * C::K_TILE;  // K tile pstep
    // One instruction sequence for every step the wave takes part in (a single
    // variant keeps the register allocation tight): at step s_lo the P.V
    // product multiplies the zero probabilities the item starts with (by a
    // zero-filled or fully loaded V buffer), and at step s_hi the scores of a
    // tile the wave does not need are computed and never read.
    if (pstep >= s_lo && pstep <= s_hi) {
      sel = selector();
      if constexpr (BS) {
        kexp = ebuf[EW * tile_of(pstep)];
        vexp = ebuf[EW * tile_of(pstep - 1) + EW - 1];
      }
      run_ops(std::integral_constant<int, 0>{}, std::integral_constant<int, PV_OPS + QK_OPS>{}, vb, kb);
      // shift per tile: the row sum of the probabilities just multiplied (they
      // were 2^k too large; pscale holds the E8M0 exponent of 2^-k, which is
      // also its fp32 exponent field) joins the running sum.  Its MFMAs were
      // among the first of the phase, so their result is ready.
      if constexpr (PT) wv.st.lrun = __builtin_fmaf(rs[0], __uint_as_float(wv.pscale << 23), wv.st.lrun);
    }
  };

  // ---- vector work of step pstep: online softmax of S_pstep -> probabilities.
  auto vector_work = [&](int pstep) __attribute__((always_inline)) {
    if (pstep < s_lo || pstep >= s_hi) return;
    const int kb = tile_of(pstep) * BN;
    if (kb + BN - 1 > qw0 + off) {  // the tile crosses this wave's diagonal: mask keys above each query
      // key offset k of register r is visible iff k <= lim; the sign of lim - k
      // selects -inf bit by bit (no per-element compare masks held in SGPRs)
      const int lim = my_q + off - kb - 4 * hl;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t hide = (uint32_t)((lim - (blk * 32 + 8 * (r >> 2) + (r & 3))) >> 31);
          const float x = wv.s[blk][r];  // scalar copy before the bit cast
          wv.s[blk][r] = __uint_as_float((hide & 0xff800000u) | (~hide & __float_as_uint(x)));
        }
    }
    // row max: four independent chains of 3-input max (two new values each);
    // with probability block scaling, chains 2ks and 2ks+1 cover exactly this
    // lane's keys of k-step ks (blocks 2ks, 2ks+1)
    float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float& m = mc[PS ? 2 * (blk >> 1) + ((r >> 1) & 1) : (blk * 8 + r / 2) & 3];
        m = fmaxf(fmaxf(m, wv.s[blk][r]), wv.s[blk][r + 1]);
      }
    float mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
    mx = lane_xor32_max(mx);
    const float mt = mx * c;
    if (__any(mt > wv.st.m + C::THRESH)) {  // wave-uniform; rare once the max settles
      float m_new = fmaxf(wv.st.m, mt);
      if constexpr (LEAN) {
        // round the new max up onto the grid where K = 8 (SHIFT - m) + C0 is an integer
        const float kc = floorf(8.f * (C::SHIFT - m_new) + kLeanC0);
        const bool up = mt > wv.st.m;
        m_new = up ? C::SHIFT + (kLeanC0 - kc) * 0.125f : wv.st.m;
        wv.st.kc = up ? kc : wv.st.kc;
      }
      const float alpha = fast_exp2(wv.st.m - m_new);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) wv.st.o[d] *= alpha;
      if constexpr (PS)
        wv.st.l16 *= alpha;
      else if constexpr (PT)
        wv.st.lrun *= alpha;
      else
        wv.st.l4 *= alpha;
      wv.st.m = m_new;
    }
    const float bias = C::SHIFT - wv.st.m;
    if constexpr (FP8) {
      // pk[8ks + 4hb + i] holds keys 64ks + 32hb + 8i + 4hl + {0..3}
      // Probability block scaling: k = floor(running max - the query's max
      // over the 64 keys of k-step ks) octaves, in [0, 126]; the probabilities
      // of the k-step are 2^k times larger (lean P: codes up by 8k) and the
      // MFMA scale is 2^-k (a k-step whose keys are all masked gets k = 126
      // and codes 0).  Without it, k = 0.
      // Shift per tile: one k = min(floor(running max - the query's max over
      // the tile), 126) for the whole tile (k may be slightly negative while
      // the tile max runs ahead of the lazy running max; the largest
      // probability is then at most 2^SHIFT).
      float kst[NBLK / 2];
      if constexpr (PT) {
        const float kt = fminf(floorf(wv.st.m - mt), 126.f);
        wv.pscale = (uint32_t)(127 - (int)kt);  // E8M0 exponent of 2^-k
#pragma unroll
        for (int ks = 0; ks < NBLK / 2; ++ks) kst[ks] = kt;
      }
      if constexpr (PS) {
        uint32_t ps = 0;
#pragma unroll
        for (int ks = 0; ks < NBLK / 2; ++ks) {
          const float bmax = lane_xor32_max(fmaxf(mc[2 * ks], mc[2 * ks + 1]));
          kst[ks] = fminf(fmaxf(floorf(__builtin_fmaf(-bmax, c, wv.st.m)), 0.f), 126.f);
          ps |= (uint32_t)(127 - (int)kst[ks]) << (8 * ks);
        }
        wv.pscale = ps;
      }
      if constexpr (LEAN) {
        // lean P: one FMA gives MAGIC + the code (low mantissa byte), one SDWA
        // max clamps it and inserts the byte
        const float c8 = 8.f * c, b8 = kLeanMagic + wv.st.kc, magic = kLeanMagic;
        float bks[NBLK / 2];  // code offset of k-step ks
#pragma unroll
        for (int ks = 0; ks < NBLK / 2; ++ks) bks[ks] = PSH != kShiftNone ? __builtin_fmaf(8.f, kst[ks], b8) : b8;
        // Two passes: the FMAs in place, then the byte inserts byte-major over
        // all words, so consecutive inserts are independent (the four inserts
        // of one word form a chain: each keeps the bytes written before it).
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) wv.s[blk][r] = __builtin_fmaf(wv.s[blk][r], c8, bks[blk >> 1]);
        __builtin_amdgcn_sched_barrier(0);
        lean_insert_bytes<NBLK>(wv.pk, wv.s, magic);
      } else {
        // exact P: exp2 and the hardware round-to-nearest-even e4m3 conversion
        float bexp[NBLK / 2];  // log2-domain offset of k-step ks
#pragma unroll
        for (int ks = 0; ks < NBLK / 2; ++ks) bexp[ks] = PSH != kShiftNone ? bias + kst[ks] : bias;
        // (three passes in place -- arguments, exp2, conversions -- so that no
        // instruction waits on the one before it; see the BF16 branch)
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) wv.s[blk][r] = __builtin_fmaf(wv.s[blk][r], c, bexp[blk >> 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) wv.s[blk][r] = fast_exp2(wv.s[blk][r]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wv.pk[4 * blk + i] = pack_fp8x4(wv.s[blk][4 * i], wv.s[blk][4 * i + 1], wv.s[blk][4 * i + 2],
                                            wv.s[blk][4 * i + 3]);
      }
    } else {
      // pk[2r' + e] with r' = 8blk + ... : register pair (r, r+1) of block blk.
      // Three passes in place over the scores -- the exp2 arguments, exp2, the
      // packs -- separated by scheduling barriers: interleaved, each exp2 read
      // the FMA just before it and each pack the exp2 results just before it
      // (0.8% slower on the 32K workload, same bits).
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) wv.s[blk][r] = __builtin_fmaf(wv.s[blk][r], c, bias);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) wv.s[blk][r] = fast_exp2(wv.s[blk][r]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 8; ++i) wv.pk[8 * blk + i] = pack_bf16x2(wv.s[blk][2 * i], wv.s[blk][2 * i + 1]);
    }
  };

  // ---- prologue: the tiles' scale exponents (block scales) into LDS; K tile 0
  // into buffer 0; V buffer 1 (read by the empty P.V product of step 0) and the
  // probabilities start at zero.
  if constexpr (BS) {
    // 128-key tiles: word t = E8M0 of K blocks 2t, 2t+1 and V blocks 2t, 2t+1;
    // 192-key tiles: word 2t = K blocks 3t .. 3t+2, word 2t+1 = V blocks 3t ..
    // 3t+2 (indices past the last block repeat it: those keys load as zeros and
    // are masked)
    const int nbk = (Nk + 63) / 64;
    const float* ksc = p.k_scale + ((size_t)b * p.Hkv + g) * nbk;
    const float* vsc = p.v_scale + ((size_t)b * p.Hkv + g) * nbk;
    auto e8 = [](float x) __attribute__((always_inline)) { return (__float_as_uint(x) >> 23) & 0xffu; };
    for (int t = tid; t <= T; t += kThreads) {
      if constexpr (BN == 192) {
        const int i0 = min(3 * t, nbk - 1), i1 = min(3 * t + 1, nbk - 1), i2 = min(3 * t + 2, nbk - 1);
        ebuf[2 * t] = e8(ksc[i0]) | (e8(ksc[i1]) << 8) | (e8(ksc[i2]) << 16);
        ebuf[2 * t + 1] = e8(vsc[i0]) | (e8(vsc[i1]) << 8) | (e8(vsc[i2]) << 16);
      } else {
        const int i0 = min(2 * t, nbk - 1), i1 = min(2 * t + 1, nbk - 1);
        ebuf[t] = e8(ksc[i0]) | (e8(ksc[i1]) << 8) | (e8(vsc[i0]) << 16) | (e8(vsc[i1]) << 24);
      }
    }
  }
  issue_k(tile_of(0), 0);
#pragma unroll
  for (int i = 0; i < C::V_TILE / (16 * kThreads); ++i)
    lds_store16(Vs + C::V_TILE + 16 * (tid + kThreads * i), i32x4{0, 0, 0, 0});
#pragma unroll
  for (int i = 0; i < (int)(sizeof(wv.pk) / sizeof(wv.pk[0])); ++i) wv.pk[i] = 0u;
  wv.pscale = 0x7f7f7f7fu;  // unit scales
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (!SOLO && grp == 1) {
    issue_step(0);
    barrier(false);  // group B starts one phase later
  }

  // ---- main loop: steps 0..T (step T only drains P_{T-1} V_{T-1})
  // Both groups run the same matrix/vector code; only where each issues its
  // share of the tile loads and which barrier waits for them differ:
  //   group A: matrix(p) | barrier | vector(p), wait | barrier
  //   group B: matrix(p), wait | barrier | vector(p), loads(p+1) | barrier
  // Group A issues its loads of step p before its matrix work for FP8 and at
  // the start of its vector work for BF16, group B at the end of its vector
  // work: the placements that measured fastest (a burst of loads holds the
  // issuing waves for a few hundred cycles while the CU accepts them).  Every load of step p is waited for
  // at the barrier that ends phase 2p+1, when all waves have issued theirs.
  // No step runs past T, so no loads are issued for one either: an item ends
  // with no load in flight that could land in the next item's first tiles.
  auto step = [&](int ps, auto parity, auto group) __attribute__((always_inline)) {
    constexpr bool GA = decltype(group)::value == 0;
    if (GA && FP8) issue_step(ps);
    // The wave in its matrix phase takes issue priority over the other wave of
    // its SIMD, so a ready MFMA does not wait behind vector work (BF16 1.3%
    // faster; FP8 0.4% faster with 192-key tiles, 0.8% slower when its tiles
    // held 128 keys).
    __builtin_amdgcn_s_setprio(1);
    matrix_work(ps, parity);
    __builtin_amdgcn_s_setprio(0);
    barrier(!GA);
    if (GA && !FP8) issue_step(ps);
    vector_work(ps);
    if (!GA && ps + 1 <= NT) issue_step(ps + 1);
    barrier(GA);
  };
  // one loop per group, so the group decisions inside a step are compile-time
  auto run_steps = [&](auto group) __attribute__((always_inline)) {
    for (int ps = 0; ps <= NT; ps += 2) {
      step(ps, std::integral_constant<int, 0>{}, group);
      if (ps + 1 <= NT) step(ps + 1, std::integral_constant<int, 1>{}, group);
    }
  };
  if constexpr (SOLO) {
    // One wave per SIMD does the matrix and then the vector work of each step.
    // The loads of step p (K tile p+1, V tile p) are issued when step p starts,
    // after the barrier that follows every wave's matrix work of step p-1 (the
    // last reader of the buffers they fill), and are waited for at the barrier
    // that starts step p+1.
    auto solo_step = [&](int ps, auto parity) __attribute__((always_inline)) {
      if (ps > 0) barrier(true);
      if (ps < NT) issue_step(ps);
      matrix_work(ps, parity);
      vector_work(ps);
    };
    for (int ps = 0; ps <= NT; ps += 2) {
      solo_step(ps, std::integral_constant<int, 0>{});
      if (ps + 1 <= NT) solo_step(ps + 1, std::integral_constant<int, 1>{});
    }
    barrier(false);  // every wave is out of the loop before the epilogue reuses the tile buffers
  } else {
    if (grp == 0)
      run_steps(std::integral_constant<int, 0>{});
    else
      run_steps(std::integral_constant<int, 1>{});
    if (grp == 0) barrier(false);
  }

  // ---- epilogue: normalise by the row sum and store BF16
  const float lsum = PS ? wv.st.l16[0] : (PT ? wv.st.lrun : wv.st.l4[0]);
  if (SPLIT && slot >= 0) {
    // one key range of a split query tile: the rows normalised over the range,
    // in fp32, and the range's log2 sum of exp, for the merge.  A row that sees
    // no key of the range (its position lies before the range) has lsum = 0:
    // output 0 and sum -inf, a weight of 0 in the merge.
    const bool seen = lsum > 0.f;
    const float inv = seen ? sv / lsum : 0.f;
    if (my_q < Nq && hl == 0)
      p.ws_lse[(size_t)slot * kBM + (my_q - q0)] = seen ? wv.st.m - C::SHIFT + __log2f(lsum) : -INFINITY;
    // The fp32 rows go out through LDS as the BF16 rows below do (whole rows
    // per store), in two passes of 16 rows: a wave's 16 rows take 8 KB, 16-byte
    // chunk c of row r at chunk position c ^ 2r.  The range's rows are
    // consecutive in the workspace, so each pass stores one contiguous 8 KB.
    static_assert(DV == 128, "the staging layout holds 512-byte rows");
    static_assert(C::LDS_BYTES >= kWaves * 16 * DV * 4, "every wave's half rows fit in the tile buffers");
    uint8_t* const stage = smem + w * (16 * DV * 4);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // addresses computed here (see the BF16 rows below)
    const int r16 = ln & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (((ln >> 4) & 1) == half) {
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int chunk = 8 * d + 2 * i + (ln >> 5);  // channels 4 chunk .. 4 chunk + 3
            const f32x4 o4 = {wv.st.o[d][4 * i] * inv, wv.st.o[d][4 * i + 1] * inv, wv.st.o[d][4 * i + 2] * inv,
                              wv.st.o[d][4 * i + 3] * inv};
            *reinterpret_cast<f32x4*>(stage + r16 * (DV * 4) + 16 * (chunk ^ (2 * r16))) = o4;
          }
      }
      const int cc = ln & 31;  // the chunk this lane stores
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 2 * k + (ln >> 5), q = qw0 + 16 * half + row;
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(stage + row * (DV * 4) + 16 * (cc ^ (2 * row)));
        if (q < Nq) *reinterpret_cast<f32x4*>(p.ws_o + ((size_t)slot * kBM + (q - q0)) * DV + 4 * cc) = v4;
      }
    }
    barrier(false);
    return;
  }
  const float inv = sv / lsum;
  // the probabilities are 2^(x - m + SHIFT) for log2-domain scores x, so
  // log2 sum_j 2^x_j = m - SHIFT + log2(l); lanes l and l + 32 share a query
  if (p.lse != nullptr && hl == 0 && my_q < Nq)
    p.lse[((size_t)b * p.Hq + h) * Nq + my_q] = (wv.st.m - C::SHIFT + __log2f(lsum)) * 0.69314718055994531f;
  // The output rows go out through LDS.  In registers lane (query l32, half hl)
  // holds 4-channel pieces of its row, so stores straight from them cover 16
  // bytes of each of 32 rows per instruction; staged, every store writes four
  // whole 256-byte rows.  Each wave stages its 32 rows (8 KB) in a region of
  // its own, 16-byte chunk c of row r at chunk position c ^ (r & 15) (the
  // writes of a lane half and the reads of a row then spread over all banks).
  // Every tile load of the item has completed and every wave has left the
  // loop, so the tile buffers are free; the barrier at the end keeps the next
  // item's first loads and zero fill out of regions still being read.
  static_assert(DV == 128, "the staging layout holds 256-byte rows");
  static_assert(C::LDS_BYTES >= kWaves * 32 * DV * 2, "every wave's rows fit in the tile buffers");
  uint8_t* const stage = smem + w * (32 * DV * 2);
  // (the lane index passes through an empty asm so that the addresses below
  // are computed here, per item, and not hoisted out of the item loop into
  // registers that would be spilled across it)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r32 = ln & 31;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = 4 * d + i;  // channels 8 chunk .. 8 chunk + 7; this lane's half at byte 8 hl
      const i32x2 v2 = {(int)pack_bf16x2(wv.st.o[d][4 * i] * inv, wv.st.o[d][4 * i + 1] * inv),
                        (int)pack_bf16x2(wv.st.o[d][4 * i + 2] * inv, wv.st.o[d][4 * i + 3] * inv)};
      *reinterpret_cast<i32x2*>(stage + r32 * (DV * 2) + 16 * (chunk ^ (r32 & 15)) + 8 * (ln >> 5)) = v2;
    }
  {
    const int cc = ln & 15;  // the chunk this lane stores
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * r + (ln >> 4), q = qw0 + row;
      const i32x4 v4 = *reinterpret_cast<const i32x4*>(stage + row * (DV * 2) + 16 * (cc ^ (row & 15)));
      if (q < Nq)
        *reinterpret_cast<i32x4*>(static_cast<__bf16*>(p.out) + (((size_t)b * Nq + q) * p.Hq + h) * DV + 8 * cc) = v4;
    }
  }
  barrier(false);
}

// Persistent workgroups (at most one per CU) walk a static list of work units.
// A unit is a pair of query tiles of one (batch, head), the j-th from the end
// and the j-th from the start of the causal triangle, so every unit costs about
// the same and the workgroups finish together (separate per-tile workgroups
// left CUs idle between workgroups and at the tail).  When there are no more
// tiles than CUs, each workgroup takes a single tile instead (pairing would
// only serialize short work).  Workgroup w runs on XCD w % 8 (round-robin
// dispatch); when the (batch, head) count splits evenly over the 8 XCDs, XCD x
// takes the heads bh = x (mod 8) and its workgroups sweep one head at a time,
// so the K/V tiles they stream are shared in that XCD's L2.  The heavier tile of
// a unit walks its keys upward and the lighter one downward: with units of
// equal cost started together, every workgroup of an XCD then reads key tile t
// at about the same moment in both halves (time t in the heavy half, a constant
// minus t in the light half), so the workgroups stream two shared fronts of K/V
// tiles instead of one stream each.  SNAKE: the tiles dealt one by one in snake
// order of cost instead, for launches whose pairs do not split evenly over the
// workgroups.
template <int DQK, int DV, bool FP8, bool BS, int PSH, bool LEAN, bool SPLIT, bool SHORT, int NW, bool SNAKE = false>
__global__ __launch_bounds__(64 * NW, 1) void attn_fwd_kernel(AttnParams p) {
  using C = Cfg<FP8, DQK, DV, tile_keys<FP8, DQK, BS, PSH, SHORT>(), NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
  // (block scales: words for tiles 0 .. T, T = ceil(keys / BN) at most)
  __shared__ uint32_t ebuf[BS ? (C::BN == 192 ? 2 : 1) * ((kBlock64MaxKeys + C::BN - 1) / C::BN + 1) : 1];
  const int nqt = (p.Nq + 32 * NW - 1) / (32 * NW);  // work items of 32 queries per wave
  const int nbh = p.B * p.Hq;
  const int G = gridDim.x, wg = blockIdx.x;
  const bool by_xcd = (nbh % 8 == 0) && (G % 8 == 0);
  if constexpr (SPLIT) {
    // key split: one workgroup per key range, B * Hq * split_units of them; the
    // ranges of a (batch, head) are its query tiles' ranges in order
    const int L = p.split_tiles, per_bh = p.split_units;
    const int bh = by_xcd ? 8 * ((wg / 8) / per_bh) + wg % 8 : wg / per_bh;
    const int j = (by_xcd ? wg / 8 : wg) % per_bh;
    int qt = 0, r = j;
    for (; qt < nqt - 1; ++qt) {
      const int nr = (qtile_key_tiles(qt, p.Nq, p.Nk, C::BN) + L - 1) / L;
      if (r < nr) break;
      r -= nr;
    }
    const bool multi = (qtile_key_tiles(qt, p.Nq, p.Nk, C::BN) + L - 1) / L > 1;
    attn_item<DQK, DV, FP8, BS, PSH, LEAN, true, SHORT, NW>(p, smem, ebuf, bh, qt, false, r * L, r * L + L,
                                                 multi ? bh * per_bh + j : -1);
  } else if constexpr (SNAKE) {
    // The tiles sorted by cost, heaviest first (position pos: query tile
    // nqt - 1 - pos / nbh of (batch, head) pos % nbh), dealt in snake order:
    // round r gives workgroup wg position r * G + wg (r even) or
    // r * G + G - 1 - wg (r odd).  Used where heavy/light pairs would not
    // split evenly over the workgroups.  The odd rounds walk their keys
    // downward, as the lighter tile of a pair does.
    const int ntiles = nbh * nqt;
    for (int r = 0; r * G < ntiles; ++r) {
      const int pos = r * G + ((r & 1) ? G - 1 - wg : wg);
      if (pos < ntiles)
        attn_item<DQK, DV, FP8, BS, PSH, LEAN, false, SHORT, NW>(p, smem, ebuf, pos % nbh, nqt - 1 - pos / nbh,
                                                                (r & 1) != 0, 0, 0, -1);
    }
  } else {
    const bool single = (long long)nbh * nqt <= G;  // one tile per unit
    const int per_bh = single ? nqt : (nqt + 1) / 2;  // units per (batch, head)
    const int rank = by_xcd ? wg / 8 : wg, nrank = by_xcd ? G / 8 : G;
    const int nunit = by_xcd ? (nbh / 8) * per_bh : nbh * per_bh;
    // one call site (the item body is large): the two tiles of a unit are
    // iterations half = 0 (the later, heavier tile) and half = 1
    int u = rank, half = 0;
    while (u < nunit) {
      const int bh = by_xcd ? 8 * (u / per_bh) + wg % 8 : u / per_bh;
      const int j = u % per_bh;
      const int qt = half == 0 ? nqt - 1 - j : j;
      if (half == 0 || j != nqt - 1 - j)
        attn_item<DQK, DV, FP8, BS, PSH, LEAN, false, SHORT, NW>(p, smem, ebuf, bh, qt, !single && half == 1, 0, 0,
                                                                -1);
      if (single) {
        u += nrank;
      } else {
        u += half * nrank;
        half ^= 1;
      }
    }
  }
}

// Launch one variant (d_v = 128) on `grid` persistent workgroups: the split
// instantiation when the launch splits its keys, the 4-wave one when the
// launch runs 128-query items (p.solo), the snake-order one when its pairs do
// not split evenly over the workgroups (p.snake), and the short-sequence tile
// size where it differs (kShortKeys).
template <int DQK, bool FP8, bool BS, int PSH, bool LEAN, bool SHORT>
hipError_t launch_attn_tiles(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.split_tiles > 0) {
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, 128, FP8, BS, PSH, LEAN, true, SHORT, 8>), grid, dim3(512), 0, stream, p);
  } else if (p.snake) {
    // (per-head scales only: the block-scaled kernels keep the pairs, as their
    // snake-order build reloads spilled scalars in its main loop)
    if constexpr (!BS)
      hipLaunchKernelGGL((attn_fwd_kernel<DQK, 128, FP8, BS, PSH, LEAN, false, SHORT, 8, true>), grid, dim3(512), 0,
                         stream, p);
    else
      return hipErrorInvalidValue;
  } else if (p.solo) {
    // (the 4-wave mode exists for tiles of at most 128 keys; the host picks it
    // only for those)
    if constexpr (tile_keys<FP8, DQK, BS, PSH, SHORT>() <= 128)
      hipLaunchKernelGGL((attn_fwd_kernel<DQK, 128, FP8, BS, PSH, LEAN, false, SHORT, 4>), grid, dim3(256), 0, stream,
                         p);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, 128, FP8, BS, PSH, LEAN, false, SHORT, 8>), grid, dim3(512), 0, stream,
                       p);
  }
  return hipGetLastError();
}
template <int DQK, bool FP8, bool BS, int PSH, bool LEAN>
hipError_t launch_attn_variant(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if constexpr (tile_keys<FP8, DQK, BS, PSH, true>() != tile_keys<FP8, DQK, BS, PSH, false>()) {
    if (p.Nk <= kShortKeys) return launch_attn_tiles<DQK, FP8, BS, PSH, LEAN, true>(p, grid, stream);
  }
  return launch_attn_tiles<DQK, FP8, BS, PSH, LEAN, false>(p, grid, stream);
}

// The probability modes of the FP8 kernels with one scale granularity.
template <int DQK, bool BS>
hipError_t launch_attn_fp8_modes(const AttnParams& p, dim3 grid, hipStream_t stream) {
  switch (p.p_mode) {
    case kPLean: return launch_attn_variant<DQK, true, BS, kShiftNone, true>(p, grid, stream);
    case kPLeanBlock: return launch_attn_variant<DQK, true, BS, kShiftStep, true>(p, grid, stream);
    case kPLeanTile: return launch_attn_variant<DQK, true, BS, kShiftTile, true>(p, grid, stream);
    case kPExact: return launch_attn_variant<DQK, true, BS, kShiftNone, false>(p, grid, stream);
    case kPExactBlock: return launch_attn_variant<DQK, true, BS, kShiftStep, false>(p, grid, stream);
    case kPExactTile: return launch_attn_variant<DQK, true, BS, kShiftTile, false>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace miattn
