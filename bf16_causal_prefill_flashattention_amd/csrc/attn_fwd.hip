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
// Work decomposition.  One workgroup = 8 waves = 256 consecutive queries of one
// (batch, query head); each wave owns 32 queries, and two waves share each
// SIMD.  The workgroup walks key tiles (64 keys for BF16, 128 for FP8) from key
// 0 up to its last query; the causal mask is applied only on the tiles that
// cross the diagonal, and a wave skips the tiles wholly above its queries.
//
// Matrix layout.  A wave computes S^T = K_tile * Q^T (keys on MFMA rows,
// queries on MFMA columns), so lane l owns query (l % 32) and holds that
// query's scores for half of the tile's keys; the other half sits in lane
// l ^ 32.  Row max stays inside a lane plus one exchange with lane l ^ 32.  The
// output is accumulated transposed, O^T += V^T * P^T, so probabilities leave
// the S^T accumulator straight into the MFMA B operand, and V^T is read from a
// transposed LDS copy of the V tile whose key order matches the k-slots.
//
// Pipeline.  K/V tiles stream HBM/L2 -> registers -> LDS through two LDS
// stages with one barrier per tile: while tile j is consumed, tile j+1 is
// written to the other stage and tile j+2 is in flight in registers (waves 0-3
// stage V, waves 4-7 stage K).  The two waves of a SIMD run the same
// S -> softmax -> P.V sequence; while one turns scores into probabilities on
// the vector ALU, the other's matrix instructions keep the matrix core busy,
// the two-wave overlap the pages describe ([P3] "ZYFA 如何工作？").
//
// Probabilities.  The running max is only raised when a tile's max exceeds it
// by more than a small threshold, so most tiles skip the rescale of the output
// accumulator.  The row sum is taken from the rounded probabilities that feed
// the P.V product ([P3] "ZYFA 如何工作？", rounded row sums): for FP8 with one
// extra 16x16x128 MFMA per 64 keys against a 0/1 selector matrix, for BF16 with
// bf16 dot products.  FP8 probabilities are scaled by a fixed power of two
// before rounding to e4m3, which the row sum cancels.
#include "device_common.hpp"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace miattn {

namespace {

constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kHalf = kThreads / 2;
constexpr int kBM = 256;  // queries per workgroup (8 waves x 32)
constexpr int kStages = 2;

template <bool FP8, int DQK, int DV>
struct Cfg {
  static constexpr int EB = FP8 ? 1 : 2;      // bytes per element
  static constexpr int BN = FP8 ? 128 : 64;   // keys per tile
  static constexpr int NBLK = BN / 32;        // 32-key MFMA blocks per tile
  static constexpr int KROW = DQK * EB;       // bytes of one K row
  static constexpr int K_STRIDE = KROW + 16;  // LDS row pitch; +16 keeps b128 reads conflict-free
  static constexpr int VT_STRIDE = BN * EB + 16;
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int VT_BYTES = DV * VT_STRIDE;
  static constexpr int STAGE_BYTES = K_BYTES + VT_BYTES;
  static constexpr int KCH = KROW / 16;                // 16-byte chunks per K row
  static constexpr int K_TPR = kHalf / BN;             // K-staging threads per K row
  static constexpr int K_LOADS = KCH / K_TPR;          // consecutive chunks per K-staging thread
  static constexpr int VCH = DV * EB / 16;             // 16-byte channel chunks per V row
  static constexpr int NREG = K_LOADS > 4 ? K_LOADS : 4;
  static constexpr int QK_STEPS = FP8 ? DQK / 64 : DQK / 16;
  // log2-domain growth of the running max tolerated before rescaling, and the
  // power-of-two shift applied to FP8 probabilities (p <= 2^(THRESH+SHIFT) <= 256)
  static constexpr float THRESH = FP8 ? 2.0f : 8.0f;
  static constexpr float SHIFT = FP8 ? 6.0f : 0.0f;
  static_assert((BN / 4) * VCH == kHalf, "one V unit (4 keys x 16 bytes) per V-staging thread");
  static_assert(K_TPR * BN == kHalf && K_LOADS * K_TPR == KCH, "K tile splits evenly over the K-staging threads");
};

// Map the linear workgroup id to (batch*head, query tile).  Workgroups are
// dispatched round-robin over the 8 XCDs (id % 8), each XCD with its own L2;
// giving every XCD a contiguous range of work items keeps the query tiles that
// run together on an XCD on the same key/value head, so the K/V tiles they
// stream are shared in that XCD's L2.  Within a head the heaviest (latest)
// query tiles come first, so the short diagonal tiles fill the tail.
__device__ __forceinline__ void decode_item(int bid, int nblocks, int nqt, int& bh, int& qt) {
  const int xcd = bid & 7, j = bid >> 3;
  const int base = nblocks >> 3, rem = nblocks & 7;
  const int item = xcd * base + min(xcd, rem) + j;
  bh = item / nqt;
  qt = nqt - 1 - (item % nqt);
}

// Position of key k of a tile in a row of the transposed V tile (in elements).
// BF16: P.V consumes 16 keys per MFMA; lane half hl holds keys 8a + 4hl + j of
// each chunk in k-slot 4a + j, so the key's bits 2 and 3 swap.
// FP8: P.V consumes 64 keys per MFMA; lane half hl holds keys 32bb + 8i + 4hl + j
// in k-slot 16bb + 4i + j, stored at offset 32hl of the chunk.
template <bool FP8>
__device__ __forceinline__ int vt_pos(int k) {
  if constexpr (FP8)
    return (k & ~63) | (((k >> 2) & 1) << 5) | (((k >> 5) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
  else
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <class C>
struct TileRegs {
  i32x4 r[C::NREG];
};

// V-staging thread t (0..255) -> (4-key group kg, 16-byte channel chunk dc).  A
// wave covers all key groups of two (FP8) or four (BF16) channel chunks.
template <bool FP8>
__device__ __forceinline__ void v_unit(int t, int& kg, int& dc) {
  if constexpr (FP8) {
    kg = t & 31;
    dc = t >> 5;
  } else {
    kg = t & 15;
    dc = t >> 4;
  }
}

// Global -> registers.  Threads 0..255 fetch the V tile (4 keys x 16 bytes
// each), threads 256..511 the K tile.  Rows at or beyond N read as zeros
// (buffer bounds), so a ragged last tile needs no branches; keys >= N lie
// above the diagonal of every valid query and are masked later.
template <class C, bool FP8>
__device__ __forceinline__ void load_tile(TileRegs<C>& t, const uint8_t* K, const uint8_t* V, uint32_t k_pitch,
                                          uint32_t v_pitch, int kb, int N, int tid) {
  const uint32_t rows = (uint32_t)min(N - kb, C::BN);
  if (__builtin_amdgcn_readfirstlane(tid) < kHalf) {  // wave-uniform role
    const auto rv = make_rsrc(V + (size_t)kb * v_pitch, rows * v_pitch);
    int kg, dc;
    v_unit<FP8>(tid, kg, dc);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.r[i] = bload16(rv, (uint32_t)(4 * kg + i) * v_pitch + dc * 16);
  } else {
    const auto rk = make_rsrc(K + (size_t)kb * k_pitch, rows * k_pitch);
    const int tk = tid - kHalf, r = tk / C::K_TPR, ch0 = (tk % C::K_TPR) * C::K_LOADS;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) t.r[i] = bload16(rk, (uint32_t)r * k_pitch + (ch0 + i) * 16);
  }
}

// Registers -> LDS stage: K rows as they are (padded pitch), V transposed to
// channel rows with the key order of vt_pos.
template <class C, bool FP8>
__device__ __forceinline__ void store_tile(const TileRegs<C>& t, uint8_t* Ks, uint8_t* Vt, int tid) {
  if (__builtin_amdgcn_readfirstlane(tid) >= kHalf) {  // wave-uniform role
    const int tk = tid - kHalf, r = tk / C::K_TPR, ch0 = (tk % C::K_TPR) * C::K_LOADS;
    uint8_t* dst = Ks + r * C::K_STRIDE + ch0 * 16;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) lds_store16(dst + i * 16, t.r[i]);
    return;
  }
  int kg, dc;
  v_unit<FP8>(tid, kg, dc);
  const int pos = vt_pos<FP8>(4 * kg) * C::EB;
  if constexpr (FP8) {
    // dword e of each 16-byte chunk holds channels 4e..4e+3 of one key; write
    // channel rows 16dc + 4e + {0..3}, 4 keys (4 bytes) each.
    uint8_t* dst = Vt + dc * 16 * C::VT_STRIDE + pos;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x0 = (uint32_t)t.r[0][e], x1 = (uint32_t)t.r[1][e];
      const uint32_t x2 = (uint32_t)t.r[2][e], x3 = (uint32_t)t.r[3][e];
      const uint32_t t01l = perm(x1, x0, 0x05010400u), t01h = perm(x1, x0, 0x07030602u);
      const uint32_t t23l = perm(x3, x2, 0x05010400u), t23h = perm(x3, x2, 0x07030602u);
      uint8_t* row = dst + 4 * e * C::VT_STRIDE;
      lds_store4(row, (int)perm(t23l, t01l, 0x05040100u));
      lds_store4(row + C::VT_STRIDE, (int)perm(t23l, t01l, 0x07060302u));
      lds_store4(row + 2 * C::VT_STRIDE, (int)perm(t23h, t01h, 0x05040100u));
      lds_store4(row + 3 * C::VT_STRIDE, (int)perm(t23h, t01h, 0x07060302u));
    }
  } else {
    // dword e holds channels 2e, 2e+1 of one key; write channel rows
    // 8dc + 2e + {0, 1}, 4 keys (8 bytes) each.
    uint8_t* dst = Vt + dc * 8 * C::VT_STRIDE + pos;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x0 = (uint32_t)t.r[0][e], x1 = (uint32_t)t.r[1][e];
      const uint32_t x2 = (uint32_t)t.r[2][e], x3 = (uint32_t)t.r[3][e];
      uint8_t* row = dst + 2 * e * C::VT_STRIDE;
      lds_store8(row, i32x2{(int)perm(x1, x0, 0x05040100u), (int)perm(x3, x2, 0x05040100u)});
      lds_store8(row + C::VT_STRIDE, i32x2{(int)perm(x1, x0, 0x07060302u), (int)perm(x3, x2, 0x07060302u)});
    }
  }
}

template <bool FP8>
using QOperand = typename std::conditional<FP8, i32x8, bf16x8>::type;

// S^T (32 keys x 32 queries per block) = K_tile * Q^T for the first nb blocks.
template <class C, bool FP8>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[C::NBLK], const uint8_t* Ks,
                                        const QOperand<FP8> (&q)[C::QK_STEPS], int l32, int hl) {
#pragma unroll
  for (int blk = 0; blk < C::NBLK; ++blk) {
    f32x16 acc = zero16();
#pragma unroll
    for (int kk = 0; kk < C::QK_STEPS; ++kk) {
      if constexpr (FP8) {
        const uint8_t* src = Ks + (blk * 32 + l32) * C::K_STRIDE + kk * 64 + hl * 32;
        const i32x4 lo = lds_load16(src), hi = lds_load16(src + 16);
        const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc = mfma_fp8_32x32x64(a, q[kk], acc);
      } else {
        const i32x4 a = lds_load16(Ks + (blk * 32 + l32) * C::K_STRIDE + kk * 32 + hl * 16);
        acc = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), q[kk], acc);
      }
    }
    s[blk] = acc;
  }
}

// Running state of one wave's 32 queries.
template <int DV>
struct RowState {
  f32x16 o[DV / 32];  // O^T accumulator: lane owns query l % 32, channels 32d + 8i + 4hl + j
  float m;            // running max, log2 domain
  float l;            // BF16: this lane's share of the row sum
  f32x4 l4;           // FP8: the full row sum (every entry)
};

// Online softmax of one tile and the P.V product.  MASK: the tile crosses the
// diagonal (keys above a query are set to -inf first).
template <class C, bool FP8, bool MASK, int DV>
__device__ __forceinline__ void softmax_pv(f32x16 (&s)[C::NBLK], RowState<DV>& st, const uint8_t* Vt, float c,
                                           int key_minus_query, int l32, int hl, const i32x8& sel) {
  constexpr int NBLK = C::NBLK;
  if constexpr (MASK) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key_minus_query + blk * 32 + 8 * (r >> 2) + (r & 3) > 0) s[blk][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[blk][r], s[blk][r + 1]));
  mx = fmaxf(mx, xor32(mx));
  const float mt = mx * c;
  if (__any(mt > st.m + C::THRESH)) {  // wave-uniform; rare once the max settles
    const float m_new = fmaxf(st.m, mt);
    const float alpha = fast_exp2(st.m - m_new);
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) st.o[d] *= alpha;
    st.l *= alpha;
    st.l4 *= alpha;
    st.m = m_new;
  }
  const float bias = C::SHIFT - st.m;

  if constexpr (FP8) {
#pragma unroll
    for (int ks = 0; ks < C::BN / 64; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      uint32_t pk[8];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float e[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) e[jj] = fast_exp2(__builtin_fmaf(s[2 * ks + hb][4 * i + jj], c, bias));
          pk[4 * hb + i] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
      const i32x8 pb = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                        (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
      st.l4 = mfma_fp8_16x16x128(sel, pb, st.l4);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) {
        const uint8_t* src = Vt + (d * 32 + l32) * C::VT_STRIDE + ks * 64 + hl * 32;
        const i32x4 lo = lds_load16(src), hi = lds_load16(src + 16);
        const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        st.o[d] = mfma_fp8_32x32x64(a, pb, st.o[d]);
      }
    }
  } else {
    const uint32_t ones = 0x3f803f80u;  // two bf16 1.0
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        __builtin_amdgcn_sched_barrier(0);
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * half + 2 * i;
          const float p0 = fast_exp2(__builtin_fmaf(s[blk][r], c, bias));
          const float p1 = fast_exp2(__builtin_fmaf(s[blk][r + 1], c, bias));
          pk[i] = pack_bf16x2(p0, p1);
          st.l = dot2_bf16(pk[i], ones, st.l);
        }
        const i32x4 pw = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const int chunk = 2 * blk + half;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const i32x4 a = lds_load16(Vt + (d * 32 + l32) * C::VT_STRIDE + chunk * 32 + hl * 16);
          st.o[d] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), pb, st.o[d]);
        }
      }
  }
}

template <int DQK, int DV, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(AttnParams p) {
  using C = Cfg<FP8, DQK, DV>;
  constexpr int NBLK = C::NBLK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * C::STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int N = p.N;
  const int nqt = (N + kBM - 1) / kBM;
  int bh, qt;
  decode_item(blockIdx.x, gridDim.x, nqt, bh, qt);
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / (p.Hq / p.Hkv);
  const int q0 = qt * kBM;
  const int qw0 = q0 + 32 * w;  // first query of this wave
  const int my_q = qw0 + l32;   // query owned by this lane

  const size_t q_pitch = (size_t)p.Hq * C::KROW;  // bytes between consecutive positions
  const uint32_t k_pitch = (uint32_t)p.Hkv * C::KROW;  // the host bounds Hkv * d * bytes per element
  const uint32_t v_pitch = (uint32_t)p.Hkv * DV * C::EB;
  const uint8_t* Q = static_cast<const uint8_t*>(p.q) + ((size_t)b * N * p.Hq + h) * C::KROW;
  const uint8_t* K = static_cast<const uint8_t*>(p.k) + ((size_t)b * N * p.Hkv + g) * C::KROW;
  const uint8_t* V = static_cast<const uint8_t*>(p.v) + ((size_t)b * N * p.Hkv + g) * DV * C::EB;

  float c = p.sm_scale_log2;  // log2-domain score scale (dequantisation folded in for FP8)
  float sv = 1.f;
  if constexpr (FP8) {
    c *= p.q_scale[b * p.Hq + h] * p.k_scale[b * p.Hkv + g];
    sv = p.v_scale[b * p.Hkv + g];
  }

  // Q^T operand in registers.  BF16: k-step kk = channels [16kk, 16kk+16), lane
  // half hl holds 8 of them; FP8: k-step kk = channels [64kk, 64kk+64), 32 each.
  QOperand<FP8> qreg[C::QK_STEPS];
#pragma unroll
  for (int kk = 0; kk < C::QK_STEPS; ++kk) {
    if constexpr (FP8) {
      const uint8_t* src = Q + (size_t)my_q * q_pitch + kk * 64 + hl * 32;
      const i32x4 lo = gload16(src, my_q < N), hi = gload16(src + 16, my_q < N);
      qreg[kk] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      qreg[kk] = __builtin_bit_cast(bf16x8, gload16(Q + (size_t)my_q * q_pitch + kk * 32 + hl * 16, my_q < N));
    }
  }

  const int kend = min(q0 + kBM, N);
  const int ntiles = (kend + C::BN - 1) / C::BN;
  const int first_diag = q0 / C::BN;  // tiles from here on may hold keys above the diagonal

  // Prologue: tile 0 into LDS stage 0, tile 1 in flight in registers.
  TileRegs<C> pre;
  load_tile<C, FP8>(pre, K, V, k_pitch, v_pitch, 0, N, tid);
  store_tile<C, FP8>(pre, smem, smem + C::K_BYTES, tid);
  if (ntiles > 1) load_tile<C, FP8>(pre, K, V, k_pitch, v_pitch, C::BN, N, tid);

  RowState<DV> st;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) st.o[d] = zero16();
  st.m = -1e30f;
  st.l = 0.f;
  st.l4 = f32x4{0.f, 0.f, 0.f, 0.f};
  // FP8 row-sum selector: 16x16x128 A operand, 1.0 where the lane group's
  // parity matches its row group's parity, else 0.
  const int sel_on = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? 0x38383838 : 0;
  const i32x8 sel = {sel_on, sel_on, sel_on, sel_on, sel_on, sel_on, sel_on, sel_on};

  // One tile; the LDS stage is a compile-time constant so every LDS access is a
  // per-lane base plus an immediate offset.
  auto tile_step = [&](int j, auto stage_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    uint8_t* const cur_k = smem + S * C::STAGE_BYTES;
    uint8_t* const cur_v = cur_k + C::K_BYTES;
    uint8_t* const nxt_k = smem + (1 - S) * C::STAGE_BYTES;
    uint8_t* const nxt_v = nxt_k + C::K_BYTES;
    __syncthreads();  // tile j is visible; every wave is done with tile j-1
    if (j + 1 < ntiles) store_tile<C, FP8>(pre, nxt_k, nxt_v, tid);
    if (j + 2 < ntiles) load_tile<C, FP8>(pre, K, V, k_pitch, v_pitch, (j + 2) * C::BN, N, tid);

    const int kb = j * C::BN;
    if (kb > qw0 + 31) return;  // the whole tile lies above this wave's queries
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s[NBLK];
    qk_tile<C, FP8>(s, cur_k, qreg, l32, hl);
    __builtin_amdgcn_sched_barrier(0);
    if (j < first_diag)
      softmax_pv<C, FP8, false, DV>(s, st, cur_v, c, 0, l32, hl, sel);
    else
      softmax_pv<C, FP8, true, DV>(s, st, cur_v, c, kb + 4 * hl - my_q, l32, hl, sel);
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile_step(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntiles) tile_step(j + 1, std::integral_constant<int, 1>{});
  }

  // Epilogue: normalise by the row sum and store BF16.
  float inv;
  if constexpr (FP8) {
    inv = sv / st.l4[0];
  } else {
    inv = 1.0f / (st.l + xor32(st.l));
  }
  if (my_q < N) {
    __bf16* O = static_cast<__bf16*>(p.out) + (((size_t)b * N + my_q) * p.Hq + h) * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = d * 32 + 8 * i + 4 * hl;
        const i32x2 v2 = {(int)pack_bf16x2(st.o[d][4 * i] * inv, st.o[d][4 * i + 1] * inv),
                          (int)pack_bf16x2(st.o[d][4 * i + 2] * inv, st.o[d][4 * i + 3] * inv)};
        *reinterpret_cast<i32x2*>(O + ch) = v2;
      }
    }
  }
}

}  // namespace

int attn_fwd_workgroups(int B, int Hq, int N) {
  const long long nqt = (N + kBM - 1) / kBM;
  const long long n = (long long)B * Hq * nqt;
  return n > 0x7fffffffLL ? -1 : (int)n;
}

hipError_t launch_attn_fwd(const AttnParams& p, int dtype, int d_qk, int d_v, hipStream_t stream) {
  const int grid = attn_fwd_workgroups(p.B, p.Hq, p.N);
  if (grid <= 0) return hipErrorInvalidValue;
  const dim3 g(grid), blk(kThreads);
  if (d_v != 128) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (d_qk == 128)
      hipLaunchKernelGGL((attn_fwd_kernel<128, 128, false>), g, blk, 0, stream, p);
    else if (d_qk == 192)
      hipLaunchKernelGGL((attn_fwd_kernel<192, 128, false>), g, blk, 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (d_qk == 128)
      hipLaunchKernelGGL((attn_fwd_kernel<128, 128, true>), g, blk, 0, stream, p);
    else if (d_qk == 192)
      hipLaunchKernelGGL((attn_fwd_kernel<192, 128, true>), g, blk, 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace miattn
