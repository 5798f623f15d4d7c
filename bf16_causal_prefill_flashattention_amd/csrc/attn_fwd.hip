// Causal forward (prefill) attention for gfx950: O = softmax(Q K^T tau + mask) V.
//
// Page legend: [P1] "Zyphra ZYFA: 1.76x FP8 FlashAttention Speedup on AMD
// MI355X"; [P3] "Zyphra 开源 ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速
// 1.76 倍".
//
// What is computed: exact causal softmax attention, evaluated tile by tile with
// an online softmax so the N x N score matrix never reaches HBM ([P1] "Why
// prefill attention deserves dedicated optimization").  FP8 e4m3 inputs carry
// per-(batch, head) fp32 scales that are folded in before the softmax; both
// matrix products accumulate in FP32 ([P1] "ZYFA's performance and accuracy
// data"; [P3] "为什么 FP8 注意力在 MI355X 上表现不佳？").  Output is BF16.
//
// Work decomposition.  One workgroup = NW waves = 32*NW consecutive queries of
// one (batch, query head).  Each wave owns 32 queries.  The workgroup walks key
// tiles of BN keys from key 0 up to its last query; tiles wholly above a
// wave's queries are skipped by that wave, and the causal mask is applied only
// on tiles that cross the diagonal.
//
// Matrix layout.  The wave computes S^T = K_tile * Q^T (keys on MFMA rows,
// queries on MFMA columns), so lane l owns query (l % 32) and holds that
// query's scores for half of the tile's keys; the other half sits in lane
// l ^ 32.  Row max and row sum therefore stay inside a lane plus one exchange
// with lane l ^ 32.  The output is accumulated transposed, O^T += V^T * P^T,
// so the probabilities leave the S^T accumulator straight into the MFMA B
// operand with no data movement, and V^T is read from a transposed LDS copy of
// the V tile whose key order matches the lanes' k-slots.
#include "device_common.hpp"
#include "kernels.h"

#include <math.h>

namespace miattn {

namespace {

constexpr int kThreads = 256;
constexpr int kNW = kThreads / kWave;  // waves per workgroup
constexpr int kBM = 32 * kNW;          // queries per workgroup

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

// ---------------------------------------------------------------------------
// BF16 kernel: BN = 64 keys per tile.
// ---------------------------------------------------------------------------
template <int DQK, int DV>
struct Bf16Cfg {
  static constexpr int BN = 64;
  static constexpr int K_STRIDE = DQK * 2 + 16;  // bytes; +16 keeps b128 LDS reads conflict-free
  static constexpr int VT_STRIDE = BN * 2 + 16;
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int VT_BYTES = DV * VT_STRIDE;
};

// Position of key k (0..63 inside the tile) in a row of the transposed V tile.
// The PV product consumes keys in chunks of 16; in S^T lane half hl holds the
// keys 8a + 4hl + j (a, j bits) of each chunk in k-slot 4a + j, so the slot
// order within a chunk is the key order with bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos_bf16(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(AttnParams p) {
  using C = Bf16Cfg<DQK, DV>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::K_BYTES + C::VT_BYTES];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + C::K_BYTES;

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

  const size_t q_row = (size_t)p.Hq * DQK;
  const size_t k_row = (size_t)p.Hkv * DQK;
  const size_t v_row = (size_t)p.Hkv * DV;
  const __bf16* Q = static_cast<const __bf16*>(p.q) + ((size_t)b * N * p.Hq + h) * DQK;
  const __bf16* K = static_cast<const __bf16*>(p.k) + ((size_t)b * N * p.Hkv + g) * DQK;
  const __bf16* V = static_cast<const __bf16*>(p.v) + ((size_t)b * N * p.Hkv + g) * DV;

  // Q^T operand, kept in registers: k-step kk covers channels [16kk, 16kk+16);
  // lane half hl holds channels 16kk + 8hl .. +8 of query my_q.
  bf16x8 qreg[DQK / 16];
#pragma unroll
  for (int kk = 0; kk < DQK / 16; ++kk) {
    i32x4 x = gload16(Q + (size_t)my_q * q_row + kk * 16 + hl * 8, my_q < N);
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = zero16();
  float m_run = -1e30f;  // running max of the log2-domain scores
  float l_run = 0.f;     // running sum of this lane's probabilities
  const float c = p.sm_scale_log2;

  const int kend = min(q0 + kBM, N);
  const int ntiles = (kend + BN - 1) / BN;
  const int wave_qmax = qw0 + 31;

  for (int j = 0; j < ntiles; ++j) {
    const int kb = j * BN;
    __syncthreads();  // every wave is done with the previous tile
    {
      constexpr int KCH = DQK * 2 / 16;
      for (int cidx = tid; cidx < BN * KCH; cidx += kThreads) {
        const int r = cidx / KCH, ch = cidx % KCH, key = kb + r;
        i32x4 x = gload16(reinterpret_cast<const uint8_t*>(K + (size_t)key * k_row) + ch * 16, key < N);
        lds_store16(Ks + r * C::K_STRIDE + ch * 16, x);
      }
      constexpr int VCH = DV / 8;
      for (int cidx = tid; cidx < (BN / 4) * VCH; cidx += kThreads) {
        const int dc = cidx % VCH, kg = cidx / VCH;
        i32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 4 * kg + i;
          x[i] = gload16(V + (size_t)key * v_row + dc * 8, key < N);
        }
        const int pos = vt_pos_bf16(4 * kg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo01 = perm(x[1][e], x[0][e], 0x05040100u);
          const uint32_t lo23 = perm(x[3][e], x[2][e], 0x05040100u);
          const uint32_t hi01 = perm(x[1][e], x[0][e], 0x07060302u);
          const uint32_t hi23 = perm(x[3][e], x[2][e], 0x07060302u);
          lds_store8(Vt + (dc * 8 + 2 * e) * C::VT_STRIDE + pos * 2, i32x2{(int)lo01, (int)lo23});
          lds_store8(Vt + (dc * 8 + 2 * e + 1) * C::VT_STRIDE + pos * 2, i32x2{(int)hi01, (int)hi23});
        }
      }
    }
    __syncthreads();

    // Number of 32-key blocks of this tile that hold a key visible to the wave.
    const int nblk = wave_qmax < kb ? 0 : min(BN / 32, (wave_qmax - kb) / 32 + 1);
    f32x16 s[BN / 32];
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
      s[blk] = zero16();
      if (blk < nblk) {
#pragma unroll
        for (int kk = 0; kk < DQK / 16; ++kk) {
          i32x4 a = lds_load16(Ks + (blk * 32 + l32) * C::K_STRIDE + (kk * 16 + hl * 8) * 2);
          s[blk] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), qreg[kk], s[blk]);
        }
      }
    }

    // Online softmax in the log2 domain.
    const bool diag = kb + BN - 1 > qw0;
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + blk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float x = s[blk][r];
        if (blk >= nblk || (diag && key > my_q)) x = -INFINITY;
        s[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    uint32_t pk[BN / 32][8];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[blk][r], c, -m_new));
        const float p1 = fast_exp2(__builtin_fmaf(s[blk][r + 1], c, -m_new));
        psum += p0 + p1;
        pk[blk][r >> 1] = pack_bf16x2(p0, p1);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;

#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
      if (blk < nblk) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int chunk = 2 * blk + half;
          i32x4 pw = {(int)pk[blk][4 * half], (int)pk[blk][4 * half + 1], (int)pk[blk][4 * half + 2],
                      (int)pk[blk][4 * half + 3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
          for (int d = 0; d < DV / 32; ++d) {
            i32x4 a = lds_load16(Vt + (d * 32 + l32) * C::VT_STRIDE + (chunk * 16 + hl * 8) * 2);
            o[d] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), pb, o[d]);
          }
        }
      }
    }
  }

  // Epilogue: combine the two lane halves' partial sums, normalise, store BF16.
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.0f / l_tot;
  if (my_q < N) {
    __bf16* O = static_cast<__bf16*>(p.out) + (((size_t)b * N + my_q) * p.Hq + h) * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = d * 32 + 8 * i + 4 * hl;
        i32x2 v2 = {(int)pack_bf16x2(o[d][4 * i] * inv, o[d][4 * i + 1] * inv),
                    (int)pack_bf16x2(o[d][4 * i + 2] * inv, o[d][4 * i + 3] * inv)};
        *reinterpret_cast<i32x2*>(O + ch) = v2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 e4m3 kernel: BN = 128 keys per tile (the 32-query x 128-key wave tile of
// [P3] "为什么 FP8 注意力在 MI355X 上表现不佳？").
// ---------------------------------------------------------------------------
template <int DQK, int DV>
struct Fp8Cfg {
  static constexpr int BN = 128;
  static constexpr int K_STRIDE = DQK + 16;
  static constexpr int VT_STRIDE = BN + 16;
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int VT_BYTES = DV * VT_STRIDE;
};

// Probabilities are scaled by 2^8 before rounding to e4m3 so that small ones
// stay out of the subnormal range; the factor cancels against the row sum.
constexpr float kFp8PShift = 8.0f;

// Position of key k (0..127) in a row of the transposed FP8 V tile.  The PV
// product consumes 64 keys per MFMA; lane half hl holds the keys
// 32*bb + 8*i + 4*hl + j (bb, i, j bits) in k-slot 16*bb + 4*i + j, and its 32
// slots are stored contiguously at offset 32*hl of the 64-key chunk.
__device__ __forceinline__ int vt_pos_fp8(int k) {
  return (k & ~63) | (((k >> 2) & 1) << 5) | (((k >> 5) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_kernel(AttnParams p) {
  using C = Fp8Cfg<DQK, DV>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::K_BYTES + C::VT_BYTES];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + C::K_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int N = p.N;
  const int nqt = (N + kBM - 1) / kBM;
  int bh, qt;
  decode_item(blockIdx.x, gridDim.x, nqt, bh, qt);
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / (p.Hq / p.Hkv);
  const int q0 = qt * kBM;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + l32;

  const size_t q_row = (size_t)p.Hq * DQK;
  const size_t k_row = (size_t)p.Hkv * DQK;
  const size_t v_row = (size_t)p.Hkv * DV;
  const uint8_t* Q = static_cast<const uint8_t*>(p.q) + ((size_t)b * N * p.Hq + h) * DQK;
  const uint8_t* K = static_cast<const uint8_t*>(p.k) + ((size_t)b * N * p.Hkv + g) * DQK;
  const uint8_t* V = static_cast<const uint8_t*>(p.v) + ((size_t)b * N * p.Hkv + g) * DV;

  // Dequantisation folded into the log2-domain score scale.
  const float sq = p.q_scale[b * p.Hq + h];
  const float sk = p.k_scale[b * p.Hkv + g];
  const float sv = p.v_scale[b * p.Hkv + g];
  const float c = p.sm_scale_log2 * sq * sk;

  // Q^T operand: k-step kk covers channels [64kk, 64kk+64); lane half hl holds
  // channels 64kk + 32hl .. +32.
  i32x8 qreg[DQK / 64];
#pragma unroll
  for (int kk = 0; kk < DQK / 64; ++kk) {
    const uint8_t* src = Q + (size_t)my_q * q_row + kk * 64 + hl * 32;
    i32x4 lo = gload16(src, my_q < N), hi = gload16(src + 16, my_q < N);
    qreg[kk] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = zero16();
  float m_run = -1e30f;
  float l_run = 0.f;

  const int kend = min(q0 + kBM, N);
  const int ntiles = (kend + BN - 1) / BN;
  const int wave_qmax = qw0 + 31;

  for (int j = 0; j < ntiles; ++j) {
    const int kb = j * BN;
    __syncthreads();
    {
      constexpr int KCH = DQK / 16;
      for (int cidx = tid; cidx < BN * KCH; cidx += kThreads) {
        const int r = cidx / KCH, ch = cidx % KCH, key = kb + r;
        i32x4 x = gload16(K + (size_t)key * k_row + ch * 16, key < N);
        lds_store16(Ks + r * C::K_STRIDE + ch * 16, x);
      }
      constexpr int VCH = DV / 16;
      for (int cidx = tid; cidx < (BN / 4) * VCH; cidx += kThreads) {
        const int dc = cidx % VCH, kg = cidx / VCH;
        i32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 4 * kg + i;
          x[i] = gload16(V + (size_t)key * v_row + dc * 16, key < N);
        }
        const int pos = vt_pos_fp8(4 * kg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t t01l = perm(x[1][e], x[0][e], 0x05010400u);
          const uint32_t t01h = perm(x[1][e], x[0][e], 0x07030602u);
          const uint32_t t23l = perm(x[3][e], x[2][e], 0x05010400u);
          const uint32_t t23h = perm(x[3][e], x[2][e], 0x07030602u);
          uint8_t* row = Vt + (dc * 16 + 4 * e) * C::VT_STRIDE + pos;
          lds_store4(row, (int)perm(t23l, t01l, 0x05040100u));
          lds_store4(row + C::VT_STRIDE, (int)perm(t23l, t01l, 0x07060302u));
          lds_store4(row + 2 * C::VT_STRIDE, (int)perm(t23h, t01h, 0x05040100u));
          lds_store4(row + 3 * C::VT_STRIDE, (int)perm(t23h, t01h, 0x07060302u));
        }
      }
    }
    __syncthreads();

    const int nblk = wave_qmax < kb ? 0 : min(BN / 32, (wave_qmax - kb) / 32 + 1);
    f32x16 s[BN / 32];
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
      s[blk] = zero16();
      if (blk < nblk) {
#pragma unroll
        for (int kk = 0; kk < DQK / 64; ++kk) {
          const uint8_t* src = Ks + (blk * 32 + l32) * C::K_STRIDE + kk * 64 + hl * 32;
          i32x4 lo = lds_load16(src), hi = lds_load16(src + 16);
          i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          s[blk] = mfma_fp8_32x32x64(a, qreg[kk], s[blk]);
        }
      }
    }

    const bool diag = kb + BN - 1 > qw0;
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + blk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float x = s[blk][r];
        if (blk >= nblk || (diag && key > my_q)) x = -INFINITY;
        s[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    const float bias = kFp8PShift - m_new;

    uint32_t pk[BN / 32][4];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) e[jj] = fast_exp2(__builtin_fmaf(s[blk][4 * i + jj], c, bias));
        psum += (e[0] + e[1]) + (e[2] + e[3]);
        pk[blk][i] = pack_fp8x4(e[0], e[1], e[2], e[3]);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;

#pragma unroll
    for (int ks = 0; ks < BN / 64; ++ks) {
      if (2 * ks < nblk) {
        i32x8 pb = {(int)pk[2 * ks][0],     (int)pk[2 * ks][1],     (int)pk[2 * ks][2],     (int)pk[2 * ks][3],
                    (int)pk[2 * ks + 1][0], (int)pk[2 * ks + 1][1], (int)pk[2 * ks + 1][2], (int)pk[2 * ks + 1][3]};
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const uint8_t* src = Vt + (d * 32 + l32) * C::VT_STRIDE + ks * 64 + hl * 32;
          i32x4 lo = lds_load16(src), hi = lds_load16(src + 16);
          i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[d] = mfma_fp8_32x32x64(a, pb, o[d]);
        }
      }
    }
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = sv / l_tot;
  if (my_q < N) {
    __bf16* O = static_cast<__bf16*>(p.out) + (((size_t)b * N + my_q) * p.Hq + h) * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = d * 32 + 8 * i + 4 * hl;
        i32x2 v2 = {(int)pack_bf16x2(o[d][4 * i] * inv, o[d][4 * i + 1] * inv),
                    (int)pack_bf16x2(o[d][4 * i + 2] * inv, o[d][4 * i + 3] * inv)};
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
  if (dtype == 0) {
    if (d_qk == 128 && d_v == 128)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 128>), g, blk, 0, stream, p);
    else if (d_qk == 192 && d_v == 128)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, 128>), g, blk, 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (d_qk == 128 && d_v == 128)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, 128>), g, blk, 0, stream, p);
    else if (d_qk == 192 && d_v == 128)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, 128>), g, blk, 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace miattn
