/* miattn -- causal forward (prefill) attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmiattn.so.  Plain pointers and sizes only; every device pointer
 * is a HIP device address owned by the caller.  The library never allocates,
 * frees or synchronises: all work is enqueued on the caller's stream and the
 * calls return as soon as it is enqueued.  Arguments are validated on the host
 * before anything is enqueued, so a call that returns an error has launched
 * nothing.  No C++ exception crosses this interface.  The only state the
 * library keeps is a per-device cache of the compute-unit count (atomic);
 * calls are reentrant and may come from several host threads.
 *
 * Page legend for the citations:
 *   [P1] "Zyphra ZYFA: 1.76x FP8 FlashAttention Speedup on AMD MI355X"
 *   [P2] "Zyphra Says Its AMD MI355X Attention Kernel Is 1.76x Faster"
 *   [P3] "Zyphra 开源 ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速 1.76 倍"
 */
#ifndef MIATTN_H_
#define MIATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIATTN_ABI_VERSION 7

/* Element types of Q, K, V. */
#define MIATTN_DTYPE_BF16 0     /* bfloat16 */
#define MIATTN_DTYPE_FP8_E4M3 1 /* OCP FP8 e4m3fn codes, one byte each, with fp32 scales */

/* Element types accepted by attn_quantize_fp8. */
#define MIATTN_SRC_FP32 0
#define MIATTN_SRC_BF16 1

/* Status codes (0 = success, negative = error; nothing was enqueued). */
#define MIATTN_OK 0
#define MIATTN_ERR_NULL (-1)     /* a required pointer is NULL */
#define MIATTN_ERR_SIZE (-2)     /* a size is negative, zero where it may not be, Hq % Hkv != 0, Nq > Nk, or too large */
#define MIATTN_ERR_SHAPE (-3)    /* unsupported head dimensions */
#define MIATTN_ERR_DTYPE (-4)    /* unknown dtype / source type code, or a flag outside {0, 1} */
#define MIATTN_ERR_HIP (-5)      /* the HIP runtime reported an error when enqueuing */
#define MIATTN_ERR_ALIGN (-6)    /* a tensor pointer is not 16-byte aligned (scales, lse: 4-byte) */
#define MIATTN_ERR_VALUE (-7)    /* a scalar argument is out of range (softmax scale) */
#define MIATTN_ERR_SCRATCH (-8)  /* attn_fwd_noalloc: the launch needs more than the static scratch holds */

/* Causal forward attention, O = softmax(tau * Q K^T + causal mask) V.
 *
 * Defines: the causal forward (prefill) attention pass in BF16 and FP8 e4m3
 * with FP32 accumulation ([P2] "What Zyphra Reported"; [P3] "TL;DR"),
 * computed tile by tile with an online softmax so the N x N score matrix is
 * never stored ([P1] "Why prefill attention deserves dedicated
 * optimization"); head dim 128 (with grouped-query attention) and the
 * multi-head-latent shape d_qk = 192, d_v = 128 ([P2] "What Zyphra Reported").
 *
 * Layout: every tensor is contiguous [batch, sequence, head, channel] (BSHD):
 *   q   [B, N, Hq,  d_qk]  dtype
 *   k   [B, N, Hkv, d_qk]  dtype
 *   v   [B, N, Hkv, d_v]   dtype
 *   out [B, N, Hq,  d_v]   bfloat16 (written)
 * Query i attends to keys j <= i (queries and keys share positions 0..N-1).
 * Query head h reads key/value head h / (Hq / Hkv) (integer division).
 * Softmax scale tau = 1 / sqrt(d_qk).
 *
 * dtype = MIATTN_DTYPE_FP8_E4M3: q, k, v hold e4m3fn codes and the real input
 * is code * scale with one fp32 scale per (batch, head):
 *   q_scale [B, Hq], k_scale [B, Hkv], v_scale [B, Hkv]   (device memory)
 * The scales are folded into the scores before the softmax and into the
 * output; probabilities are rounded to e4m3 for the P.V product with lean P
 * against each key tile's own maximum (MIATTN_P_DEFAULT, see attn_fwd_fp8),
 * so keys are lost only about 12 octaves below the maximum of their own tile.
 * dtype = MIATTN_DTYPE_BF16: the scale pointers are ignored and may be NULL.
 *
 * Sizes: B >= 0, N >= 0 (B == 0 or N == 0 is an empty call: success, nothing
 * enqueued), Hq >= 1, Hkv >= 1, Hq % Hkv == 0, (d_qk, d_v) in
 * {(128, 128), (192, 128)}.  Any N is accepted (ragged tails are masked).
 * stream: a hipStream_t, or NULL for the default stream.
 * The result is bitwise reproducible from launch to launch on one device (no
 * atomics, fixed reduction order); the order in which a query row meets its
 * key tiles follows the work schedule, which depends on the device's compute
 * unit count, so another device may differ in the last bits.
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d_qk,
             int d_v, int dtype, const float* q_scale, const float* k_scale, const float* v_scale, void* stream);

/* One chunk of a chunked causal prefill: the last Nq positions of a sequence
 * attend to its first Nk keys and values (Nq <= Nk), with an optional
 * log-sum-exp output and an explicit softmax scale.
 *
 * Defines: the same causal attention as attn_fwd (see there for the pages'
 * passages), with the queries placed after a prefix of Nk - Nq keys that they
 * all see.  The pages stop at plain causal prefill; this entry point is the
 * step beside it that lets a long prefill run in chunks against the keys and
 * values already computed, and lets partial results over separate key ranges
 * be combined through their log-sum-exp.
 *
 * Layout (contiguous BSHD, as attn_fwd):
 *   q   [B, Nq, Hq,  d_qk]  dtype       query row i is sequence position i + Nk - Nq
 *   k   [B, Nk, Hkv, d_qk]  dtype
 *   v   [B, Nk, Hkv, d_v]   dtype
 *   out [B, Nq, Hq,  d_v]   bfloat16 (written)
 *   lse [B, Hq, Nq]         fp32 (written unless NULL):
 *        lse[b, h, i] = ln sum_{j <= i + Nk - Nq} exp(tau * <q_i, k_j>),
 *        on the dequantized inputs for FP8.
 * Query row i attends to keys j <= i + Nk - Nq.  Nq == Nk with lse == NULL and
 * softmax_scale == 0 is exactly attn_fwd.
 * softmax_scale: tau; 0 selects 1 / sqrt(d_qk); otherwise it must be finite
 * and positive (else MIATTN_ERR_VALUE).
 * Scales, dtypes, head dimensions, stream and determinism as for attn_fwd.
 * Sizes: B >= 0, 0 <= Nq <= Nk, Hq >= 1, Hkv >= 1, Hq % Hkv == 0; B == 0 or
 * Nq == 0 is an empty call (success, nothing enqueued).
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_chunk(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                   const float* v_scale, float softmax_scale, void* stream);

/* Per-(batch, head) FP8 e4m3fn quantization, the front end of the FP8 path.
 *
 * Defines: per-head scale factors that bring activations into the e4m3 range
 * ([P1] "ZYFA's performance and accuracy data"), scale = amax / 448; with
 * hadamard = 1 a 128-point Hadamard rotation of the channel dimension first,
 * which the pages apply to Q and K to cut quantization error ([P3] "ZYFA 的
 * FP8 注意力有多准确？"; [P2] "Accuracy and Code").
 *
 * x      [B, N, H, d] contiguous, fp32 (x_dtype = MIATTN_SRC_FP32) or bf16
 *        (MIATTN_SRC_BF16), read only.
 * x_fp8  [B, N, H, d] contiguous uint8, written with the e4m3fn codes.
 * scale  [B, H] fp32, written with the per-(batch, head) scale; it is also used
 *        as the amax accumulator while the call's kernels run, so it must not
 *        alias x or x_fp8.
 * Steps, each in fp32: y = x, or with hadamard = 1 the unnormalised Sylvester
 * transform of the channels (d = 128: x H_128, butterfly stages of width 1, 2,
 * ..., 64; d = 192: H_64 on each of the three groups of 64 channels, stages
 * 1, ..., 32 -- the pages show the rotation at d = 128 only);
 * amax = max |y| over the (b, h) slice; inv = 448 / amax; code =
 * round-to-nearest-even e4m3(clamp(y * inv, -448, 448)); scale = amax / 448,
 * times the normalisation when hadamard = 1 (fp32(2^-3.5) for d = 128, 2^-3
 * for d = 192).  amax == 0 gives inv = 1, scale = 1 (times the normalisation
 * with hadamard), all codes 0.  The dequantized value code * scale is what
 * attn_fwd consumes.
 * Sizes: B >= 0, N >= 0, H >= 1, d in {128, 192}; hadamard in {0, 1}.
 * B == 0 is an empty call; N == 0 writes the scales only.  Deterministic.
 * Returns MIATTN_OK or MIATTN_ERR_*. */
int attn_quantize_fp8(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N, int d,
                      int hadamard, void* stream);

/* Per-64-position FP8 e4m3fn quantization with power-of-two scales.
 *
 * Defines: the finer scaling granularity the pages name as a lever on FP8
 * accuracy ([P1] "ZYFA's performance and accuracy data": per-tensor or
 * per-head scales, block-wise scaling, scaling granularity): one scale per
 * (batch, head, block of 64 consecutive positions).  The scales are powers of
 * two, the form the scaled matrix instructions of CDNA4 apply exactly, so
 * attn_fwd_block64 applies the K and V block scales inside its MFMAs.
 *
 * x      [B, N, H, d] contiguous, fp32 (MIATTN_SRC_FP32) or bf16
 *        (MIATTN_SRC_BF16), read only.
 * x_fp8  [B, N, H, d] contiguous uint8, written with the e4m3fn codes.
 * scale  [B, H, ceil(N / 64)] fp32, written: scale[b, h, j] = 2^e covers
 *        positions 64j .. 64j + 63 (the last block may be shorter).
 * Steps, each in fp32: z = x, or with hadamard = 1 z = (x H) * norm with the
 * rotation and normalisation of attn_quantize_fp8 (the normalisation goes into
 * the values: a power of two cannot hold 2^-3.5); amax = max |z| over the
 * block; e = the smallest integer with amax <= 448 * 2^e, but at least -126
 * (e = 0 when amax == 0); code = round-to-nearest-even e4m3(z * 2^-e), which
 * never exceeds 448.  The dequantized value is code * scale[b, h, n / 64].
 * Sizes as attn_quantize_fp8 (d in {128, 192}, hadamard in {0, 1}); B == 0
 * or N == 0 is an empty call.  x is read once.  Deterministic.
 * Returns MIATTN_OK or MIATTN_ERR_*. */
int attn_quantize_fp8_block64(const void* x, int x_dtype, void* x_fp8, float* scale, int B, int H, int N, int d,
                              int hadamard, void* stream);

/* FP8 causal attention with per-64-position scales (one chunk of a chunked
 * prefill, as attn_fwd_chunk).
 *
 * Defines: the causal forward attention of attn_fwd / attn_fwd_chunk (see
 * there for the pages' passages) on FP8 e4m3 inputs whose scales change every
 * 64 positions ([P1] "ZYFA's performance and accuracy data", scaling
 * granularity).  The K and V block scales are applied as E8M0 exponents by the
 * scaled MFMAs of CDNA4 (the pages' kernel uses those instructions to undo
 * power-of-two block scales, [P3] "ZYFA 如何工作？"), so they cost no vector
 * work; Q's block scale is folded into the score multiplier.
 *
 * Layout (contiguous BSHD, e4m3fn codes, as attn_fwd_chunk):
 *   q [B, Nq, Hq, d_qk], k [B, Nk, Hkv, d_qk], v [B, Nk, Hkv, d_v] (uint8)
 *   q_scale [B, Hq,  ceil(Nq / 64)]  fp32, positive (any value)
 *   k_scale [B, Hkv, ceil(Nk / 64)]  fp32, each a power of two in [2^-126, 2^127]
 *   v_scale [B, Hkv, ceil(Nk / 64)]  fp32, each a power of two in [2^-126, 2^127]
 *   out [B, Nq, Hq, d_v] bfloat16 (written); lse [B, Hq, Nq] fp32 (written
 *   unless NULL).  The real inputs are code * scale of the element's block
 *   (blocks of q count query rows, blocks of k and v count key rows).
 * K and V scales are read through their exponent bits only: a value that is
 * not a power of two acts as the power of two below it.  The quantizer
 * attn_quantize_fp8_block64 writes exactly this form.
 * Query row i sits at position i + Nk - Nq and attends to keys
 * j <= i + Nk - Nq; softmax_scale: tau, 0 selects 1 / sqrt(d_qk), otherwise
 * finite and positive (else MIATTN_ERR_VALUE).
 * p_block_scale = 1 also scales the probabilities by powers of two: each
 * query's 64 probabilities of a 64-key P.V step are shifted up by k octaves,
 * k = floor(running max - their max) in [0, 126], before
 * rounding to e4m3, and the scaled MFMAs multiply them by 2^-k ([P3] "ZYFA
 * 如何工作？": per-block power-of-two scaling of P undone by the scaled MFMA).
 * It keeps key blocks whose scores lie far below the row max (more than about
 * 13 octaves, where unshifted probabilities round to zero) at e4m3 precision,
 * at the cost of some vector work per step; p_block_scale = 0 rounds every
 * probability against the running max.  Any other value: MIATTN_ERR_DTYPE.
 * Sizes: B >= 0, 0 <= Nq <= Nk <= 2^20 (the exponents of a query tile's keys
 * are staged on chip), Hq >= 1, Hkv >= 1, Hq % Hkv == 0, (d_qk, d_v) in
 * {(128, 128), (192, 128)}; B == 0 or Nq == 0 is an empty call.  Alignment,
 * stream, asynchrony and determinism as attn_fwd.
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_block64(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d_qk, int d_v, const float* q_scale, const float* k_scale,
                     const float* v_scale, float softmax_scale, int p_block_scale, void* stream);

/* Scale granularities of attn_fwd_fp8. */
#define MIATTN_SCALES_HEAD 0    /* one fp32 scale per (batch, head), as attn_fwd */
#define MIATTN_SCALES_BLOCK64 1 /* one scale per (batch, head, 64 positions), as attn_fwd_block64 */

/* Probability modes of attn_fwd_fp8: how the softmax probabilities are rounded
 * to e4m3 for the P.V product.  Every mode multiplies them by a fixed 2^6
 * first (so the largest lies in [2^6, 2^8.75]) and divides the output by the
 * sum of the rounded values. */
#define MIATTN_P_LEAN 0        /* lean P: the e4m3 code of 2^x written from one FMA on the
                                  log2-domain score x (attn_fwd's mode) */
#define MIATTN_P_LEAN_BLOCK 1  /* lean P, and each query's probabilities of every 64-key step
                                  shifted up by 2^k (k = octaves their max lies below the running
                                  max, in [0, 126]); the scaled MFMAs multiply them by 2^-k */
#define MIATTN_P_EXACT 2       /* exp2 and the hardware round-to-nearest-even e4m3 conversion */
#define MIATTN_P_EXACT_BLOCK 3 /* exact, with the per-64-key shift of MIATTN_P_LEAN_BLOCK */
#define MIATTN_P_LEAN_TILE 4   /* lean P, and each query's probabilities of every key tile (192
                                  keys at d_qk = 128 in launches of more than 4096 keys, else
                                  128) shifted up by
                                  2^k (k = min(floor(running max - their max), 126)); the scaled
                                  MFMAs multiply them by 2^-k */
#define MIATTN_P_EXACT_TILE 5  /* exact, with the per-tile shift of MIATTN_P_LEAN_TILE */
#define MIATTN_P_DEFAULT MIATTN_P_LEAN_TILE /* the mode of attn_fwd and attn_fwd_chunk on FP8 inputs */

/* FP8 causal attention with a chosen scale granularity and probability mode.
 *
 * Defines: the causal forward attention of attn_fwd / attn_fwd_chunk (see
 * there) on FP8 e4m3 inputs, with the probabilities formed in one of the ways
 * the pages weigh against each other ([P3] "ZYFA 如何工作？": lean P, an
 * e4m3 code written straight from the score, against exp plus conversion; and
 * per-64-key power-of-two scaling of P undone by the scaled MFMA).
 *
 * Layout, sizes, softmax_scale, lse, stream, asynchrony and determinism as
 * attn_fwd_chunk (scales = MIATTN_SCALES_HEAD: q_scale [B, Hq], k_scale and
 * v_scale [B, Hkv]) or attn_fwd_block64 (scales = MIATTN_SCALES_BLOCK64:
 * per-64-position scales, Nk <= 2^20).  attn_fwd_fp8(..., MIATTN_SCALES_HEAD,
 * MIATTN_P_LEAN, ...) is attn_fwd_chunk on FP8 inputs, bit for bit;
 * (MIATTN_SCALES_BLOCK64, MIATTN_P_LEAN or MIATTN_P_LEAN_BLOCK) is
 * attn_fwd_block64 with p_block_scale 0 or 1.
 * Input domain: in the modes without a shift (MIATTN_P_LEAN, MIATTN_P_EXACT),
 * a probability more than about 12 octaves below its row's running max
 * (2^-12 of it) is rounded to zero (below about 15 octaves) or to a subnormal
 * e4m3 value; rows whose softmax mass lies largely that far below their
 * largest score (long rows of keys whose magnitudes vary by block) lose that
 * mass.  The block and tile modes round every 64-key step or key tile
 * against its own maximum, so only keys about 12 octaves below the maximum of
 * their own step or tile are lost.
 * scales or p_mode outside the values above: MIATTN_ERR_DTYPE.
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d_qk, int d_v, const float* q_scale, const float* k_scale, const float* v_scale,
                 float softmax_scale, int scales, int p_mode, void* stream);

/* Workspace of attn_fwd_ws: the bytes a launch with these arguments needs on
 * the current device, written to *bytes; 0 when the launch does not split its
 * keys (then attn_fwd_ws needs no workspace).
 *
 * Arguments as attn_fwd_ws (no tensors).  bytes NULL: MIATTN_ERR_NULL; invalid
 * arguments give attn_fwd_ws's error codes, with *bytes = 0.  The figure
 * depends on the device's compute-unit count, so query it with the device of
 * the launch current.
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_ws_size(int B, int Hq, int Hkv, int Nq, int Nk, int d_qk, int d_v, int dtype, int scales, int p_mode,
                     size_t* bytes);

/* Causal attention with a caller-provided workspace, which lets short launches
 * split their keys.
 *
 * Defines: the causal forward attention of attn_fwd_chunk (BF16, dtype =
 * MIATTN_DTYPE_BF16: scales and p_mode are checked but not used) or
 * attn_fwd_fp8 (dtype = MIATTN_DTYPE_FP8_E4M3) -- see there for the pages'
 * passages -- evaluated with the online softmax over key ranges whose partial
 * results are combined through their log-sum-exp, the identity that makes the
 * tiled evaluation exact ([P1] "Why prefill attention deserves dedicated
 * optimization": the scores are never materialised).
 *
 * Work split: the kernel gives each 256-query tile of a (batch, head) to one
 * workgroup, so a launch with fewer query tiles than compute units (short
 * sequences, or a short chunk against a long prefix) leaves units idle and
 * takes as long as its last query tile, which walks every key.  When
 * attn_fwd_ws_size is positive, every query tile is cut into ranges of at most
 * L key tiles, L the smallest for which every range gets a compute unit of its
 * own; the ranges of a query tile with more than one are written to the
 * workspace (normalised fp32 rows and log2 sums of exp) and merged in a second
 * kernel, in range order.
 * Layout, sizes, scales, softmax_scale, lse, stream and asynchrony as
 * attn_fwd_chunk / attn_fwd_fp8.  The result is bitwise reproducible from
 * launch to launch on one device (no atomics, fixed merge order); it may
 * differ in the last bits from attn_fwd_chunk / attn_fwd_fp8 where the launch
 * splits.
 * workspace: device memory of at least attn_fwd_ws_size bytes, 16-byte
 * aligned, owned by the caller; the call's kernels use it as scratch, so no
 * work that may run at the same time may use it; its contents afterwards are
 * unspecified.  May be NULL when attn_fwd_ws_size is 0.  Too small:
 * MIATTN_ERR_SIZE; NULL where it is needed: MIATTN_ERR_NULL; misaligned:
 * MIATTN_ERR_ALIGN (nothing enqueued in each case).
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Nq,
                int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                const float* v_scale, float softmax_scale, int scales, int p_mode, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of the static scratch attn_fwd_noalloc uses on each GPU: the most any
 * key-split plan needs on a device with 256 compute units (256 ranges of 256
 * fp32 rows of d_v = 128 plus their log2 sums of exp). */
#define MIATTN_NOALLOC_SCRATCH_BYTES 33816576

/* attn_fwd_ws without a workspace argument, allocating nothing.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The call is
 * attn_fwd_ws (arguments, layout, results and errors as there) with its
 * workspace in the library's own static scratch: a device array of
 * MIATTN_NOALLOC_SCRATCH_BYTES bytes per GPU, part of the library's device
 * code, held from the library's first use of that GPU until the process ends.
 * The call allocates and frees nothing.  Every call on one GPU uses that GPU's
 * one array, so calls that can overlap on one GPU (other streams, other host
 * threads) race on it: the caller must order them (one stream, or events).
 * Nothing in it needs to start at zero; its contents after a call are
 * unspecified.  A launch whose split plan needs more than the array holds
 * (possible only on devices with more than 256 compute units):
 * MIATTN_ERR_SCRATCH, nothing enqueued.
 * Returns MIATTN_OK or a negative MIATTN_ERR_* code. */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d_qk, int d_v, int dtype, const float* q_scale, const float* k_scale,
                     const float* v_scale, float softmax_scale, int scales, int p_mode, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

/* MIATTN_ABI_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H_ */
