/*
 * moe.h - C ABI of the MI355X (gfx950) quantized Mixture-of-Experts grouped
 * GEMM library (libqmoe.so).
 *
 * The method: M tokens with K features are routed to top_k of E experts; each
 * (token, expert) pair multiplies the token's row by that expert's quantized
 * weight matrix W[e] (N x K); the result is scaled by the router weight and the
 * top_k results of each token are summed.  Problem sizes are named as in the
 * column heads (M, K, N, E, top_k) of the FP8_W8A8 and INT8_W8A16 benchmark
 * tables on "Tianxing/moe quantization" (ROCm Triton pull request).  Formats:
 *   - fp8 W8A8  : e4m3 activations (one fp32 scale per tensor) x e4m3 weights
 *                 (one fp32 scale per expert)            ("FP8_W8A8 Benchmark")
 *   - int8 W8A16: bf16 activations x int8 weights with one fp32 scale per
 *                 expert and output channel             ("INT8_W8A16 Benchmark";
 *                 "INT8 quantization support", AutoAWQ issue)
 *   - MXFP8     : e4m3 data with one e8m0 scale per 32 values along K for both
 *                 operands, rows concatenated by expert, each expert's rowwise
 *                 scales padded to 128 rows    ("[PyTorch] Let GroupedLinear
 *                 accept MXFP8 input and gradient", Description and the reply
 *                 on padding the scaling factors)
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees memory and keeps no device state (the one
 *     exception, moe_quantize_act_noalloc, says so): every other launch
 *     depends only on its arguments, so calls may run concurrently on
 *     different streams.  On the host it keeps a thread-local record of the
 *     last error and the compute-unit count of the device (which sizes the
 *     persistent grids).
 *   - Every call only enqueues work on `stream` (0 = the null stream) and never
 *     synchronises; results are valid once the stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and no output is touched.
 *   - Return value: MOE_OK, or a negative MOE_E* code.  moe_last_error()
 *     describes the last failure of the calling thread; for MOE_EHIP,
 *     moe_last_hip_error() holds the hipError_t of the failed launch.
 *   - Pointers to arrays read or written with 16-byte vector accesses
 *     (activations, weights, quantized data, per-slot results) must be 16-byte
 *     aligned.
 *   - Array shapes are row-major, last index fastest.
 *   - Byte formats: e4m3 is OCP E4M3FN (bias 7, max 448, NaN = S.1111.111, no
 *     infinity); e8m0 byte b means 2^(b-127); bf16 is passed as uint16 bits.
 */
#ifndef QMOE_MOE_H
#define QMOE_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK            0
#define MOE_EINVAL       (-1)  /* null pointer, bad size, top_k > E, misaligned pointer */
#define MOE_EUNSUPPORTED (-2)  /* valid but unsupported: block_m, K granularity, limits */
#define MOE_EHIP         (-3)  /* a HIP launch failed; see moe_last_hip_error() */

/* ---- quantization modes ------------------------------------------------- */
#define MOE_Q_FP8_PER_TENSOR   0  /* e4m3 + one fp32 scale per tensor (per expert for weights) */
#define MOE_Q_MXFP8            1  /* e4m3 + one e8m0 scale per 32 values along K */
#define MOE_Q_INT8_PER_CHANNEL 2  /* int8 + one fp32 scale per row: per output channel
                                     (weights), per token (activations) */
#define MOE_Q_FP8_PER_CHANNEL  3  /* e4m3 + one fp32 scale per output channel (weights only) */
#define MOE_Q_INT4_PER_CHANNEL 4  /* int4 (two per byte) + one fp32 scale per output channel
                                     (weights only) */
#define MOE_Q_MXFP8_COLWISE    5  /* e4m3 + one e8m0 scale per 32 values along N, stored
                                     transposed (weights only: the input gradient) */

/* ---- activations fused with the quantization (moe_act_quantize) -------- */
#define MOE_ACT_SWIGLU 0  /* y = silu(g) * u, row = [g | u] (2H inputs -> H outputs) */
#define MOE_ACT_SRELU  1  /* y = max(x, 0)^2 (H inputs -> H outputs) */

/* ---- expert weight layouts (fp8 and int8 weights) ------------------------ */
#define MOE_W_ROWMAJOR 0  /* [E, N, K] bytes, K fastest */
#define MOE_W_TILED    1  /* as written by moe_pack_weights (see there) */
#define MOE_W_FRAG     2  /* as written by moe_pack_weights (see there); block_m 16 only */

/* ---- limits ------------------------------------------------------------- */
#define MOE_MAX_EXPERTS   128     /* E */
#define MOE_MAX_TOPK      8       /* top_k */
#define MOE_MAX_SLOTS     65536   /* M * top_k handled by one align call */

/* Message describing the last failure on the calling thread ("" if none). */
const char *moe_last_error(void);
/* hipError_t of the last MOE_EHIP failure on the calling thread (0 if none). */
int moe_last_hip_error(void);

/* ======================================================================== *
 * Sizes
 * ======================================================================== */

/* Length of the sorted-slot buffer for moe_align_block_size:
 * M*top_k + E*(block_m-1) rounded up to a multiple of block_m.  The expert-id
 * buffer holds moe_align_max_padded(...)/block_m entries.  Returns a negative
 * MOE_E* code for invalid sizes. */
int moe_align_max_padded(int M, int E, int top_k, int block_m);

/* block_m the grouped GEMMs run fastest with for this routing shape: 16 while
 * the average expert holds few rows (the weight-streaming kernel), else 128
 * (the tiled MFMA kernel).  Both are accepted by every routed GEMM. */
int moe_recommended_block_m(int M, int E, int top_k);

/* Bytes of device workspace moe_quantize_act / moe_quantize_weights need for
 * `mode` on `tensors` independent tensors (1 for activations, E for weights);
 * 0 when the mode needs none. */
size_t moe_quantize_workspace_bytes(int mode, int tensors);

/* Bytes of E x N x K one-byte weights in `layout`: MOE_W_TILED
 * E * ceil(N/64) * ceil(K/128) * 8192, MOE_W_FRAG E * ceil(N/16) *
 * ceil(K/64) * 1024, MOE_W_ROWMAJOR E * N * K; 0 for an unknown layout or a
 * size below 1. */
size_t moe_packed_weight_bytes(int E, int N, int K, int layout);

/* Upper bound on the rows of the padded MXFP8 rowwise scale matrix for `rows`
 * rows spread over E experts: rows + E*127 (each expert's block is padded to
 * a multiple of 128 rows).  rows > 2^30 -> MOE_EUNSUPPORTED. */
int moe_mx_scale_rows(int rows, int E);

/* ======================================================================== *
 * a1 + a2: routing and block alignment
 * ======================================================================== */

/* Top-k routing of every token and grouping of the routed slots by expert.
 * The grouped GEMM runs as one linear op per expert over that expert's
 * (unequal) set of routed rows ("Enabling MOE Quantization using linear
 * decomposition", Summary); this call forms those row sets for the (M, E,
 * top_k) of the benchmark tables on "Tianxing/moe quantization".  The pages
 * give no block size: padding each set to a multiple of block_m is the
 * tiling these kernels use.
 *
 * Routing: for token t the top_k experts with the largest float32 logits are
 * chosen (on equal logits the lower expert index first); router weights are
 * exp(l_e - l_max) over the chosen experts divided by their sum (the softmax
 * over all E logits restricted to the chosen experts and renormalised).
 * Slot i = t*top_k + j is the j-th choice of token t.
 *
 * Alignment: the slots are grouped by expert (ascending expert; inside an
 * expert ascending slot), every group is padded to a multiple of block_m with
 * the sentinel M*top_k, and every block of block_m sorted slots is labelled
 * with its expert.
 *
 *   logits                 [M, E] float32, read
 *   topk_ids               [M, top_k] int32, written
 *   topk_weights           [M, top_k] float32, written
 *   sorted_token_ids       [moe_align_max_padded()] int32, written in full:
 *                          slots, then the sentinel M*top_k in padding and tail
 *   expert_ids             [moe_align_max_padded()/block_m] int32, written in
 *                          full: expert of each block, -1 after the last block
 *   num_tokens_post_padded [1] int32, written: padded length (multiple of block_m)
 *
 * Limits: 1 <= E <= MOE_MAX_EXPERTS, 1 <= top_k <= min(E, MOE_MAX_TOPK),
 * 0 <= M*top_k <= MOE_MAX_SLOTS, block_m in {16, 32, 64, 128, 256}.
 * M = 0 is valid (no slots; the buffers are still written).
 * Up to 1024 tokens one workgroup does the whole call; above that the top-k
 * choice runs on a grid of its own first.  Either way the call enqueues
 * its kernels on `s` and never synchronizes. */
int moe_align_block_size(const float *logits, int M, int E, int top_k, int block_m,
                         int *topk_ids, float *topk_weights, int *sorted_token_ids,
                         int *expert_ids, int *num_tokens_post_padded,
                         hipStream_t stream);

/* ======================================================================== *
 * a3: activation quantization
 * ======================================================================== */

/* Dynamic quantization of bf16 activations x [rows, K] to e4m3.
 *
 * mode MOE_Q_FP8_PER_TENSOR: amax = max|x| over the whole tensor,
 *   s = fl32(amax/448) (s = 1 if amax = 0), q = e4m3(fl32(x * fl32(1/s)))
 *   rounded to nearest even and saturated to +-448.  Writes q [rows, K] and
 *   scale[0] = s.  `workspace` must hold moe_quantize_workspace_bytes(mode, 1)
 *   bytes (contents on entry are ignored).  m_offsets/E/scale_e8m0 unused.
 * mode MOE_Q_MXFP8: for each row and each block of 32 values along K,
 *   b = clamp(exponent_field(amax_block) - 8, 0, 254) (the shared exponent
 *   floor(log2 amax) - 8 of the OCP MX rule for e4m3), q = e4m3(x * 2^(127-b))
 *   saturated.  m_offsets [E+1] (device, int32, non-decreasing, m_offsets[0]=0,
 *   m_offsets[E]=rows) splits the rows by expert; the scale byte of row r of
 *   expert e goes to row P_e + (r - m_offsets[e]) of scale_e8m0 [*, K/32],
 *   where P_e = sum over e' < e of roundup(m_e', 128); the pad rows of every
 *   expert's block are written with 0.  scale_e8m0 must hold
 *   moe_mx_scale_rows(rows, E) rows; rows past the padded total are not
 *   touched.  scale/workspace unused (may be NULL).
 * mode MOE_Q_INT8_PER_CHANNEL: dynamic per-token int8 ("Enabling MOE
 *   Quantization using linear decomposition", Summary: the int8 dynamic
 *   activation family), per row t s_t = fl32(amax_t/127) (1 if zero),
 *   q = clamp(round_half_even(fl32(x * fl32(1/s_t))), -127, 127).  Writes q
 *   [rows, K] (int8 in the uint8 buffer, 8-byte aligned) and scale [rows].
 *   m_offsets/E/scale_e8m0/workspace unused.
 *
 * K must be a multiple of 32 (MXFP8) or 8 (fp8, int8); MXFP8 takes at most
 * 2^30 rows.  rows = 0 is valid. */
int moe_quantize_act(const uint16_t *x, int rows, int K, int mode,
                     const int *m_offsets, int E, uint8_t *q, float *scale,
                     uint8_t *scale_e8m0, void *workspace, hipStream_t stream);

/* Allocation-free variant of moe_quantize_act, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as moe_quantize_act without `workspace`: the partial
 * maxima of MOE_Q_FP8_PER_TENSOR go to a static device array of the library
 * (4 KiB per device, kept until the process ends; its address is looked up on
 * the first call on each device, which is not graph-capturable), whose
 * capacity covers any tensor size (MOE_EUNSUPPORTED if a mode needed more).
 * The other modes use no scratch.  Nothing is allocated and nothing needs to
 * start at zero.  Calls that overlap on one device share the array and race:
 * serialize them (one stream, or events between streams). */
int moe_quantize_act_noalloc(const uint16_t *x, int rows, int K, int mode,
                             const int *m_offsets, int E, uint8_t *q, float *scale_fp32,
                             uint8_t *scale_e8m0, hipStream_t stream);

/* Activation fused with its quantization: the expert FFN's step between the
 * up and the down projection ("[PyTorch] Let GroupedLinear accept MXFP8 input
 * and gradient", Description: SwiGLU / SReLU + MXFP8 quantization of an
 * expert-concatenated (8*4000, 4096) input, quantized as a whole with the
 * scaling factors padded per expert).  For every row r and output column
 * n < H, in float32 on the bf16 inputs:
 *   MOE_ACT_SWIGLU: x [rows, 2H], g = x[r, n], u = x[r, H + n],
 *                   y = (g / (1 + exp(-g))) * u
 *   MOE_ACT_SRELU : x [rows, H], y = max(x[r, n], 0)^2 (exact)
 * SReLU is exact in float32; SwiGLU uses the hardware exp2 (with the
 * exponent split into a float32 sum so its rounding does not grow with |g|)
 * and the hardware reciprocal, within about 7 float32 units of the exact
 * value (|g| >= 128 gives g * u or a signed zero, as exp(-g) is 0 or
 * infinite in float32 there).
 * y [rows, H] is quantized as moe_quantize_act quantizes x with the same
 * mode (MXFP8 with per-expert padded scale blocks and m_offsets / E, or fp8
 * per tensor with a workspace of moe_quantize_workspace_bytes(mode, 1) bytes);
 * y itself is never stored.  q [rows, H] e4m3; scale / scale_e8m0 /
 * workspace as for moe_quantize_act with K = H.
 *
 * x must be 16-byte aligned; H must be a multiple of 32 (MXFP8) or 8 (fp8);
 * at most 2^30 rows.  rows = 0 is valid. */
int moe_act_quantize(const uint16_t *x, int rows, int H, int act, int mode,
                     const int *m_offsets, int E, uint8_t *q, float *scale,
                     uint8_t *scale_e8m0, void *workspace, hipStream_t stream);

/* Offline quantization of float32 expert weights w [E, N, K].
 *
 * MOE_Q_FP8_PER_TENSOR  : per expert s_e = fl32(amax(W[e])/448) (1 if zero),
 *                         q = e4m3(fl32(w * fl32(1/s_e))); q is uint8 [E,N,K],
 *                         scale [E].  Needs workspace of
 *                         moe_quantize_workspace_bytes(mode, E) bytes.
 * MOE_Q_FP8_PER_CHANNEL : per row (output channel) s = fl32(amax_row/448)
 *                         (1 if zero), q = e4m3(fl32(w * fl32(1/s))) with
 *                         saturation to +-448; q is uint8 [E,N,K], scale
 *                         [E,N] ("Enabling MOE Quantization using linear
 *                         decomposition", Summary: fp8 weight-only).
 * MOE_Q_INT4_PER_CHANNEL: per row s = fl32(amax_row/7) (1 if zero),
 *                         q = clamp(round_half_even(fl32(w * fl32(1/s))), -7, 7)
 *                         ("Enabling MOE Quantization using linear
 *                         decomposition", Summary: int4 weight-only); q is
 *                         uint8 [E, N, K/2] (4-byte aligned): the 8 codes of
 *                         k = 8c .. 8c+7 of a row form the little-endian dword
 *                         c of that row (bytes 4c .. 4c+3), code k = 8c + j
 *                         stored as the 4-bit number q + 8 (1 .. 15) in bits
 *                         4f .. 4f+3 with f = (j >> 1) + 4 (j & 1); scale [E,N].
 * MOE_Q_INT8_PER_CHANNEL: per row s = fl32(amax_row/127) (1 if zero),
 *                         q = clamp(round_half_even(fl32(w * fl32(1/s))),
 *                         -127, 127); q is int8 [E,N,K], scale [E,N].
 * MOE_Q_MXFP8_COLWISE   : blocks of 32 along N (per k and expert) by the MXFP8
 *                         rule, stored transposed: q uint8 [E, K, N] (q[e,k,n]
 *                         the code of w[e,n,k]), scale_e8m0 [E, K, N/32]; the
 *                         weights of the input gradient ("[PyTorch] Let
 *                         GroupedLinear accept MXFP8 input and gradient").
 *                         N must be a multiple of 128 and K of 64.
 * MOE_Q_MXFP8           : per row and block of 32 along K as in
 *                         moe_quantize_act; q uint8 [E,N,K], scale_e8m0
 *                         [E,N,K/32] (no padding).
 * K must be a multiple of 32 (MXFP8) or 8. */
int moe_quantize_weights(const float *w, int E, int N, int K, int mode,
                         void *q, float *scale, uint8_t *scale_e8m0,
                         void *workspace, hipStream_t stream);

/* Offline re-layout of one-byte expert weights (e4m3 or int8) for streaming.
 *
 * MOE_W_FRAG (for block_m 16): the weights of expert e are cut into 16-row
 * groups j = n / 16 (J = ceil(N/16)) and 64-byte k blocks b = k / 64
 * (B = ceil(K/64)); the 1024-byte block (e, j, b) is stored at byte offset
 * ((e*B + b)*J + j) * 1024 (k block outside row group: at any moment the
 * workgroups streaming one expert read one contiguous stretch of it, which
 * spreads the reads evenly over the HBM channels), and its 16-byte piece
 * p = 16*q + r (q = 0..3,
 * r = 0..15) holds row n = 16j + r, k = 64b + 16q .. 64b + 16q + 15.  This is
 * the order in which the 64 lanes of a wavefront take one MFMA operand
 * fragment (lane p: row r, k group q), so each fragment is one contiguous
 * 1 KB read straight into registers.  Rows n >= N and k >= K are zero.
 *
 * MOE_W_TILED: the weights of expert e are cut into 64-row tiles t = n / 64
 * (T = ceil(N/64)) and 128-byte k slices s = k / 128 (S = ceil(K/128)); the
 * 64 x 128-byte block (e, t, s) is stored contiguously (8192 bytes) at byte
 * offset ((e*T + t)*S + s) * 8192, rows in order, 128 bytes per row, and the
 * 16-byte chunk c of row r (k = 128s + 16c .. 128s + 16c + 15) at chunk
 * position c ^ ((r >> 1) & 7) of that row.  Rows n >= N and
 * k >= K are zero.
 * Every block is then one contiguous HBM read of the decode GEMM, landing in
 * LDS in the bank-conflict-free order its MFMA reads use.
 *
 *   w_q      [E, N, K] bytes (MOE_W_ROWMAJOR), read
 *   layout   MOE_W_TILED or MOE_W_FRAG
 *   w_packed moe_packed_weight_bytes(E, N, K, layout) bytes, written in full
 * K must be a multiple of 16; the packed size must stay below 4 GiB. */
int moe_pack_weights(const void *w_q, int E, int N, int K, int layout, void *w_packed,
                     hipStream_t stream);

/* ======================================================================== *
 * a4 + a5: grouped GEMM with the fused scale / router-weight epilogue
 * ======================================================================== */

/* Routed fp8 W8A8 grouped GEMM.  For every sorted slot i of expert e (from
 * moe_align_block_size run with the same M, E, top_k, block_m), token
 * t = i / top_k, and every column n < N:
 *     y[i, n] = bf16( (sum_k a[t,k] * w[e,n,k]) * (a_scale[0] * w_scale[e]) * topk_weights[i] )
 * with e4m3 operands, fp32 accumulation, rounding to nearest even, and
 * padding slots skipped.  The per-slot results are stored as bf16, two bytes
 * per slot and column as in the output term of the byte accounting behind the
 * FP8_W8A8 / INT8_W8A16 benchmark tables ("Tianxing/moe quantization").
 *
 *   a_q [M, K] uint8 e4m3, a_scale [1] f32, w_q e4m3 weights in layout
 *   w_layout (MOE_W_ROWMAJOR [E, N, K], MOE_W_TILED or, with block_m 16 only,
 *   MOE_W_FRAG), w_scale [E] f32,
 *   topk_weights [M*top_k] f32, routing buffers as written by
 *   moe_align_block_size, y [M*top_k, N] uint16 bf16, 16-byte aligned (rows
 *   of slots that are not routed are not written; with every slot routed, y
 *   is written in full).
 *
 * K must be a multiple of 128 and N of 8; block_m must be 16 or 128.
 * block_m 16 runs the weight-streaming kernel (fastest with MOE_W_FRAG), 128
 * the tiled one (MOE_W_FRAG is rejected there with MOE_EUNSUPPORTED).  The
 * other routed GEMMs below take the same layouts under the same rule. */
int moe_grouped_gemm_fp8w8a8(const uint8_t *a_q, const float *a_scale,
                             const uint8_t *w_q, const float *w_scale, int w_layout,
                             const int *sorted_token_ids, const int *expert_ids,
                             const int *num_tokens_post_padded,
                             const float *topk_weights, int M, int K, int N, int E,
                             int top_k, int block_m, uint16_t *y, hipStream_t stream);

/* Routed int8 W8A8 grouped GEMM with dynamic per-token activation scales
 * ("Enabling MOE Quantization using linear decomposition", Summary: int8
 * dynamic activations x int8 weights): as moe_grouped_gemm_fp8w8a8 with
 *     y[i, n] = bf16( (sum_k a[t,k] * w[e,n,k]) * a_scale[t] * w_scale[e, n] * topk_weights[i] )
 * for int8 a_q [M, K] with a_scale [M] f32 (moe_quantize_act with
 * MOE_Q_INT8_PER_CHANNEL), int8 w_q in layout w_layout with w_scale [E, N]
 * f32 (moe_quantize_weights with MOE_Q_INT8_PER_CHANNEL).  The products are
 * accumulated exactly in int32 on the int8 MFMA and converted to fp32 once.
 * K must be a multiple of 128 and N of 8; block_m must be 16 or 128. */
int moe_grouped_gemm_int8w8a8(const int8_t *a_q, const float *a_scale,
                              const int8_t *w_q, const float *w_scale, int w_layout,
                              const int *sorted_token_ids, const int *expert_ids,
                              const int *num_tokens_post_padded,
                              const float *topk_weights, int M, int K, int N, int E,
                              int top_k, int block_m, uint16_t *y, hipStream_t stream);

/* Routed int8 W8A16 grouped GEMM: as moe_grouped_gemm_fp8w8a8 with
 *     y[i, n] = bf16( (sum_k a[t,k] * w[e,n,k]) * w_scale[e, n] * topk_weights[i] )
 * for bf16 a [M, K] (uint16 bits), int8 w_q in layout w_layout, w_scale
 * [E, N] f32.  The int8 weights are converted exactly to bf16 inside the
 * kernel and the products are accumulated in fp32.  K must be a multiple of
 * 64 and N of 8; block_m must be 16 or 128. */
int moe_grouped_gemm_int8w8a16(const uint16_t *a, const int8_t *w_q,
                               const float *w_scale, int w_layout,
                               const int *sorted_token_ids, const int *expert_ids,
                               const int *num_tokens_post_padded,
                               const float *topk_weights, int M, int K, int N, int E,
                               int top_k, int block_m, uint16_t *y, hipStream_t stream);

/* Routed fp8 weight-only grouped GEMM ("Enabling MOE Quantization using
 * linear decomposition", Summary: bf16 activations x fp8 weights with a scale
 * per output channel): as moe_grouped_gemm_int8w8a16 with e4m3 w_q in layout
 * w_layout and w_scale [E, N] f32 (moe_quantize_weights with
 * MOE_Q_FP8_PER_CHANNEL).  Every e4m3 value is exactly a bf16 value, so the
 * weights are converted exactly to bf16 inside the kernel and the products
 * are accumulated in fp32:
 *     y[i, n] = bf16( (sum_k a[t,k] * w[e,n,k]) * w_scale[e, n] * topk_weights[i] )
 * K must be a multiple of 64 and N of 8; block_m must be 16 or 128. */
int moe_grouped_gemm_fp8w8a16(const uint16_t *a, const uint8_t *w_q,
                              const float *w_scale, int w_layout,
                              const int *sorted_token_ids, const int *expert_ids,
                              const int *num_tokens_post_padded,
                              const float *topk_weights, int M, int K, int N, int E,
                              int top_k, int block_m, uint16_t *y, hipStream_t stream);

/* Routed int4 weight-only grouped GEMM ("Enabling MOE Quantization using
 * linear decomposition", Summary: bf16 activations x int4 weights with one
 * scale per output channel): as moe_grouped_gemm_int8w8a16 with
 *     y[i, n] = bf16( (sum_k a[t,k] * q[e,n,k]) * w_scale[e, n] * topk_weights[i] )
 * for the codes q of w_q (moe_quantize_weights with MOE_Q_INT4_PER_CHANNEL),
 * given as that [E, N, K/2] byte matrix (MOE_W_ROWMAJOR) or as its
 * MOE_W_FRAG packing (moe_pack_weights of the byte matrix with K/2 in place
 * of K); w_scale [E, N] f32.  The kernel turns each code into the bf16 value
 * 136 + q exactly, accumulates in fp32 on the bf16 MFMA and subtracts 136
 * times the row sum of the activations (accumulated the same way) before the
 * epilogue.  K must be a multiple of 128 and N of 8; block_m must be 16
 * (other block_m and MOE_W_TILED give MOE_EUNSUPPORTED). */
int moe_grouped_gemm_int4w4a16(const uint16_t *a, const uint8_t *w_q,
                               const float *w_scale, int w_layout,
                               const int *sorted_token_ids, const int *expert_ids,
                               const int *num_tokens_post_padded,
                               const float *topk_weights, int M, int K, int N, int E,
                               int top_k, int block_m, uint16_t *y, hipStream_t stream);

/* MXFP8 grouped linear over expert-contiguous rows (no router): for row r of
 * expert e (m_offsets[e] <= r < m_offsets[e+1]) and column n < N,
 *     out[r, n] = bf16( sum over blocks kb of 2^(ba[r,kb] + bw[e,n,kb] - 254)
 *                       * sum_{k in kb} a[r,k] * w[e,n,k] )
 * accumulated in fp32 and rounded to nearest even.
 *
 *   a_q [rows, K] uint8 e4m3; a_sf padded rowwise scales as written by
 *   moe_quantize_act(MOE_Q_MXFP8) with the same m_offsets; w_q [E, N, K]
 *   uint8 e4m3; w_sf [E, N, K/32] e8m0; m_offsets [E+1] int32 (device);
 *   out [rows, N] uint16 bf16, written in full.
 *
 * With the output gradient dy as a (moe_quantize_act(MOE_Q_MXFP8), K = the
 * layer's N) and the weights quantized with MOE_Q_MXFP8_COLWISE as w ([E, K,
 * N], N = the layer's K) the same call computes the input gradient
 * dx[r, k] = sum_n dy[r, n] w[e, n, k] of the grouped linear.
 *
 * K must be a multiple of 128. */
int moe_grouped_gemm_mxfp8(const uint8_t *a_q, const uint8_t *a_sf,
                           const uint8_t *w_q, const uint8_t *w_sf,
                           const int *m_offsets, int rows, int K, int N, int E,
                           uint16_t *out, hipStream_t stream);

/* ======================================================================== *
 * MXFP8 backward of the grouped linear ("[PyTorch] Let GroupedLinear accept
 * MXFP8 input and gradient": colwise scaling factors for the gradient)
 * ======================================================================== */

/* Columnwise MXFP8 of expert-concatenated bf16 rows (activations x or output
 * gradients dy) for the weight gradient: for expert e (rows m_offsets[e] ..
 * m_offsets[e+1]-1, m_e of them) the rows are padded with zeros to
 * Rp_e = roundup(m_e, 128); column c, padded rows 32j .. 32j+31 form one
 * block with one e8m0 scale by the MXFP8 rule (moe_quantize_act).  Stored
 * transposed, expert by expert, with P_e = Rp_0 + .. + Rp_{e-1}:
 *   qT  code of row m_offsets[e] + i, column c at byte C*P_e + c*Rp_e + i
 *       (zero for the padding rows)
 *   sfT scale of block j of column c at byte C*P_e/32 + c*Rp_e/32 + j
 * x [rows, C] bf16 (16-byte aligned), m_offsets [E+1] int32 (device), qT at
 * least C * moe_mx_scale_rows(rows, E) bytes (16-byte aligned), sfT at least
 * C * moe_mx_scale_rows(rows, E) / 32 bytes.  C must be a multiple of 64;
 * rows + 127 E at most 65535 * 128. */
int moe_quantize_act_colwise(const uint16_t *x, int rows, int C, const int *m_offsets, int E,
                             uint8_t *qT, uint8_t *sfT, hipStream_t stream);

/* Weight gradient of the MXFP8 grouped linear y = x W_e^T: for every expert
 *     dw[e, n, k] = bf16( sum over the padded rows i of expert e, in blocks of
 *                   32, of 2^(b_dy + b_x - 254) * dyT[n, i] * xT[k, i] )
 * accumulated in fp32 (an expert without rows gets zeros).  dyT_q / dyT_sf
 * and xT_q / xT_sf are moe_quantize_act_colwise of dy [rows, N] and
 * x [rows, K] with the same expert segments; m_splits [E] are the rows per
 * expert in HOST memory (the caller knows the split; no device read or
 * synchronisation is needed to size the launches).  dw [E, N, K] uint16 bf16,
 * 16-byte aligned, written in full.  N must be a multiple of 128 and K of
 * 64.  One launch covers every expert. */
int moe_grouped_gemm_mxfp8_wgrad(const uint8_t *dyT_q, const uint8_t *dyT_sf,
                                 const uint8_t *xT_q, const uint8_t *xT_sf, const int *m_splits,
                                 int E, int N, int K, uint16_t *dw, hipStream_t stream);

/* ======================================================================== *
 * a6: combine
 * ======================================================================== */

/* Per-token combine: the sum over a token's top_k experts of their
 * router-weighted results (the method statement at the top of this file; the
 * MoE layer as a sum of per-expert linear outputs, "Enabling MOE Quantization
 * using linear decomposition", Summary):
 *     out[t, n] = bf16( y[t*top_k, n] + ... + y[t*top_k+top_k-1, n] )
 * over the bf16 per-slot results, with the adds done in float32 in slot order
 * and the sum rounded to nearest even.  y [M*top_k, N] uint16 bf16, out
 * [M, N] uint16 bf16, both 16-byte aligned.  N must be a multiple of 8. */
int moe_combine(const uint16_t *y, int M, int N, int top_k, uint16_t *out,
                hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_MOE_H */
