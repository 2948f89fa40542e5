// C ABI of libqmoe.so (declared in include/moe.h): argument validation on the
// host, then the launches on the caller's stream.  No entry point allocates,
// frees or synchronises; on a validation error nothing is enqueued.
#include "moe.h"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "qmoe_internal.h"

namespace {

// MXFP8 row counts: rows plus the per-expert padding stay within int.
constexpr int kMxMaxRows = 1 << 30;

thread_local char g_err[512] = "";
thread_local int g_hip_err = 0;

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  g_hip_err = 0;
  return MOE_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  g_hip_err = (int)e;
  return fail(MOE_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_block_m(int b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

#define REQUIRE(cond, code, ...)                  \
  do {                                            \
    if (!(cond)) return fail((code), __VA_ARGS__); \
  } while (0)

int check_routing_sizes(int M, int E, int top_k, const char *fn) {
  REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d outside [1, %d]", fn, E,
          MOE_MAX_EXPERTS);
  REQUIRE(top_k >= 1 && top_k <= E, MOE_EINVAL, "%s: top_k=%d outside [1, E=%d]", fn, top_k, E);
  REQUIRE(top_k <= MOE_MAX_TOPK, MOE_EUNSUPPORTED, "%s: top_k=%d above %d", fn, top_k,
          MOE_MAX_TOPK);
  REQUIRE(M >= 0, MOE_EINVAL, "%s: M=%d is negative", fn, M);
  REQUIRE((long long)M * top_k <= MOE_MAX_SLOTS, MOE_EUNSUPPORTED,
          "%s: M*top_k=%lld above %d", fn, (long long)M * top_k, MOE_MAX_SLOTS);
  return MOE_OK;
}

long long max_padded_ll(int M, int E, int top_k, int block_m) {
  const long long n = (long long)M * top_k + (long long)E * (block_m - 1);
  return (n + block_m - 1) / block_m * block_m;
}

// Outputs written by 32-bit buffer offsets (the out-of-range offset of the
// tile GEMM's dropped stores lies above this)
constexpr long long kMaxOutBytes = 0xFFFFFF00ll;

int check_routed_gemm(const void *a, const void *w, const void *w_scale, int w_layout,
                      const int *sorted, const int *expert_ids, const int *num_post,
                      const float *topk_w, const uint16_t *y, int M, int K, int N, int E, int top_k,
                      int block_m, int k_mult, const char *fn) {
  int rc = check_routing_sizes(M, E, top_k, fn);
  if (rc) return rc;
  REQUIRE(w_layout == MOE_W_ROWMAJOR || w_layout == MOE_W_TILED || w_layout == MOE_W_FRAG,
          MOE_EINVAL, "%s: unknown weight layout %d", fn, w_layout);
  REQUIRE(K > 0 && N > 0, MOE_EINVAL, "%s: K=%d and N=%d must be positive", fn, K, N);
  REQUIRE(K % k_mult == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of %d", fn, K, k_mult);
  REQUIRE(N % 8 == 0, MOE_EUNSUPPORTED, "%s: N=%d is not a multiple of 8", fn, N);
  REQUIRE(block_m == 16 || block_m == 128, MOE_EUNSUPPORTED,
          "%s: block_m=%d (supported: 16, 128)", fn, block_m);
  REQUIRE(w_layout != MOE_W_FRAG || block_m == 16, MOE_EUNSUPPORTED,
          "%s: MOE_W_FRAG weights need block_m 16", fn);
  if (M == 0) return MOE_OK;               // nothing to do; buffers may be empty
  REQUIRE(a && w && w_scale && sorted && expert_ids && num_post && topk_w && y, MOE_EINVAL,
          "%s: null pointer argument", fn);
  REQUIRE(aligned16(a) && aligned16(w) && aligned16(y), MOE_EINVAL,
          "%s: activation, weight and output pointers must be 16-byte aligned", fn);
  REQUIRE((long long)E * N * (long long)K < (1ll << 32) &&
              moe_packed_weight_bytes(E, N, K, MOE_W_TILED) < (1ull << 32) &&
              moe_packed_weight_bytes(E, N, K, MOE_W_FRAG) < (1ull << 32),
          MOE_EUNSUPPORTED, "%s: weight tensor must stay below 4 GiB", fn);
  REQUIRE((long long)M * (long long)K * 2 < (1ll << 32), MOE_EUNSUPPORTED,
          "%s: activation tensor must stay below 4 GiB", fn);
  REQUIRE((long long)M * top_k * (long long)N * 2 < kMaxOutBytes, MOE_EUNSUPPORTED,
          "%s: per-slot results must stay below 4 GiB", fn);
  return MOE_OK;
}

// ---- scratch of moe_quantize_act_noalloc ------------------------------------
// The per-tensor fp8 quantizer's partial maxima live in this device array
// instead of a caller workspace.  Host code never uses the array's name as a
// device address: the address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int kScratchFloats = qmoe::kAmaxPartials;     // 4 KiB
__device__ __align__(256) float scratch[kScratchFloats];
constexpr int kMaxDevices = 64;
float *g_scratch_dev[kMaxDevices] = {};
std::mutex g_scratch_mu;

// this device's copy of `scratch` (resolved on the first call on the device)
int scratch_for_current_device(float **out, const char *fn) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    const hipError_t es = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (es != hipSuccess || !ptr) return hip_status(es != hipSuccess ? es : hipErrorInvalidSymbol, fn);
    g_scratch_dev[dev] = static_cast<float *>(ptr);
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_last_error(void) { return g_err; }
int moe_last_hip_error(void) { return g_hip_err; }

int moe_align_max_padded(int M, int E, int top_k, int block_m) {
  int rc = check_routing_sizes(M, E, top_k, "moe_align_max_padded");
  if (rc) return rc;
  REQUIRE(valid_block_m(block_m), MOE_EUNSUPPORTED, "moe_align_max_padded: block_m=%d",
          block_m);
  ok();
  return (int)max_padded_ll(M, E, top_k, block_m);
}

int moe_recommended_block_m(int M, int E, int top_k) {
  int rc = check_routing_sizes(M, E, top_k, "moe_recommended_block_m");
  if (rc) return rc;
  ok();
  // few rows per expert: stream the weights once with all rows in registers
  const long long avg_rows = ((long long)M * top_k + E - 1) / E;
  return avg_rows <= 48 ? 16 : 128;
}

size_t moe_quantize_workspace_bytes(int mode, int tensors) {
  if (mode != MOE_Q_FP8_PER_TENSOR || tensors <= 0) return 0;
  return (size_t)tensors * qmoe::kAmaxPartials * sizeof(float);
}

size_t moe_packed_weight_bytes(int E, int N, int K, int layout) {
  if (E < 1 || N < 1 || K < 1) return 0;
  if (layout == MOE_W_TILED)
    return (size_t)E * (size_t)((N + qmoe::kPackRows - 1) / qmoe::kPackRows) *
           (size_t)((K + qmoe::kPackK - 1) / qmoe::kPackK) *
           (size_t)(qmoe::kPackRows * qmoe::kPackK);
  if (layout == MOE_W_FRAG)
    return (size_t)E * (size_t)((N + 15) / 16) * (size_t)((K + 63) / 64) * 1024u;
  if (layout == MOE_W_ROWMAJOR) return (size_t)E * (size_t)N * (size_t)K;
  return 0;
}

int moe_pack_weights(const void *w_q, int E, int N, int K, int layout, void *w_packed,
                     hipStream_t stream) {
  const char *fn = "moe_pack_weights";
  REQUIRE(E >= 1 && N > 0 && K > 0, MOE_EINVAL, "%s: E=%d N=%d K=%d", fn, E, N, K);
  REQUIRE(layout == MOE_W_TILED || layout == MOE_W_FRAG, MOE_EINVAL, "%s: layout %d", fn, layout);
  REQUIRE(w_q && w_packed, MOE_EINVAL, "%s: null pointer argument", fn);
  REQUIRE(aligned16(w_q) && aligned16(w_packed), MOE_EINVAL, "%s: pointers must be 16-byte aligned",
          fn);
  REQUIRE(K % 16 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 16", fn, K);
  REQUIRE(moe_packed_weight_bytes(E, N, K, layout) < (1ull << 32), MOE_EUNSUPPORTED,
          "%s: packed weights must stay below 4 GiB", fn);
  return hip_status(qmoe::launch_pack_weights((const uint8_t *)w_q, E, N, K, layout,
                                              (uint8_t *)w_packed, stream),
                    fn);
}

int moe_mx_scale_rows(int rows, int E) {
  if (rows < 0 || E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_EINVAL, "moe_mx_scale_rows: rows=%d E=%d", rows, E);
  if (rows > kMxMaxRows)
    return fail(MOE_EUNSUPPORTED, "moe_mx_scale_rows: rows=%d exceeds %d", rows, kMxMaxRows);
  ok();
  return rows + E * (qmoe::kMxRowPad - 1);
}

int moe_align_block_size(const float *logits, int M, int E, int top_k, int block_m,
                         int *topk_ids, float *topk_weights, int *sorted_token_ids,
                         int *expert_ids, int *num_tokens_post_padded, hipStream_t stream) {
  const char *fn = "moe_align_block_size";
  int rc = check_routing_sizes(M, E, top_k, fn);
  if (rc) return rc;
  REQUIRE(valid_block_m(block_m), MOE_EUNSUPPORTED, "%s: block_m=%d", fn, block_m);
  REQUIRE(sorted_token_ids && expert_ids && num_tokens_post_padded, MOE_EINVAL,
          "%s: null output pointer", fn);
  REQUIRE(M == 0 || (logits && topk_ids && topk_weights), MOE_EINVAL, "%s: null pointer", fn);
  const int max_padded = (int)max_padded_ll(M, E, top_k, block_m);
  return hip_status(qmoe::launch_route_align(logits, M, E, top_k, block_m, max_padded, topk_ids,
                                             topk_weights, sorted_token_ids, expert_ids,
                                             num_tokens_post_padded, stream),
                    fn);
}

int moe_quantize_act(const uint16_t *x, int rows, int K, int mode, const int *m_offsets, int E,
                     uint8_t *q, float *scale, uint8_t *scale_e8m0, void *workspace,
                     hipStream_t stream) {
  const char *fn = "moe_quantize_act";
  REQUIRE(rows >= 0 && K > 0, MOE_EINVAL, "%s: rows=%d K=%d", fn, rows, K);
  if (mode == MOE_Q_FP8_PER_TENSOR) {
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    if (rows == 0) return ok();
    REQUIRE(x && q && scale && workspace, MOE_EINVAL, "%s: null pointer argument", fn);
    REQUIRE(aligned16(x) && ((uintptr_t)q & 7u) == 0 && ((uintptr_t)workspace & 3u) == 0,
            MOE_EINVAL, "%s: x must be 16-byte and q 8-byte aligned", fn);
    return hip_status(qmoe::launch_quant_fp8_tensor_bf16(x, (long long)rows * K, q, scale,
                                                         (float *)workspace, stream),
                      fn);
  }
  if (mode == MOE_Q_INT8_PER_CHANNEL) {                  // activations: one scale per row
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    if (rows == 0) return ok();
    REQUIRE(x && q && scale, MOE_EINVAL, "%s: null pointer argument", fn);
    REQUIRE(aligned16(x) && ((uintptr_t)q & 7u) == 0, MOE_EINVAL,
            "%s: x must be 16-byte and q 8-byte aligned", fn);
    return hip_status(qmoe::launch_quant_int8_rows_bf16(x, rows, K, (int8_t *)q, scale, stream),
                      fn);
  }
  if (mode == MOE_Q_MXFP8) {
    REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d", fn, E);
    REQUIRE(K % 32 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 32", fn, K);
    REQUIRE(rows <= kMxMaxRows, MOE_EUNSUPPORTED, "%s: rows=%d exceeds %d", fn, rows, kMxMaxRows);
    if (rows == 0) return ok();
    REQUIRE(x && q && scale_e8m0 && m_offsets, MOE_EINVAL, "%s: null pointer argument", fn);
    REQUIRE(aligned16(x) && aligned16(q), MOE_EINVAL, "%s: x and q must be 16-byte aligned", fn);
    return hip_status(
        qmoe::launch_quant_mx_act_bf16(x, rows, K, m_offsets, E, q, scale_e8m0, stream), fn);
  }
  return fail(MOE_EINVAL, "%s: unknown mode %d", fn, mode);
}

int moe_quantize_act_noalloc(const uint16_t *x, int rows, int K, int mode, const int *m_offsets,
                             int E, uint8_t *q, float *scale, uint8_t *scale_e8m0,
                             hipStream_t stream) {
  const char *fn = "moe_quantize_act_noalloc";
  if (mode != MOE_Q_FP8_PER_TENSOR)       // the other modes use no scratch
    return moe_quantize_act(x, rows, K, mode, m_offsets, E, q, scale, scale_e8m0, nullptr, stream);
  REQUIRE(rows >= 0 && K > 0, MOE_EINVAL, "%s: rows=%d K=%d", fn, rows, K);
  REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
  const size_t need = moe_quantize_workspace_bytes(mode, 1);
  REQUIRE(need <= sizeof(float) * kScratchFloats, MOE_EUNSUPPORTED,
          "%s: %zu bytes of scratch needed, the static scratch holds %zu", fn, need,
          sizeof(float) * kScratchFloats);
  if (rows == 0) return ok();
  REQUIRE(x && q && scale, MOE_EINVAL, "%s: null pointer argument", fn);
  REQUIRE(aligned16(x) && ((uintptr_t)q & 7u) == 0, MOE_EINVAL,
          "%s: x must be 16-byte and q 8-byte aligned", fn);
  float *ws = nullptr;
  const int rc = scratch_for_current_device(&ws, fn);
  if (rc != MOE_OK) return rc;
  return hip_status(qmoe::launch_quant_fp8_tensor_bf16(x, (long long)rows * K, q, scale, ws, stream),
                    fn);
}

int moe_act_quantize(const uint16_t *x, int rows, int H, int act, int mode, const int *m_offsets,
                     int E, uint8_t *q, float *scale, uint8_t *scale_e8m0, void *workspace,
                     hipStream_t stream) {
  const char *fn = "moe_act_quantize";
  REQUIRE(rows >= 0 && H > 0, MOE_EINVAL, "%s: rows=%d H=%d", fn, rows, H);
  REQUIRE(act == MOE_ACT_SWIGLU || act == MOE_ACT_SRELU, MOE_EINVAL, "%s: unknown activation %d",
          fn, act);
  REQUIRE(mode == MOE_Q_FP8_PER_TENSOR || mode == MOE_Q_MXFP8, MOE_EINVAL, "%s: unknown mode %d",
          fn, mode);
  const int mult = mode == MOE_Q_MXFP8 ? 32 : 8;
  REQUIRE(H % mult == 0, MOE_EUNSUPPORTED, "%s: H=%d is not a multiple of %d", fn, H, mult);
  REQUIRE((long long)rows * H * (act == MOE_ACT_SWIGLU ? 2 : 1) * 2 < (1ll << 40), MOE_EUNSUPPORTED,
          "%s: input too large", fn);
  REQUIRE(rows <= kMxMaxRows, MOE_EUNSUPPORTED, "%s: rows=%d exceeds %d", fn, rows, kMxMaxRows);
  if (mode == MOE_Q_MXFP8) REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d", fn, E);
  if (rows == 0) return ok();
  REQUIRE(x && q, MOE_EINVAL, "%s: null pointer argument", fn);
  if (mode == MOE_Q_MXFP8) {
    REQUIRE(scale_e8m0 && m_offsets, MOE_EINVAL, "%s: null scale or m_offsets", fn);
    REQUIRE(aligned16(x) && aligned16(q), MOE_EINVAL, "%s: x and q must be 16-byte aligned", fn);
  } else {
    REQUIRE(scale && workspace, MOE_EINVAL, "%s: null scale or workspace", fn);
    REQUIRE(aligned16(x) && ((uintptr_t)q & 7u) == 0 && ((uintptr_t)workspace & 3u) == 0,
            MOE_EINVAL, "%s: x must be 16-byte and q 8-byte aligned", fn);
  }
  return hip_status(qmoe::launch_act_quant(x, rows, H, act, mode, m_offsets, E, q, scale,
                                           scale_e8m0, (float *)workspace, stream),
                    fn);
}

int moe_quantize_weights(const float *w, int E, int N, int K, int mode, void *q, float *scale,
                         uint8_t *scale_e8m0, void *workspace, hipStream_t stream) {
  const char *fn = "moe_quantize_weights";
  REQUIRE(E >= 1 && N > 0 && K > 0, MOE_EINVAL, "%s: E=%d N=%d K=%d", fn, E, N, K);
  REQUIRE(w && q, MOE_EINVAL, "%s: null pointer argument", fn);
  REQUIRE(aligned16(w) && ((uintptr_t)q & 7u) == 0, MOE_EINVAL,
          "%s: w must be 16-byte and q 8-byte aligned", fn);
  const long long per = (long long)N * K;
  if (mode == MOE_Q_FP8_PER_TENSOR) {
    REQUIRE(scale && workspace, MOE_EINVAL, "%s: null scale or workspace", fn);
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    REQUIRE(E <= 65535, MOE_EUNSUPPORTED, "%s: E=%d", fn, E);
    return hip_status(qmoe::launch_quant_fp8_experts_f32(w, E, per, (uint8_t *)q, scale,
                                                         (float *)workspace, stream),
                      fn);
  }
  if (mode == MOE_Q_INT4_PER_CHANNEL) {
    REQUIRE(scale, MOE_EINVAL, "%s: null scale", fn);
    REQUIRE(((uintptr_t)q & 3u) == 0, MOE_EINVAL, "%s: q must be 4-byte aligned", fn);
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    return hip_status(qmoe::launch_quant_int4_rows_f32(w, (long long)E * N, K, (uint8_t *)q, scale,
                                                       stream),
                      fn);
  }
  if (mode == MOE_Q_FP8_PER_CHANNEL) {
    REQUIRE(scale, MOE_EINVAL, "%s: null scale", fn);
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    return hip_status(qmoe::launch_quant_fp8_rows_f32(w, (long long)E * N, K, (uint8_t *)q, scale,
                                                      stream),
                      fn);
  }
  if (mode == MOE_Q_INT8_PER_CHANNEL) {
    REQUIRE(scale, MOE_EINVAL, "%s: null scale", fn);
    REQUIRE(K % 8 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    return hip_status(qmoe::launch_quant_int8_rows_f32(w, (long long)E * N, K, (int8_t *)q,
                                                       scale, stream),
                      fn);
  }
  if (mode == MOE_Q_MXFP8_COLWISE) {
    REQUIRE(scale_e8m0, MOE_EINVAL, "%s: null scale_e8m0", fn);
    REQUIRE(aligned16(q), MOE_EINVAL, "%s: q must be 16-byte aligned", fn);
    REQUIRE(N % 128 == 0 && K % 64 == 0, MOE_EUNSUPPORTED,
            "%s: N=%d must be a multiple of 128 and K=%d of 64", fn, N, K);
    REQUIRE((long long)E * N / 128 <= 65535, MOE_EUNSUPPORTED, "%s: E*N too large", fn);
    return hip_status(
        qmoe::launch_mx_colwise_weights(w, E, N, K, (uint8_t *)q, scale_e8m0, stream), fn);
  }
  if (mode == MOE_Q_MXFP8) {
    REQUIRE(scale_e8m0, MOE_EINVAL, "%s: null scale_e8m0", fn);
    REQUIRE(aligned16(q), MOE_EINVAL, "%s: q must be 16-byte aligned", fn);
    REQUIRE(K % 32 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 32", fn, K);
    return hip_status(
        qmoe::launch_quant_mx_rows_f32(w, (long long)E * N, K, (uint8_t *)q, scale_e8m0, stream),
        fn);
  }
  return fail(MOE_EINVAL, "%s: unknown mode %d", fn, mode);
}

int moe_grouped_gemm_fp8w8a8(const uint8_t *a_q, const float *a_scale, const uint8_t *w_q,
                             const float *w_scale, int w_layout, const int *sorted_token_ids,
                             const int *expert_ids, const int *num_tokens_post_padded,
                             const float *topk_weights, int M, int K, int N, int E, int top_k,
                             int block_m, uint16_t *y, hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_fp8w8a8";
  int rc = check_routed_gemm(a_q, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, y, M, K, N, E, top_k, block_m,
                             128, fn);
  if (rc) return rc;
  if (M == 0) return ok();
  REQUIRE(a_scale, MOE_EINVAL, "%s: null a_scale", fn);
  qmoe::RoutedArgs r{sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, M, K, N,
                     E, top_k, block_m, (int)(max_padded_ll(M, E, top_k, block_m) / block_m),
                     w_layout, y};
  return hip_status(qmoe::launch_gemm_fp8(a_q, a_scale, w_q, w_scale, r, stream), fn);
}

int moe_grouped_gemm_fp8w8a16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                              int w_layout, const int *sorted_token_ids, const int *expert_ids,
                              const int *num_tokens_post_padded, const float *topk_weights,
                              int M, int K, int N, int E, int top_k, int block_m, uint16_t *y,
                              hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_fp8w8a16";
  int rc = check_routed_gemm(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, y, M, K, N, E, top_k, block_m,
                             64, fn);
  if (rc) return rc;
  if (M == 0) return ok();
  qmoe::RoutedArgs r{sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, M, K, N,
                     E, top_k, block_m, (int)(max_padded_ll(M, E, top_k, block_m) / block_m),
                     w_layout, y};
  return hip_status(qmoe::launch_gemm_fp8w8a16(a, w_q, w_scale, r, stream), fn);
}

int moe_grouped_gemm_int4w4a16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                               int w_layout, const int *sorted_token_ids, const int *expert_ids,
                               const int *num_tokens_post_padded, const float *topk_weights,
                               int M, int K, int N, int E, int top_k, int block_m, uint16_t *y,
                               hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_int4w4a16";
  int rc = check_routed_gemm(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, y, M, K, N, E, top_k, block_m,
                             128, fn);
  if (rc) return rc;
  REQUIRE(block_m == 16, MOE_EUNSUPPORTED, "%s: block_m=%d (int4 weights: 16 only)", fn, block_m);
  REQUIRE(w_layout != MOE_W_TILED, MOE_EUNSUPPORTED, "%s: MOE_W_TILED is not offered for int4",
          fn);
  if (M == 0) return ok();
  qmoe::RoutedArgs r{sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, M, K, N,
                     E, top_k, block_m, (int)(max_padded_ll(M, E, top_k, block_m) / block_m),
                     w_layout, y};
  return hip_status(qmoe::launch_gemm_int4w16(a, w_q, w_scale, r, stream), fn);
}

int moe_grouped_gemm_int8w8a8(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
                              const float *w_scale, int w_layout, const int *sorted_token_ids,
                              const int *expert_ids, const int *num_tokens_post_padded,
                              const float *topk_weights, int M, int K, int N, int E, int top_k,
                              int block_m, uint16_t *y, hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_int8w8a8";
  int rc = check_routed_gemm(a_q, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, y, M, K, N, E, top_k, block_m,
                             128, fn);
  if (rc) return rc;
  if (M == 0) return ok();
  REQUIRE(a_scale, MOE_EINVAL, "%s: null a_scale", fn);
  qmoe::RoutedArgs r{sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, M, K, N,
                     E, top_k, block_m, (int)(max_padded_ll(M, E, top_k, block_m) / block_m),
                     w_layout, y};
  return hip_status(qmoe::launch_gemm_int8w8a8(a_q, a_scale, w_q, w_scale, r, stream), fn);
}

int moe_grouped_gemm_int8w8a16(const uint16_t *a, const int8_t *w_q, const float *w_scale,
                               int w_layout, const int *sorted_token_ids, const int *expert_ids,
                               const int *num_tokens_post_padded, const float *topk_weights,
                               int M, int K, int N, int E, int top_k, int block_m, uint16_t *y,
                               hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_int8w8a16";
  int rc = check_routed_gemm(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, y, M, K, N, E, top_k, block_m,
                             64, fn);
  if (rc) return rc;
  if (M == 0) return ok();
  qmoe::RoutedArgs r{sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, M, K, N,
                     E, top_k, block_m, (int)(max_padded_ll(M, E, top_k, block_m) / block_m),
                     w_layout, y};
  return hip_status(qmoe::launch_gemm_int8(a, w_q, w_scale, r, stream), fn);
}

int moe_grouped_gemm_mxfp8(const uint8_t *a_q, const uint8_t *a_sf, const uint8_t *w_q,
                           const uint8_t *w_sf, const int *m_offsets, int rows, int K, int N,
                           int E, uint16_t *out, hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_mxfp8";
  REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d", fn, E);
  REQUIRE(rows >= 0 && K > 0 && N > 0, MOE_EINVAL, "%s: rows=%d K=%d N=%d", fn, rows, K, N);
  REQUIRE(a_q && a_sf && w_q && w_sf && m_offsets && out, MOE_EINVAL, "%s: null pointer", fn);
  REQUIRE(aligned16(a_q) && aligned16(w_q) && ((uintptr_t)a_sf & 3u) == 0 &&
              ((uintptr_t)w_sf & 3u) == 0,
          MOE_EINVAL, "%s: data must be 16-byte and scales 4-byte aligned", fn);
  REQUIRE(K % 128 == 0, MOE_EUNSUPPORTED, "%s: K=%d is not a multiple of 128", fn, K);
  REQUIRE(N % 8 == 0, MOE_EUNSUPPORTED, "%s: N=%d is not a multiple of 8", fn, N);
  REQUIRE(aligned16(out), MOE_EINVAL, "%s: out must be 16-byte aligned", fn);
  // every offset inside the kernels is 32-bit: activation codes (with the
  // scale rows padded to 128 per expert), weight codes and the output
  REQUIRE(((long long)rows + (long long)E * 127) * K < (1ll << 32) &&
              (long long)E * N * (long long)K < (1ll << 32) &&
              (long long)rows * N * 2 < kMaxOutBytes,
          MOE_EUNSUPPORTED, "%s: operands and output must stay below 4 GiB", fn);
  if (rows == 0) return ok();
  return hip_status(
      qmoe::launch_gemm_mxfp8(a_q, a_sf, w_q, w_sf, m_offsets, rows, K, N, E, out, stream), fn);
}

int moe_quantize_act_colwise(const uint16_t *x, int rows, int C, const int *m_offsets, int E,
                             uint8_t *qT, uint8_t *sfT, hipStream_t stream) {
  const char *fn = "moe_quantize_act_colwise";
  REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d", fn, E);
  REQUIRE(rows >= 0 && C > 0, MOE_EINVAL, "%s: rows=%d C=%d", fn, rows, C);
  REQUIRE(C % 64 == 0, MOE_EUNSUPPORTED, "%s: C=%d is not a multiple of 64", fn, C);
  REQUIRE((long long)rows + (long long)E * 127 <= 65535ll * 128, MOE_EUNSUPPORTED,
          "%s: rows=%d beyond the supported %d", fn, rows, 65535 * 128 - E * 127);
  REQUIRE(((long long)rows + (long long)E * 127) * C < (1ll << 32), MOE_EUNSUPPORTED,
          "%s: the transposed codes must stay below 4 GiB", fn);
  if (rows == 0) return ok();
  REQUIRE(x && m_offsets && qT && sfT, MOE_EINVAL, "%s: null pointer argument", fn);
  REQUIRE(aligned16(x) && aligned16(qT), MOE_EINVAL, "%s: x and qT must be 16-byte aligned", fn);
  return hip_status(qmoe::launch_mx_colwise_bf16(x, rows, C, m_offsets, E, qT, sfT, stream), fn);
}

int moe_grouped_gemm_mxfp8_wgrad(const uint8_t *dyT_q, const uint8_t *dyT_sf,
                                 const uint8_t *xT_q, const uint8_t *xT_sf, const int *m_splits,
                                 int E, int N, int K, uint16_t *dw, hipStream_t stream) {
  const char *fn = "moe_grouped_gemm_mxfp8_wgrad";
  REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL, "%s: E=%d", fn, E);
  REQUIRE(N > 0 && K > 0, MOE_EINVAL, "%s: N=%d K=%d", fn, N, K);
  REQUIRE(N % 128 == 0 && K % 64 == 0, MOE_EUNSUPPORTED,
          "%s: N=%d must be a multiple of 128 and K=%d of 64", fn, N, K);
  REQUIRE(m_splits && dyT_q && dyT_sf && xT_q && xT_sf && dw, MOE_EINVAL,
          "%s: null pointer argument", fn);
  REQUIRE(aligned16(dyT_q) && aligned16(xT_q) && aligned16(dw) && ((uintptr_t)dyT_sf & 3u) == 0 &&
              ((uintptr_t)xT_sf & 3u) == 0,
          MOE_EINVAL, "%s: codes and output must be 16-byte and scales 4-byte aligned", fn);
  REQUIRE((long long)E * N * (long long)K * 2 < kMaxOutBytes, MOE_EUNSUPPORTED,
          "%s: the weight gradient must stay below 4 GiB", fn);
  long long total = 0;
  for (int e = 0; e < E; ++e) {
    REQUIRE(m_splits[e] >= 0, MOE_EINVAL, "%s: m_splits[%d]=%d", fn, e, m_splits[e]);
    total += (m_splits[e] + 127) / 128 * 128;
  }
  REQUIRE(total * (long long)(N > K ? N : K) < (1ll << 32), MOE_EUNSUPPORTED,
          "%s: the transposed operands must stay below 4 GiB", fn);
  int po[MOE_MAX_EXPERTS + 1];                            // padded row offsets (host)
  po[0] = 0;
  for (int e = 0; e < E; ++e) po[e + 1] = po[e] + (m_splits[e] + 127) / 128 * 128;
  const hipError_t err =
      qmoe::launch_gemm_mxfp8_wgrad(dyT_q, dyT_sf, xT_q, xT_sf, po, E, N, K, dw, stream);
  if (err != hipSuccess) return hip_status(err, fn);
  return ok();
}

int moe_combine(const uint16_t *y, int M, int N, int top_k, uint16_t *out, hipStream_t stream) {
  const char *fn = "moe_combine";
  REQUIRE(M >= 0 && N > 0 && top_k >= 1 && top_k <= MOE_MAX_TOPK, MOE_EINVAL,
          "%s: M=%d N=%d top_k=%d", fn, M, N, top_k);
  REQUIRE(N % 8 == 0, MOE_EUNSUPPORTED, "%s: N=%d is not a multiple of 8", fn, N);
  if (M == 0) return ok();
  REQUIRE(y && out, MOE_EINVAL, "%s: null pointer argument", fn);
  REQUIRE(aligned16(y) && aligned16(out), MOE_EINVAL, "%s: y and out must be 16-byte aligned", fn);
  return hip_status(qmoe::launch_combine(y, M, N, top_k, out, stream), fn);
}

}  // extern "C"
