// Internal declarations shared by the HIP sources of libqmoe.so: vector types,
// small device helpers and the host-side launchers that the C ABI
// (qmoe_api.cpp) calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace qmoe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxExperts = 128;
constexpr int kMaxTopK = 8;
constexpr int kMaxSlots = 65536;
constexpr int kAmaxPartials = 1024;   // per-tensor amax partial results (floats)
constexpr int kMxBlock = 32;
constexpr int kMxRowPad = 128;
constexpr int kPackRows = 64;         // tiled weight layout: rows per tile
constexpr int kPackK = 128;           // tiled weight layout: bytes of k per slice


// Saturate to the e4m3 range so the conversion below can never overflow.
__device__ __forceinline__ float sat448(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Four float32 -> four e4m3 bytes packed little-endian in one dword (round to
// nearest even after saturation to +-448; v_cvt_pk_fp8_f32).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// float32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}


// ---- launchers (return the launch status; all arguments already validated) --
hipError_t launch_route_align(const float *logits, int M, int E, int top_k, int block_m,
                              int max_padded, int *topk_ids, float *topk_w,
                              int *sorted_ids, int *expert_ids, int *num_post,
                              hipStream_t s);

hipError_t launch_quant_fp8_tensor_bf16(const uint16_t *x, long long numel, uint8_t *q,
                                        float *scale, float *ws, hipStream_t s);
hipError_t launch_quant_fp8_experts_f32(const float *w, int E, long long per_expert,
                                        uint8_t *q, float *scale, float *ws, hipStream_t s);
hipError_t launch_quant_int8_rows_f32(const float *w, long long rows, int K, int8_t *q,
                                      float *scale, hipStream_t s);
hipError_t launch_quant_int4_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                      float *scale, hipStream_t s);
hipError_t launch_quant_fp8_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                     float *scale, hipStream_t s);
hipError_t launch_quant_int8_rows_bf16(const uint16_t *x, long long rows, int K, int8_t *q,
                                       float *scale, hipStream_t s);
hipError_t launch_quant_mx_act_bf16(const uint16_t *x, int rows, int K, const int *m_offsets,
                                    int E, uint8_t *q, uint8_t *sf, hipStream_t s);
hipError_t launch_act_quant(const uint16_t *x, int rows, int H, int act, int mode,
                            const int *m_offsets, int E, uint8_t *q, float *scale, uint8_t *sf,
                            float *ws, hipStream_t s);
hipError_t launch_quant_mx_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                    uint8_t *sf, hipStream_t s);

struct RoutedArgs {
  const int *sorted_ids;
  const int *expert_ids;
  const int *num_post;
  const float *topk_w;
  int M, K, N, E, top_k, block_m, max_blocks;
  int w_layout;                        // MOE_W_ROWMAJOR, MOE_W_TILED or MOE_W_FRAG
  uint16_t *y;                  // bf16 per-slot results [M*top_k, N]
};

hipError_t launch_gemm_fp8(const uint8_t *a_q, const float *a_scale, const uint8_t *w_q,
                           const float *w_scale, const RoutedArgs &r, hipStream_t s);
hipError_t launch_gemm_int8(const uint16_t *a, const int8_t *w_q, const float *w_scale,
                            const RoutedArgs &r, hipStream_t s);
hipError_t launch_gemm_mxfp8_wgrad(const uint8_t *dyT_q, const uint8_t *dyT_sf, const uint8_t *xT_q,
                                   const uint8_t *xT_sf, const int *padded_offsets, int E, int N,
                                   int K, uint16_t *dw, hipStream_t s);
hipError_t launch_gemm_int4w16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                               const RoutedArgs &r, hipStream_t s);
hipError_t launch_gemm_fp8w8a16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                                const RoutedArgs &r, hipStream_t s);
hipError_t launch_gemm_int8w8a8(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
                               const float *w_scale, const RoutedArgs &r, hipStream_t s);
hipError_t launch_gemm_mxfp8(const uint8_t *a_q, const uint8_t *a_sf, const uint8_t *w_q,
                             const uint8_t *w_sf, const int *m_offsets, int rows, int K,
                             int N, int E, uint16_t *out, hipStream_t s);

hipError_t launch_mx_colwise_bf16(const uint16_t *x, int rows, int C, const int *m_offsets,
                                  int E, uint8_t *qT, uint8_t *sfT, hipStream_t s);
hipError_t launch_mx_colwise_weights(const float *w, int E, int N, int K, uint8_t *qT,
                                     uint8_t *sfT, hipStream_t s);
hipError_t launch_pack_weights(const uint8_t *w, int E, int N, int K, int layout, uint8_t *packed,
                               hipStream_t s);

hipError_t launch_combine(const uint16_t *y, int M, int N, int top_k, uint16_t *out,
                          hipStream_t s);

}  // namespace qmoe
