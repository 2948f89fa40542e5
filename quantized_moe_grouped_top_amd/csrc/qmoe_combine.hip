// Per-token combine of the routed results: out[t, n] = bf16(sum_j y[t*top_k+j, n])
// over the bf16 per-slot results, with the adds in float32 in slot order and
// the sum rounded to nearest even.  An HBM stream: each thread handles 8
// columns (16-byte loads and stores, with the non-temporal hint: every byte
// is read or written once).
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(int v) { return __int_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(int v) { return __int_as_float(v & (int)0xFFFF0000u); }

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t *__restrict__ y, int M,
                                                           int N, int top_k,
                                                           uint16_t *__restrict__ out) {
  const int n8 = N / 8;
  const long long work = (long long)M * n8;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < work;
       i += (long long)gridDim.x * kThreads) {
    const long long t = i / n8;
    const int c = (int)(i - t * n8) * 8;
    const uint16_t *src = y + (t * top_k) * (long long)N + c;
    // every slot's load is issued before the first is used (one memory
    // latency per token instead of top_k)
    i32x4 v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < top_k) v[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(src + (long long)j * N));
    float acc[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = bf16_lo(v[0][q]);
      acc[2 * q + 1] = bf16_hi(v[0][q]);
    }
#pragma unroll
    for (int j = 1; j < kMaxTopK; ++j) {
      if (j >= top_k) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = acc[2 * q] + bf16_lo(v[j][q]);
        acc[2 * q + 1] = acc[2 * q + 1] + bf16_hi(v[j][q]);
      }
    }
    i32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (int)f32x2_to_bf16x2(acc[2 * q], acc[2 * q + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<i32x4 *>(out + t * N + c));
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t *y, int M, int N, int top_k, uint16_t *out,
                          hipStream_t s) {
  const long long work = (long long)M * (N / 8);
  long long g = (work + kThreads - 1) / kThreads;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, y, M, N, top_k,
                     out);
  return hipGetLastError();
}

}  // namespace qmoe
