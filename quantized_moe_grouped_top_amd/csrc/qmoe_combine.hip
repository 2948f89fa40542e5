// Per-token combine of the routed results: out[t, n] = bf16(sum_j y[t*top_k+j, n])
// with the adds in float32 in slot order and the sum rounded to nearest even.
// An HBM stream: each thread handles 4 columns (16-byte loads, 8-byte stores).
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ y, int M,
                                                           int N, int top_k,
                                                           uint16_t *__restrict__ out) {
  const int n4 = N / 4;
  const long long work = (long long)M * n4;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < work;
       i += (long long)gridDim.x * kThreads) {
    const long long t = i / n4;
    const int c = (int)(i - t * n4) * 4;
    const float *src = y + (t * top_k) * (long long)N + c;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(src);
    for (int j = 1; j < top_k; ++j) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src + (long long)j * N);
      acc[0] = acc[0] + v[0];
      acc[1] = acc[1] + v[1];
      acc[2] = acc[2] + v[2];
      acc[3] = acc[3] + v[3];
    }
    i32x2 o = {(int)f32x2_to_bf16x2(acc[0], acc[1]), (int)f32x2_to_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<i32x2 *>(out + t * N + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const float *y, int M, int N, int top_k, uint16_t *out,
                          hipStream_t s) {
  const long long work = (long long)M * (N / 4);
  long long g = (work + kThreads - 1) / kThreads;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, y, M, N, top_k,
                     out);
  return hipGetLastError();
}

}  // namespace qmoe
