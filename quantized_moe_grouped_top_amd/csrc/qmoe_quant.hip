// Quantization kernels: dynamic activation quantization (fp8 per tensor,
// MXFP8 with per-expert padded scale blocks) and the offline weight
// quantizers (fp8 per expert, int8 per output channel, MXFP8 per row).
//
// All of them are HBM streams: 16-byte loads, one pass for MXFP8 and int8
// rows, two passes (amax partials, then quantize) for the per-tensor fp8
// scale.  The per-tensor amax is reduced without atomics: every workgroup of
// the first pass writes its partial maximum, and every workgroup of the second
// pass reduces the (at most kAmaxPartials) partials itself, so the result does
// not depend on scheduling and no buffer has to start at zero.
//
// Scales are computed in double and rounded once to float: s = fl32(amax/448)
// and inv = fl32(1/s) (double has more than 2*24+2 bits, so rounding the
// double quotient to float gives the correctly rounded float quotient).
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// 8 consecutive source values as float
__device__ __forceinline__ void load8(const uint16_t *p, float *v) {
  const i32x4 raw = *reinterpret_cast<const i32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, (uint32_t)raw[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)raw[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float *v) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// ---- fp8 per tensor: pass 1, partial amax ------------------------------------
// grid (P, T): tensor t = blockIdx.y covers [t*per, (t+1)*per); per % 8 == 0.
template <typename Src>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(const Src *__restrict__ x,
                                                                 long long per,
                                                                 float *__restrict__ ws) {
  __shared__ float red[kThreads / 64];
  const Src *base = x + (long long)blockIdx.y * per;
  const long long n8 = per / 8;
  float m = 0.0f;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n8;
       i += (long long)gridDim.x * kThreads) {
    float v[8];
    load8(base + i * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) ws[blockIdx.y * kAmaxPartials + blockIdx.x] = m;
}

// ---- fp8 per tensor: pass 2, quantize ------------------------------------------
template <typename Src>
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const Src *__restrict__ x,
                                                             long long per, int parts,
                                                             const float *__restrict__ ws,
                                                             uint8_t *__restrict__ q,
                                                             float *__restrict__ scale) {
  __shared__ float red[kThreads / 64];
  const int t = blockIdx.y;
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kThreads) m = fmaxf(m, ws[t * kAmaxPartials + i]);
  const float amax = block_max(m, red);
  const float s = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[t] = s;

  const Src *src = x + (long long)t * per;
  uint8_t *dst = q + (long long)t * per;
  const long long n8 = per / 8;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n8;
       i += (long long)gridDim.x * kThreads) {
    float v[8];
    load8(src + i * 8, v);
    i32x2 out;
    out[0] = (int)f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out[1] = (int)f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<i32x2 *>(dst + i * 8) = out;
  }
}

// ---- int8 per output channel: one wavefront per row --------------------------
__global__ __launch_bounds__(kThreads) void quant_int8_rows_kernel(const float *__restrict__ w,
                                                                   long long rows, int K,
                                                                   int8_t *__restrict__ q,
                                                                   float *__restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float *src = w + row * K;
  float m = 0.0f;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    float v[8];
    load8(src + k, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  const float amax = wave_max(m);
  const float s = amax > 0.0f ? (float)((double)amax / 127.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (lane == 0) scale[row] = s;
  int8_t *dst = q + row * K;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    float v[8];
    load8(src + k, v);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float r = __builtin_rintf(v[j] * inv);              // round half to even
      r = __builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
      packed[j >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (j & 3));
    }
    i32x2 out = {(int)packed[0], (int)packed[1]};
    *reinterpret_cast<i32x2 *>(dst + k) = out;
  }
}

// ---- MXFP8: one thread per block of 32 values ------------------------------
// Returns the e8m0 byte and writes the 32 e4m3 codes.
template <typename Src>
__device__ __forceinline__ uint32_t mx_block(const Src *src, uint8_t *dst) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) load8(src + 8 * i, v + 8 * i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // shared exponent floor(log2 amax) - 8 as an e8m0 byte, clamped to [0, 254]
  int b = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu) - 8;
  b = b < 0 ? 0 : (b > 254 ? 254 : b);
  // 2^(127-b): exponent field 254-b is in [8, 254] for finite inputs (b <= 246)
  const float f = __builtin_bit_cast(float, (uint32_t)(254 - b) << 23);
  i32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = (int)f32x4_to_e4m3x4(v[4 * i] * f, v[4 * i + 1] * f, v[4 * i + 2] * f, v[4 * i + 3] * f);
    o1[i] = (int)f32x4_to_e4m3x4(v[16 + 4 * i] * f, v[16 + 4 * i + 1] * f, v[16 + 4 * i + 2] * f,
                                 v[16 + 4 * i + 3] * f);
  }
  *reinterpret_cast<i32x4 *>(dst) = o0;
  *reinterpret_cast<i32x4 *>(dst + 16) = o1;
  return (uint32_t)b;
}

// Activations with per-expert scale blocks padded to 128 rows.  Work item =
// (padded scale row p, block kb); pad rows only get a zero scale byte.
__global__ __launch_bounds__(kThreads) void quant_mx_act_kernel(
    const uint16_t *__restrict__ x, int rows, int K, const int *__restrict__ m_offsets, int E,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sf, long long work_bound) {
  __shared__ int s_mo[kMaxExperts + 1];
  __shared__ int s_po[kMaxExperts + 1];
  for (int e = threadIdx.x; e <= E; e += kThreads) s_mo[e] = m_offsets[e];
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      s_po[e] = acc;
      acc += (s_mo[e + 1] - s_mo[e] + kMxRowPad - 1) / kMxRowPad * kMxRowPad;
    }
    s_po[E] = acc;
  }
  __syncthreads();
  const int nb = K / kMxBlock;
  const long long work = (long long)s_po[E] * nb;
  const long long lim = work < work_bound ? work : work_bound;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < lim;
       i += (long long)gridDim.x * kThreads) {
    const int p = (int)(i / nb);
    const int kb = (int)(i - (long long)p * nb);
    int lo = 0, hi = E - 1;                       // last e with s_po[e] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_po[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int local = p - s_po[lo];
    uint32_t b = 0;
    const long long r = (long long)s_mo[lo] + local;
    if (local < s_mo[lo + 1] - s_mo[lo] && r >= 0 && r < rows) {
      b = mx_block(x + r * K + kb * kMxBlock, q + r * K + kb * kMxBlock);
    }
    sf[(long long)p * nb + kb] = (uint8_t)b;
  }
}

// Rows without padding (weights [E*N, K]).
__global__ __launch_bounds__(kThreads) void quant_mx_rows_kernel(const float *__restrict__ w,
                                                                 long long rows, int K,
                                                                 uint8_t *__restrict__ q,
                                                                 uint8_t *__restrict__ sf) {
  const int nb = K / kMxBlock;
  const long long work = rows * nb;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < work;
       i += (long long)gridDim.x * kThreads) {
    const long long r = i / nb;
    const int kb = (int)(i - r * nb);
    sf[i] = (uint8_t)mx_block(w + r * K + kb * kMxBlock, q + r * K + kb * kMxBlock);
  }
}

// ---- weight re-layout for streaming: one thread per 16-byte chunk ----------
// Block (e, t, s) of 64 rows x 128 bytes, rows in order, chunk c of row r at
// position c ^ ((r >> 1) & 7); rows >= N and k >= K are zero.
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(const uint8_t *__restrict__ w,
                                                                int E, int N, int K,
                                                                uint8_t *__restrict__ packed) {
  const int T = (N + kPackRows - 1) / kPackRows;
  const int S = (K + kPackK - 1) / kPackK;
  const long long chunks = (long long)E * T * S * (kPackRows * kPackK / 16);
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < chunks;
       i += (long long)gridDim.x * kThreads) {
    const long long b = i >> 9;                       // 512 chunks per 8 KB block
    const int within = (int)(i & 511);
    const int r = within >> 3;
    const int c = (within & 7) ^ ((r >> 1) & 7);
    const int s_ = (int)(b % S);
    const int t = (int)((b / S) % T);
    const int e = (int)(b / ((long long)S * T));
    const int n = t * kPackRows + r;
    const int k0 = s_ * kPackK + 16 * c;
    i32x4 v = {0, 0, 0, 0};
    if (n < N && k0 < K) v = *reinterpret_cast<const i32x4 *>(w + ((long long)e * N + n) * K + k0);
    *reinterpret_cast<i32x4 *>(packed + i * 16) = v;
  }
}

int grid_for(long long items, int cap) {
  long long g = (items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_quant_fp8_tensor_bf16(const uint16_t *x, long long numel, uint8_t *q,
                                        float *scale, float *ws, hipStream_t s) {
  const int parts = grid_for(numel / 8, kAmaxPartials);
  hipLaunchKernelGGL(amax_partials_kernel<uint16_t>, dim3(parts, 1), dim3(kThreads), 0, s, x,
                     numel, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(quant_fp8_kernel<uint16_t>, dim3(grid_for(numel / 8, 8192), 1),
                     dim3(kThreads), 0, s, x, numel, parts, ws, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_experts_f32(const float *w, int E, long long per, uint8_t *q,
                                        float *scale, float *ws, hipStream_t s) {
  const int parts = grid_for(per / 8, kAmaxPartials);
  hipLaunchKernelGGL(amax_partials_kernel<float>, dim3(parts, E), dim3(kThreads), 0, s, w, per,
                     ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(quant_fp8_kernel<float>, dim3(grid_for(per / 8, 4096), E), dim3(kThreads),
                     0, s, w, per, parts, ws, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_int8_rows_f32(const float *w, long long rows, int K, int8_t *q,
                                      float *scale, hipStream_t s) {
  const long long blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(quant_int8_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, w,
                     rows, K, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_mx_act_bf16(const uint16_t *x, int rows, int K, const int *m_offsets,
                                    int E, uint8_t *q, uint8_t *sf, hipStream_t s) {
  const long long bound = ((long long)rows + (long long)E * (kMxRowPad - 1)) * (K / kMxBlock);
  hipLaunchKernelGGL(quant_mx_act_kernel, dim3(grid_for(bound, 16384)), dim3(kThreads), 0, s, x,
                     rows, K, m_offsets, E, q, sf, bound);
  return hipGetLastError();
}

hipError_t launch_quant_mx_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                    uint8_t *sf, hipStream_t s) {
  hipLaunchKernelGGL(quant_mx_rows_kernel, dim3(grid_for(rows * (K / kMxBlock), 16384)),
                     dim3(kThreads), 0, s, w, rows, K, q, sf);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const uint8_t *w, int E, int N, int K, uint8_t *packed,
                               hipStream_t s) {
  const long long chunks = (long long)E * ((N + kPackRows - 1) / kPackRows) *
                           ((K + kPackK - 1) / kPackK) * (kPackRows * kPackK / 16);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(chunks, 16384)), dim3(kThreads), 0, s, w,
                     E, N, K, packed);
  return hipGetLastError();
}

}  // namespace qmoe
