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

// 8 bf16 values (16 bytes) as float
__device__ __forceinline__ void unpack8(const i32x4 raw, float *v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, (uint32_t)raw[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)raw[i] & 0xFFFF0000u);
  }
}

// 8 consecutive source values as float
__device__ __forceinline__ void load8(const uint16_t *p, float *v) {
  unpack8(*reinterpret_cast<const i32x4 *>(p), v);
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

// Raw 16- or 32-byte loads of 8 consecutive values and their conversion, so
// that several loads can be issued before the first is used.
template <typename Src> struct Raw8;
template <> struct Raw8<uint16_t> { i32x4 a; };
template <> struct Raw8<float> { f32x4 a, b; };
__device__ __forceinline__ Raw8<uint16_t> ld8(const uint16_t *p) {
  return {*reinterpret_cast<const i32x4 *>(p)};
}
__device__ __forceinline__ Raw8<float> ld8(const float *p) {
  return {*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
}
__device__ __forceinline__ void cvt8(const Raw8<uint16_t> &r, float *v) { unpack8(r.a, v); }
__device__ __forceinline__ void cvt8(const Raw8<float> &r, float *v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = r.a[i];
    v[4 + i] = r.b[i];
  }
}

constexpr int kFlatUnroll = 4;     // 8-value items in flight per thread

// ---- fp8 per tensor: pass 1, partial amax ------------------------------------
// grid (P, T): tensor t = blockIdx.y covers [t*per, (t+1)*per); per % 8 == 0.
// Thread i takes the 8-value items i, i + stride, ... (stride = all threads of
// the tensor), kFlatUnroll of them loaded before any is used.
template <typename Src>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(const Src *__restrict__ x,
                                                                 long long per,
                                                                 float *__restrict__ ws) {
  __shared__ float red[kThreads / 64];
  const Src *base = x + (long long)blockIdx.y * per;
  const long long n8 = per / 8;
  const long long stride = (long long)gridDim.x * kThreads;
  float m = 0.0f;
  for (long long i0 = blockIdx.x * (long long)kThreads + threadIdx.x; i0 < n8;
       i0 += kFlatUnroll * stride) {
    Raw8<Src> raw[kFlatUnroll];
#pragma unroll
    for (int j = 0; j < kFlatUnroll; ++j)
      if (i0 + j * stride < n8) raw[j] = ld8(base + (i0 + j * stride) * 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kFlatUnroll; ++j) {
      if (i0 + j * stride < n8) {
        float v[8];
        cvt8(raw[j], v);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
      }
    }
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
  const Src *src = x + (long long)t * per;
  uint8_t *dst = q + (long long)t * per;
  const long long n8 = per / 8;
  const long long stride = (long long)gridDim.x * kThreads;
  auto load_round = [&](long long r0, Raw8<Src> (&raw)[kFlatUnroll]) {
#pragma unroll
    for (int j = 0; j < kFlatUnroll; ++j)
      if (r0 + j * stride < n8) raw[j] = ld8(src + (r0 + j * stride) * 8);
  };
  // the first round's loads do not depend on the scale: they are in flight
  // while the partial maxima are reduced
  long long i0 = blockIdx.x * (long long)kThreads + threadIdx.x;
  Raw8<Src> raw[kFlatUnroll];
  load_round(i0, raw);
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kThreads) m = fmaxf(m, ws[t * kAmaxPartials + i]);
  const float amax = block_max(m, red);
  const float s = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[t] = s;

  for (; i0 < n8; i0 += kFlatUnroll * stride) {
#pragma unroll
    for (int j = 0; j < kFlatUnroll; ++j) {
      const long long i = i0 + j * stride;
      if (i < n8) {
        float v[8];
        cvt8(raw[j], v);
        i32x2 out;
        out[0] = (int)f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        out[1] = (int)f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        *reinterpret_cast<i32x2 *>(dst + i * 8) = out;
      }
    }
    load_round(i0 + kFlatUnroll * stride, raw);
  }
}

// ---- int8 per row (weights: per output channel; activations: per token):
// one wavefront per row ----------------------------------------------------------
template <typename Src>
__global__ __launch_bounds__(kThreads) void quant_int8_rows_kernel(const Src *__restrict__ w,
                                                                   long long rows, int K,
                                                                   int8_t *__restrict__ q,
                                                                   float *__restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const Src *src = w + row * K;
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

// ---- int4 per output channel (int4 weight-only): one wavefront per row -----
// Codes q = clamp(rne(w * fl32(1/s)), -7, 7) with s = fl32(amax/7), stored as
// q + 8 in 4-bit fields: the 8 codes of k = 8c .. 8c+7 form dword c of the
// row, value j in field (j >> 1) + 4 (j & 1).
__global__ __launch_bounds__(kThreads) void quant_int4_rows_kernel(const float *__restrict__ w,
                                                                   long long rows, int K,
                                                                   uint8_t *__restrict__ q,
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
  const float s = amax > 0.0f ? (float)((double)amax / 7.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (lane == 0) scale[row] = s;
  uint32_t *dst = reinterpret_cast<uint32_t *>(q + row * (K / 2));
  for (int k = lane * 8; k < K; k += 64 * 8) {
    float v[8];
    load8(src + k, v);
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float r = __builtin_rintf(v[j] * inv);              // round half to even
      r = __builtin_amdgcn_fmed3f(r, -7.0f, 7.0f);
      const uint32_t field = (uint32_t)((j >> 1) + 4 * (j & 1));
      word |= ((uint32_t)((int)r + 8) & 0xFu) << (4u * field);
    }
    dst[k / 8] = word;
  }
}

// ---- fp8 per output channel (fp8 weight-only): one wavefront per row -------
__global__ __launch_bounds__(kThreads) void quant_fp8_rows_kernel(const float *__restrict__ w,
                                                                  long long rows, int K,
                                                                  uint8_t *__restrict__ q,
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
  const float s = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (lane == 0) scale[row] = s;
  uint8_t *dst = q + row * K;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    float v[8];
    load8(src + k, v);
    i32x2 out;
    out[0] = (int)f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out[1] = (int)f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<i32x2 *>(dst + k) = out;
  }
}

// ---- MXFP8: one thread per block of 32 values ------------------------------
// mx_encode: the e8m0 byte of 32 values (returned) and their 32 e4m3 codes.
__device__ __forceinline__ uint32_t mx_encode(const float *v, uint8_t *dst) {
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
  __builtin_nontemporal_store(o0, reinterpret_cast<i32x4 *>(dst));   // written once
  __builtin_nontemporal_store(o1, reinterpret_cast<i32x4 *>(dst + 16));
  return (uint32_t)b;
}

// ---- MXFP8 along the rows (columnwise scales), stored transposed ----------
// For expert e its rows are padded with zeros to Rp_e = roundup(m_e, 128);
// column c, rows 32j .. 32j+31 of the padded segment form one block.  Output,
// expert by expert (P_e = sum of Rp of the experts before e): codes at
// C * P_e + c * Rp_e + row, scale bytes at C * P_e / 32 + c * Rp_e / 32 + j.
// A workgroup takes one padded 128-row chunk of one expert x 64 columns: the
// tile is read row by row (16 bytes per lane: 8 lanes per bf16 row, 16 per
// float row; coalesced) into
// LDS transposed (a row of LDS per column), then thread (c, j) encodes block
// j of column c from LDS and four neighbouring threads write the column's
// 128 codes as one contiguous 128-byte run.
constexpr int kColwiseCols = 64;                    // columns per workgroup

template <typename Src> struct ColwiseRaw;
template <> struct ColwiseRaw<uint16_t> {
  static constexpr int kPerLane = 8;                // 8 bf16 of one row per lane
  static constexpr int kPad = 8;                    // row stride 272 bytes (16-byte aligned)
};
template <> struct ColwiseRaw<float> {
  static constexpr int kPerLane = 4;                // 4 floats of one row per lane
  static constexpr int kPad = 4;                    // row stride 528 bytes
};
__device__ __forceinline__ void put_row(float (*t)[kMxRowPad + ColwiseRaw<float>::kPad], int c, int r,
                                        const f32x4 &v) {
  t[c][r] = v[0];
  t[c + 1][r] = v[1];
  t[c + 2][r] = v[2];
  t[c + 3][r] = v[3];
}
__device__ __forceinline__ void get32(const uint16_t *p, float *v) {   // 32 bf16, 16-byte aligned
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(*reinterpret_cast<const i32x4 *>(p + 8 * i), v + 8 * i);
}
__device__ __forceinline__ void get32(const float *p, float *v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 q = *reinterpret_cast<const f32x4 *>(p + 4 * i);
    v[4 * i] = q[0];
    v[4 * i + 1] = q[1];
    v[4 * i + 2] = q[2];
    v[4 * i + 3] = q[3];
  }
}

template <typename Src>
__global__ __launch_bounds__(kThreads) void mx_colwise_kernel(const Src *__restrict__ x, int C,
                                                              const int *__restrict__ m_offsets,
                                                              int E, int uniform_rows,
                                                              uint8_t *__restrict__ qT,
                                                              uint8_t *__restrict__ sfT) {
  using R = ColwiseRaw<Src>;
  static_assert(kThreads == 256, "64 columns x 4 blocks: one thread each");
  __shared__ long long s_po[kMaxExperts + 1];               // padded start of each expert
  __shared__ int s_mo[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) Src s_t[kColwiseCols][kMxRowPad + R::kPad];
  if (threadIdx.x == 0) {
    long long acc = 0;
    for (int e = 0; e <= E; ++e) {
      // uniform_rows > 0: E segments of uniform_rows rows (weights), no m_offsets
      s_mo[e] = uniform_rows > 0 ? e * uniform_rows : m_offsets[e];
      s_po[e] = acc;
      if (e < E) {
        const int m = uniform_rows > 0 ? uniform_rows : m_offsets[e + 1] - m_offsets[e];
        acc += (long long)(m + kMxRowPad - 1) / kMxRowPad * kMxRowPad;
      }
    }
  }
  __syncthreads();
  const long long pr = (long long)kMxRowPad * blockIdx.y;   // padded row of this chunk
  if (pr >= s_po[E]) return;                                // (uniform over the workgroup)
  int e = 0;
  while (s_po[e + 1] <= pr) ++e;
  const long long rp = s_po[e + 1] - s_po[e];
  const int c0 = blockIdx.x * kColwiseCols;
  const long long row0 = s_mo[e] + (pr - s_po[e]);          // first data row of the chunk
  const long long rend = s_mo[e + 1];
  // load (16 bytes per lane, the non-temporal hint: the input is read once)
  if constexpr (R::kPerLane == 8) {
    // bf16: thread t reads rows rb = 4 (t / 8) .. rb + 3, columns
    // c0 + 8 (t % 8) .. + 7 (eight lanes cover a row's 128 bytes) and writes
    // each column's four values as one 8-byte run of its transposed row
    const int cg = 8 * (int)(threadIdx.x & 7);
    const int rb = 4 * (int)(threadIdx.x >> 3);
    i32x4 v4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4[q] = i32x4{0, 0, 0, 0};
      if (row0 + rb + q < rend)
        v4[q] = __builtin_nontemporal_load(
            reinterpret_cast<const i32x4 *>(x + (row0 + rb + q) * C + c0 + cg));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // column cg + k: the low (k even) or high (k odd) half of dword k / 2
      // of each row, two rows per dword
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      i32x2 w;
      w[0] = (int)__builtin_amdgcn_perm((uint32_t)v4[1][k >> 1], (uint32_t)v4[0][k >> 1], sel);
      w[1] = (int)__builtin_amdgcn_perm((uint32_t)v4[3][k >> 1], (uint32_t)v4[2][k >> 1], sel);
      *reinterpret_cast<i32x2 *>(&s_t[cg + k][rb]) = w;
    }
  } else {
    // float: row r = tid / 16 + 16 i, columns c0 + 4 (tid % 16) .. + 3
    constexpr int P = R::kPerLane, L = kColwiseCols / P, RS = kThreads / L;
    const int cg = P * (int)(threadIdx.x % L);
#pragma unroll
    for (int i = 0; i < kMxRowPad / RS; ++i) {
      const int r = (int)(threadIdx.x / L) + RS * i;
      f32x4 v{};
      if (row0 + r < rend)
        v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + (row0 + r) * C + c0 + cg));
      put_row(s_t, cg, r, v);
    }
  }
  __syncthreads();
  const int c = (int)(threadIdx.x >> 2), j = (int)(threadIdx.x & 3);
  float v[kMxBlock];
  get32(&s_t[c][kMxBlock * j], v);
  const size_t base = (size_t)C * (size_t)s_po[e];
  const size_t col = (size_t)(c0 + c);
  const long long j0 = pr - s_po[e] + kMxBlock * j;          // row in the padded segment
  const uint32_t b = mx_encode(v, qT + base + col * (size_t)rp + (size_t)j0);
  sfT[base / kMxBlock + col * (size_t)(rp / kMxBlock) + (size_t)(j0 / kMxBlock)] = (uint8_t)b;
}

template <typename Src>
__device__ __forceinline__ uint32_t mx_block(const Src *src, uint8_t *dst) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) load8(src + 8 * i, v + 8 * i);
  return mx_encode(v, dst);
}

// ---- fused activations (float32 arithmetic on bf16 inputs) -------------------
// SwiGLU: y = silu(g) * u with silu(g) = g / (1 + exp(-g)), the gate g in the
// first half of the row and u in the second; SReLU: y = max(x, 0)^2 (exact).
//
// silu in a few instructions: exp(-g) = 2^t with t = -g * log2(e) carried as
// an unevaluated sum t_hi + t_lo (t_lo from an fma residual and the low part
// of log2(e)).  The hardware exp2 takes t_hi and the residual enters to first
// order, 2^(t_hi + t_lo) = 2^t_hi * (1 + t_lo * ln 2) up to t_lo^2 < 2^-32.
// The exponent uses g clamped to [-128, 128]: exp(-g) is already 0 or
// infinite in float32 there, so nothing changes except that t_lo stays finite
// (the result is then g * u or a signed zero).  With the hardware reciprocal
// of 1 + 2^t the relative error stays within about 7 float32 units.
__device__ __forceinline__ float silu_mul(float g, float u) {
  constexpr float kLog2e = 1.44269502162933349609375f;     // float32 nearest log2(e)
  constexpr float kLog2eLo = 1.9259629911266175e-8f;       // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147182464599609375f;
  const float gc = __builtin_amdgcn_fmed3f(g, -128.0f, 128.0f);
  const float t = -gc * kLog2e;
  const float t_lo = fmaf(-gc, kLog2e, -t) - gc * kLog2eLo;
  const float e = __builtin_amdgcn_exp2f(t) * (1.0f + t_lo * kLn2);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <int kAct>
__device__ __forceinline__ void act8(const uint16_t *row, int H, int col, float *y) {
  if constexpr (kAct == MOE_ACT_SWIGLU) {
    float gt[8], up[8];
    load8(row + col, gt);
    load8(row + H + col, up);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = silu_mul(gt[i], up[i]);
  } else {
    float v[8];
    load8(row + col, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = fmaxf(v[i], 0.0f);
      y[i] = r * r;
    }
  }
}

// 16-byte load, with the non-temporal hint for data read once
template <bool kNT>
__device__ __forceinline__ i32x4 ld16(const uint16_t *p) {
  if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p));
  else return *reinterpret_cast<const i32x4 *>(p);
}

// Sources of the padded-row MXFP8 kernel.  load() fetches the raw bytes of 8
// consecutive values of row r from column col (col % 8 == 0), with the
// non-temporal hint when kNT (a pass that reads its input once); values()
// turns them into the 8 float values.  The kernel issues the loads of kUnroll
// chunks before it converts any, so they are in flight together.
struct Bf16Rows {
  static constexpr int kUnroll = 2;
  struct Raw { i32x4 a; };
  const uint16_t *x;
  int K;
  template <bool kNT = false>
  __device__ __forceinline__ Raw load(long long r, int col) const {
    return {ld16<kNT>(x + r * K + col)};
  }
  __device__ __forceinline__ void values(const Raw &raw, float *v) const { unpack8(raw.a, v); }
};
template <int kAct> struct ActRaw { i32x4 a, b; };           // SwiGLU: gate, up
template <> struct ActRaw<MOE_ACT_SRELU> { i32x4 a; };

template <int kAct>
struct ActRows {                   // activation of rows of width 2H (SwiGLU) or H
  static constexpr int kUnroll = kAct == MOE_ACT_SWIGLU ? 1 : 2;
  using Raw = ActRaw<kAct>;
  const uint16_t *x;
  int H;
  template <bool kNT = false>
  __device__ __forceinline__ Raw load(long long r, int col) const {
    Raw raw;
    if constexpr (kAct == MOE_ACT_SWIGLU) {
      const uint16_t *row = x + r * 2ll * H;
      raw.a = ld16<kNT>(row + col);
      raw.b = ld16<kNT>(row + H + col);
    } else {
      raw.a = ld16<kNT>(x + r * (long long)H + col);
    }
    return raw;
  }
  __device__ __forceinline__ void values(const Raw &raw, float *v) const {
    if constexpr (kAct == MOE_ACT_SWIGLU) {
      float g[8], u[8];
      unpack8(raw.a, g);
      unpack8(raw.b, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = silu_mul(g[i], u[i]);
    } else {
      unpack8(raw.a, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = fmaxf(v[i], 0.0f);
        v[i] = t * t;
      }
    }
  }
};

// max over the four lanes of a quad (lanes 4a .. 4a+3), by DPP quad
// permutations (xor 1, then xor 2); every lane of the quad must be active.
__device__ __forceinline__ float quad_max(float m) {
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m),
                                                                  0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m),
                                                                  0x4E, 0xF, 0xF, false)));
  return m;
}

__device__ __forceinline__ uint32_t e8m0_of_amax(float amax) {
  // shared exponent floor(log2 amax) - 8 as an e8m0 byte, clamped to [0, 254]
  const int b = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu) - 8;
  return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// One 8-value chunk of a 32-value block whose other chunks sit in the three
// neighbouring lanes (lanes 4a .. 4a+3): the block amax is reduced over the
// four lanes, the codes are stored, and the block's scale byte is returned.
__device__ __forceinline__ uint32_t mx_chunk(const float *v, uint8_t *dst) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = quad_max(m);
  const uint32_t b = e8m0_of_amax(m);
  const float f = __builtin_bit_cast(float, (254u - b) << 23);   // 2^(127 - b)
  i32x2 o;
  o[0] = (int)f32x4_to_e4m3x4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
  o[1] = (int)f32x4_to_e4m3x4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
  __builtin_nontemporal_store(o, reinterpret_cast<i32x2 *>(dst));
  return b;
}

// MXFP8 of expert-concatenated rows [rows, K] with the scale rows of each
// expert padded to a multiple of 128 (pad rows get zero scale bytes).
//
// Rows per workgroup step: R = 1 when a row has at least kThreads 8-value
// chunks, else R = kThreads / (K/8); thread t owns local row t / (K/8) and the
// chunks c8 = t % (K/8), + kThreads, ..., so the workgroup reads one
// contiguous span of the input per load instruction and the rows in flight
// stay close together in memory.  A workgroup takes S consecutive steps
// before striding on (S steps fill a 128-byte line of scale bytes, so one L2
// writes the whole line).  Four neighbouring threads hold one 32-value block
// (K % 32 == 0), whose amax is reduced over the quad.
//
// Software pipeline: the first kUnroll chunks of the next row are loaded
// before the current row is encoded, so a thread always has loads in flight.
// Each thread finds the expert of its rows by a forward scan (its rows only
// grow).
template <class Src>
__global__ __launch_bounds__(kThreads) void mx_padded_kernel(
    Src src, int rows, int K, const int *__restrict__ m_offsets, int E,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sf, int prow_bound) {
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
  const int n8 = K / 8, nb = K / kMxBlock;
  const int R = n8 >= kThreads ? 1 : kThreads / n8;
  const int lr = n8 >= kThreads ? 0 : (int)threadIdx.x / n8;
  const int c0 = (int)threadIdx.x - lr * n8;
  if (lr >= R) return;                            // whole quads of spare threads
  const int S = R * nb >= 128 ? 1 : 128 / (R * nb);
  const int prows = s_po[E] < prow_bound ? s_po[E] : prow_bound;
  constexpr int U = Src::kUnroll;
  using Raw = typename Src::Raw;

  // k-th row of this thread: step k % S of unit blockIdx.x + (k / S) * gridDim.x
  auto row_of = [&](int k) {
    return (blockIdx.x + (k / S) * gridDim.x) * (R * S) + (k % S) * R + lr;
  };
  int e = 0;
  auto source_row = [&](int p, long long &r) {    // is padded row p a real row, which
    while (e < E - 1 && s_po[e + 1] <= p) ++e;
    const int local = p - s_po[e];
    r = (long long)s_mo[e] + local;
    return local >= 0 && local < s_mo[e + 1] - s_mo[e] && r >= 0 && r < rows;
  };
  // The first U chunks of row r.  The loads are unconditional (chunks past the
  // row end reload chunk c0, a dead row loads row 0, which exists as rows > 0)
  // so that every step has the same number of loads in flight and the waits
  // before the encode can leave the next row's loads outstanding.
  auto load_head = [&](long long r, Raw *raw) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = c0 + kThreads * j < n8 ? c0 + kThreads * j : c0;
      raw[j] = src.template load<true>(r, 8 * c);
    }
  };
  auto encode = [&](int c8, const Raw &raw, uint8_t *q_row, uint8_t *sf_row) {
    float v[8];
    src.values(raw, v);
    const uint32_t b = mx_chunk(v, q_row + 8 * c8);
    if ((c8 & 3) == 0) sf_row[c8 >> 2] = (uint8_t)b;
  };

  // One pipeline step: issue the loads of the next row into `nxt`, then
  // encode the current row from `cur`.  Steps alternate between two buffers
  // so that no register copy forces a wait on the loads in flight.
  int k = 0;
  int p = row_of(0);
  if (p >= prows) return;
  long long r;
  bool live = source_row(p, r);
  auto step = [&](Raw *cur, Raw *nxt) {
    const int pn = row_of(k + 1);
    const bool has_next = pn < prows;
    long long rn = 0;
    const bool live_n = has_next && source_row(pn, rn);
    load_head(live_n ? rn : 0, nxt);
    __builtin_amdgcn_sched_barrier(0);            // next row's loads go out first
    uint8_t *sf_row = sf + (long long)p * nb;
    if (live) {
      uint8_t *q_row = q + r * K;
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (c0 + kThreads * j < n8) encode(c0 + kThreads * j, cur[j], q_row, sf_row);
      for (int c8 = c0 + kThreads * U; c8 < n8; c8 += kThreads)
        encode(c8, src.template load<true>(r, 8 * c8), q_row, sf_row);
    } else {
      for (int c8 = c0; c8 < n8; c8 += kThreads)
        if ((c8 & 3) == 0) sf_row[c8 >> 2] = 0;
    }
    p = pn;
    r = rn;
    live = live_n;
    ++k;
    return has_next;
  };
  Raw buf_a[U], buf_b[U];
  load_head(live ? r : 0, buf_a);
  while (step(buf_a, buf_b) && step(buf_b, buf_a)) {
  }
}

// Fused activation + fp8 per tensor.  Both passes run one wavefront per row
// (lane l takes the 8-value chunks l, l + 64, ...) with U chunks loaded
// before any is used.  Pass 1: partial amax of the activation, one per
// workgroup.
template <int kAct, int U>
__global__ __launch_bounds__(kThreads) void act_amax_kernel(ActRows<kAct> src, int rows,
                                                            float *__restrict__ ws) {
  __shared__ float red[kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int n8 = src.H / 8;
  const int waves = gridDim.x * (kThreads / 64);
  float m = 0.0f;
  for (int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows; r += waves) {
    int c8 = lane;
    for (; c8 + 64 * (U - 1) < n8; c8 += 64 * U) {
      typename ActRows<kAct>::Raw raw[U];
#pragma unroll
      for (int j = 0; j < U; ++j) raw[j] = src.load(r, 8 * (c8 + 64 * j));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        float y[8];
        src.values(raw[j], y);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(y[k]));
      }
    }
    for (; c8 < n8; c8 += 64) {
      float y[8];
      src.values(src.load(r, 8 * c8), y);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(y[k]));
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) ws[blockIdx.x] = m;
}

// Pass 2: reduce the partials, recompute the activation and quantize it.
template <int kAct, int U>
__global__ __launch_bounds__(kThreads) void act_fp8_kernel(ActRows<kAct> src, int rows, int parts,
                                                           const float *__restrict__ ws,
                                                           uint8_t *__restrict__ q,
                                                           float *__restrict__ scale) {
  __shared__ float red[kThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kThreads) m = fmaxf(m, ws[i]);
  const float amax = block_max(m, red);
  const float s = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
  const float inv = (float)(1.0 / (double)s);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  const int lane = threadIdx.x & 63;
  const int H = src.H, n8 = H / 8;
  const int waves = gridDim.x * (kThreads / 64);
  auto encode = [&](const typename ActRows<kAct>::Raw &raw, uint8_t *dst) {
    float y[8];
    src.values(raw, y);
    i32x2 out;
    out[0] = (int)f32x4_to_e4m3x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
    out[1] = (int)f32x4_to_e4m3x4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
    __builtin_nontemporal_store(out, reinterpret_cast<i32x2 *>(dst));
  };
  // rows in the reverse of pass 1's order: the rows pass 1 read last are the
  // likeliest to be still in the memory-side cache
  for (int i = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); i < rows; i += waves) {
    const int r = rows - 1 - i;
    uint8_t *q_row = q + (long long)r * H;
    int c8 = lane;
    for (; c8 + 64 * (U - 1) < n8; c8 += 64 * U) {
      typename ActRows<kAct>::Raw raw[U];
#pragma unroll
      for (int j = 0; j < U; ++j) raw[j] = src.template load<true>(r, 8 * (c8 + 64 * j));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < U; ++j) encode(raw[j], q_row + 8 * (c8 + 64 * j));
    }
    for (; c8 < n8; c8 += 64) encode(src.template load<true>(r, 8 * c8), q_row + 8 * c8);
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

// ---- MOE_W_FRAG: one thread per 16-byte piece ----------------------------
// Block (e, j, b) of 1 KB at ((e B + b) J + j) KB, piece p = 16q + r holding
// row 16j + r, k = 64b + 16q .. +15; rows >= N and k >= K are zero.
__global__ __launch_bounds__(kThreads) void pack_frag_kernel(const uint8_t *__restrict__ w, int E,
                                                             int N, int K,
                                                             uint8_t *__restrict__ packed) {
  const int J = (N + 15) / 16, B = (K + 63) / 64;
  const long long pieces = (long long)E * J * B * 64;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < pieces;
       i += (long long)gridDim.x * kThreads) {
    const long long blk = i >> 6;
    const int p = (int)(i & 63);
    const int j = (int)(blk % J);
    const int b = (int)((blk / J) % B);
    const int e = (int)(blk / ((long long)B * J));
    const int n = 16 * j + (p & 15);
    const int k0 = 64 * b + 16 * (p >> 4);
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
  const int grid = grid_for(numel / 8 / kFlatUnroll, 2048);   // one round of loads per thread
  hipLaunchKernelGGL(quant_fp8_kernel<uint16_t>, dim3(grid, 1), dim3(kThreads), 0, s, x, numel,
                     parts, ws, q, scale);
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
  hipLaunchKernelGGL(quant_int8_rows_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     w, rows, K, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_int4_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                      float *scale, hipStream_t s) {
  const long long blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(quant_int4_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, w, rows,
                     K, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                     float *scale, hipStream_t s) {
  const long long blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(quant_fp8_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, w, rows,
                     K, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_int8_rows_bf16(const uint16_t *x, long long rows, int K, int8_t *q,
                                       float *scale, hipStream_t s) {
  const long long blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(quant_int8_rows_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, x, rows, K, q, scale);
  return hipGetLastError();
}

// Workgroups of the padded-row MXFP8 kernel: one per R-row step, at most
// kMxGrid (they stride beyond that).
constexpr int kMxGrid = 8192;
static unsigned mx_padded_grid(int prow_bound, int K) {
  const int n8 = K / 8;
  const int R = n8 >= kThreads ? 1 : kThreads / n8;
  const int blocks = (prow_bound + R - 1) / R;
  return (unsigned)(blocks < kMxGrid ? (blocks > 0 ? blocks : 1) : kMxGrid);
}

hipError_t launch_quant_mx_act_bf16(const uint16_t *x, int rows, int K, const int *m_offsets,
                                    int E, uint8_t *q, uint8_t *sf, hipStream_t s) {
  const int prow_bound = rows + E * (kMxRowPad - 1);
  hipLaunchKernelGGL(mx_padded_kernel<Bf16Rows>, dim3(mx_padded_grid(prow_bound, K)), dim3(kThreads),
                     0, s, Bf16Rows{x, K}, rows, K, m_offsets, E, q, sf, prow_bound);
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t *x, int rows, int H, int act, int mode,
                            const int *m_offsets, int E, uint8_t *q, float *scale, uint8_t *sf,
                            float *ws, hipStream_t s) {
  if (mode == MOE_Q_MXFP8) {
    const int prow_bound = rows + E * (kMxRowPad - 1);
    const dim3 grid(mx_padded_grid(prow_bound, H));
    if (act == MOE_ACT_SWIGLU)
      hipLaunchKernelGGL(mx_padded_kernel<ActRows<MOE_ACT_SWIGLU>>, grid, dim3(kThreads), 0, s,
                         ActRows<MOE_ACT_SWIGLU>{x, H}, rows, H, m_offsets, E, q, sf, prow_bound);
    else
      hipLaunchKernelGGL(mx_padded_kernel<ActRows<MOE_ACT_SRELU>>, grid, dim3(kThreads), 0, s,
                         ActRows<MOE_ACT_SRELU>{x, H}, rows, H, m_offsets, E, q, sf, prow_bound);
    return hipGetLastError();
  }
  // pass 1: one workgroup per 4 rows up to kAmaxPartials workgroups; pass 2:
  // one wavefront per row (grid-stride beyond 16384 workgroups)
  const long long row_blocks = ((long long)rows + 3) / 4;
  const int parts = (int)(row_blocks < kAmaxPartials ? row_blocks : kAmaxPartials);
  const int blocks2 = (int)(row_blocks < 16384 ? row_blocks : 16384);
  if (act == MOE_ACT_SWIGLU) {
    const ActRows<MOE_ACT_SWIGLU> src{x, H};
    hipLaunchKernelGGL((act_amax_kernel<MOE_ACT_SWIGLU, 4>), dim3(parts), dim3(kThreads), 0, s,
                       src, rows, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((act_fp8_kernel<MOE_ACT_SWIGLU, 2>), dim3(blocks2), dim3(kThreads), 0, s,
                       src, rows, parts, ws, q, scale);
  } else {
    const ActRows<MOE_ACT_SRELU> src{x, H};
    hipLaunchKernelGGL((act_amax_kernel<MOE_ACT_SRELU, 8>), dim3(parts), dim3(kThreads), 0, s,
                       src, rows, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((act_fp8_kernel<MOE_ACT_SRELU, 4>), dim3(blocks2), dim3(kThreads), 0, s,
                       src, rows, parts, ws, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_quant_mx_rows_f32(const float *w, long long rows, int K, uint8_t *q,
                                    uint8_t *sf, hipStream_t s) {
  hipLaunchKernelGGL(quant_mx_rows_kernel, dim3(grid_for(rows * (K / kMxBlock), 16384)),
                     dim3(kThreads), 0, s, w, rows, K, q, sf);
  return hipGetLastError();
}

hipError_t launch_mx_colwise_bf16(const uint16_t *x, int rows, int C, const int *m_offsets,
                                  int E, uint8_t *qT, uint8_t *sfT, hipStream_t s) {
  // chunks of 128 padded rows: at most (rows + E * 127) / 128 of them
  const long long chunks = ((long long)rows + (long long)E * (kMxRowPad - 1)) / kMxRowPad;
  if (chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mx_colwise_kernel<uint16_t>, dim3((unsigned)(C / kColwiseCols), (unsigned)chunks),
                     dim3(kThreads), 0, s, x, C, m_offsets, E, 0, qT, sfT);
  return hipGetLastError();
}

hipError_t launch_mx_colwise_weights(const float *w, int E, int N, int K, uint8_t *qT,
                                     uint8_t *sfT, hipStream_t s) {
  // w [E, N, K] as E segments of N rows (N % 128 == 0) and K columns
  const long long chunks = (long long)E * N / kMxRowPad;
  hipLaunchKernelGGL(mx_colwise_kernel<float>, dim3((unsigned)(K / kColwiseCols), (unsigned)chunks),
                     dim3(kThreads), 0, s, w, K, nullptr, E, N, qT, sfT);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const uint8_t *w, int E, int N, int K, int layout,
                               uint8_t *packed, hipStream_t s) {
  if (layout == MOE_W_FRAG) {
    const long long pieces = (long long)E * ((N + 15) / 16) * ((K + 63) / 64) * 64;
    hipLaunchKernelGGL(pack_frag_kernel, dim3(grid_for(pieces, 16384)), dim3(kThreads), 0, s, w, E,
                       N, K, packed);
    return hipGetLastError();
  }
  const long long chunks = (long long)E * ((N + kPackRows - 1) / kPackRows) *
                           ((K + kPackK - 1) / kPackK) * (kPackRows * kPackK / 16);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(chunks, 16384)), dim3(kThreads), 0, s, w,
                     E, N, K, packed);
  return hipGetLastError();
}

}  // namespace qmoe
