// Device helpers shared by the grouped-GEMM sources of libqmoe.so: the
// direct-to-LDS DMA instructions, exact waits on the vector-memory counter,
// the block ranges of each expert in the aligned routing layout, and the
// format tags of the tiled GEMM kernels.
#pragma once

#include "qmoe_internal.h"

namespace qmoe {

constexpr int kXcds = 8;   // accelerator complex dies; workgroups are dealt to them round robin

// A pointer the same in every lane, in scalar registers.
static __device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// global_load_lds_dwordx4: lane l copies 16 bytes from sbase + voff to LDS
// byte address m0 + 16*l.
static __device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// global_load_lds_dword: lane l copies 4 bytes from sbase + voff to LDS byte
// address m0 + 4*l.
static __device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

static __device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63] (0 for anything else)
static __device__ __forceinline__ void wait_dma_upto(int n) {
  switch (n) {
#define QMOE_W(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
#define QMOE_W8(b) QMOE_W(b) QMOE_W(b + 1) QMOE_W(b + 2) QMOE_W(b + 3) QMOE_W(b + 4) QMOE_W(b + 5) \
    QMOE_W(b + 6) QMOE_W(b + 7)
    QMOE_W(1) QMOE_W(2) QMOE_W(3) QMOE_W(4) QMOE_W(5) QMOE_W(6) QMOE_W(7)
    QMOE_W8(8) QMOE_W8(16) QMOE_W8(24) QMOE_W8(32) QMOE_W8(40) QMOE_W8(48) QMOE_W8(56)
#undef QMOE_W8
#undef QMOE_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// First block of every expert, from the ascending block labels: s_first[e] =
// first b with expert_ids[b] >= e, for e in [0, E]; s_first[E] is the number
// of blocks in use.  The labels are scanned over the whole buffer (max_blocks
// entries, -1 after the last block), so the padded length is not needed first.
// All threads of the workgroup take part (a few loads each, no serial search);
// the caller synchronises before reading s_first.
static __device__ __forceinline__ void expert_block_starts(const int *__restrict__ expert_ids,
                                                    int max_blocks, int E, int *s_first) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) s_first[e] = max_blocks;
  __syncthreads();
  constexpr int kEnd = 1 << 30;                     // the -1 label sorts after every expert
  for (int b = threadIdx.x; b < max_blocks; b += blockDim.x) {
    int cur = expert_ids[b];
    int prev = b > 0 ? expert_ids[b - 1] : -1;
    cur = cur < 0 ? kEnd : cur;
    prev = (b > 0 && prev < 0) ? kEnd : prev;
    for (int e = prev + 1; e <= cur && e <= E; ++e) s_first[e] = b;
  }
}

// Byte weights -> bf16 MFMA operands, exactly (int8: |v| <= 128 fits the
// 8-bit bf16 significand; e4m3: 3 mantissa bits, exponents -9..8).
// 4 signed bytes -> 4 bf16 packed in two dwords (exact: |v| <= 128 fits the
// 8-bit bf16 significand)
static __device__ __forceinline__ i32x2 i8x4_to_bf16x4(uint32_t d) {
  const float f0 = (float)(int)(int8_t)(d & 0xFFu);
  const float f1 = (float)(int)(int8_t)((d >> 8) & 0xFFu);
  const float f2 = (float)(int)(int8_t)((d >> 16) & 0xFFu);
  const float f3 = (float)(int)((int32_t)d >> 24);
  return i32x2{(int)f32x2_to_bf16x2(f0, f1), (int)f32x2_to_bf16x2(f2, f3)};
}

// 16 int8 (k0+16g .. +15) -> two bf16x8 operands (first 8 k, last 8 k)
static __device__ __forceinline__ void dequant16(const i32x4 &w, i32x4 &b0, i32x4 &b1) {
  const i32x2 p0 = i8x4_to_bf16x4((uint32_t)w[0]);
  const i32x2 p1 = i8x4_to_bf16x4((uint32_t)w[1]);
  const i32x2 p2 = i8x4_to_bf16x4((uint32_t)w[2]);
  const i32x2 p3 = i8x4_to_bf16x4((uint32_t)w[3]);
  b0 = i32x4{p0[0], p0[1], p1[0], p1[1]};
  b1 = i32x4{p2[0], p2[1], p3[0], p3[1]};
}

// 16 e4m3 weights -> 16 bf16 values (exact: e4m3 has 3 mantissa bits), in
// the same order as dequant16.
static __device__ __forceinline__ void dequant16_fp8(const i32x4 &w, i32x4 &b0, i32x4 &b1) {
  int p[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[d], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[d], true);
    p[2 * d] = (int)f32x2_to_bf16x2(lo[0], lo[1]);
    p[2 * d + 1] = (int)f32x2_to_bf16x2(hi[0], hi[1]);
  }
  b0 = i32x4{p[0], p[1], p[2], p[3]};
  b1 = i32x4{p[4], p[5], p[6], p[7]};
}
template <bool kFp8W>
static __device__ __forceinline__ void dequant16w(const i32x4 &w, i32x4 &b0, i32x4 &b1) {
  if constexpr (kFp8W) dequant16_fp8(w, b0, b1);
  else dequant16(w, b0, b1);
}

// One word of dequant16w's output: bytes 2h and 2h + 1 of weight dword d as a
// bf16 pair (word 2d' + h of the eight, d' being d's index in the fragment).
template <bool kFp8W>
static __device__ __forceinline__ int dequant_pair(uint32_t d, int h) {
  if constexpr (kFp8W) {
    const f32x2 v = h ? __builtin_amdgcn_cvt_pk_f32_fp8((int)d, true)
                      : __builtin_amdgcn_cvt_pk_f32_fp8((int)d, false);
    return (int)f32x2_to_bf16x2(v[0], v[1]);
  } else {
    const float f0 = (float)(int)(int8_t)((d >> (16 * h)) & 0xFFu);
    const float f1 = (float)((int32_t)(d << (16 - 16 * h)) >> 24);
    return (int)f32x2_to_bf16x2(f0, f1);
  }
}

// grouped-GEMM formats of the tiled kernels
enum { kFmtFp8 = 0, kFmtInt8 = 1, kFmtMx = 2, kFmtI8 = 3, kFmtF8W16 = 4, kFmtMxW = 5 };

// MXFP8 weight gradient: the padded row offset of every expert's columnwise
// operands (P_e; P_E is the total), passed by value
struct WgradSeg {
  int po[kMaxExperts + 1];
};

// Operands of the 256 x 256 tile GEMM (qmoe_gemm_tile.hip).  Routed formats
// (fp8 W8A8, int8 W8A8): rows are the sorted slots of 128-row routing blocks,
// outputs the bf16 per-slot results y [M*top_k, N].  MXFP8: rows are the
// experts' contiguous segments (m_offsets), outputs bf16 rows; the weight
// gradient takes its segments from WgradSeg (M = output rows per expert).
struct TileArgs {
  const uint8_t *a;            // activation codes [rows, K] (weight gradient: dyT blocks)
  const float *a_scale;        // fp8: [1]; int8 W8A8: one per token
  const uint8_t *a_sf;         // MXFP8 activation scale bytes
  const uint8_t *w;            // weight codes [E, N, K] or MOE_W_TILED blocks
  const float *w_scale;        // fp8: [E]; int8 W8A8: [E, N]
  const uint8_t *w_sf;         // MXFP8 weight scale bytes
  const int *sorted_ids;
  const int *expert_ids;
  const float *topk_w;
  const int *m_offsets;        // MXFP8: [E + 1] device offsets, or null for one segment
  uint16_t *out;
  uint32_t out_bytes;          // size of `out` (below 0xFFFFFF00)
  int M, K, N, E, top_k, max_blocks;
};

// Launch of the tile GEMM for format kFmtFp8, kFmtI8, kFmtMx or kFmtMxW (K a
// multiple of 128; routed formats: block_m 128).  tiles_bound bounds the
// number of 256 x 256 tiles (it sizes the persistent grid).
hipError_t launch_tile_gemm(int fmt, bool tiled, const TileArgs &args, const WgradSeg *seg,
                            long long tiles_bound, hipStream_t s);

}  // namespace qmoe
