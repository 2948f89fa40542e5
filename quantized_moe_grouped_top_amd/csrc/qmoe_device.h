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
