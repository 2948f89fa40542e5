// Grouped GEMMs of the quantized MoE layer on CDNA4 MFMA (gfx950), with the
// fused epilogue (dequantization scales x router weight, written per routed
// slot).
//
// MFMA operand convention used throughout.  For a 16x16 output tile, lane l of
// the wavefront owns row (l & 15) of the A operand and column (l & 15) of the
// B operand; lane group g = l >> 4 owns a quarter of the k values of one
// instruction, with the same k assignment for A and B:
//   - fp8 / MXFP8 (v_mfma_f32_16x16x128_f8f6f4 and its scaled form): lane
//     group g holds k0 + 16g .. k0 + 16g + 15 in its first 16 bytes and
//     k0 + 64 + 16g .. k0 + 64 + 16g + 15 in its last 16 bytes.  With this
//     placement the 32 k of scale block s (k0 + 32s .. k0 + 32s + 31) sit in
//     lane groups 2(s%2) and 2(s%2)+1, and the scaled instruction takes the
//     e8m0 scale of (row or column l & 15, block s) from lane group s - the
//     hardware pairing of scale lanes and data lanes, measured on gfx950
//     (one 16-byte half of a lane belongs to a different block than the other);
//   - bf16 (v_mfma_f32_16x16x32_bf16): lane group g holds the 16 values
//     k0 + 16g .. k0 + 16g + 15, split over two instructions (first 8, then
//     last 8), for A and for B.
// The accumulator tile has column (l & 15) and rows 4*(l >> 4) + 0..3 in lane l.
//
// Kernels in this file:
//   stream_kernel (routed, block_m = 16): weight streaming for few rows per
//                   expert (decode).  One persistent workgroup per CU owns an
//                   expert and up to 7 of its 64-column tiles; each lane
//                   loads exactly the weight pieces of its MFMA operands from
//                   HBM into registers (buffer loads, up to three 128-k
//                   stages ahead), so weight bytes are read once and never
//                   pass through LDS; the expert's rows arrive in LDS by
//                   direct-to-LDS DMA.
//   gemm_big_kernel (routed fp8, block_m = 128, fewer than 256 rows per
//                   expert): 256 x 256 tiles on eight wavefronts of 128 x 64,
//                   operands DMA'd into an LDS ring.
//   gemm_kernel   (routed int8 W8A16 and fp8 weight-only, block_m = 128,
//                   fewer than 256 rows per expert): 128 x 256 tiles on eight
//                   wavefronts, weights converted to bf16 in registers for
//                   the bf16 MFMA.
// The routed GEMMs at block_m 128 with at least 256 routed rows per expert
// (int8 W8A8: always) and the MXFP8 grouped linear (forward and weight
// gradient) run the 256 x 256 tile kernel of qmoe_gemm_tile.hip.
// Routed results are written per slot as bf16; MXFP8 rows as bf16.

#include "qmoe_device.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_mx(const i32x8 &a, const i32x8 &b, f32x4 c, int sa,
                                         int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// int8 x int8 -> int32 on two 16x16x64 MFMAs (the 32 bytes of a lane's
// fragment as two 16-byte halves; A and B use the same k placement, and an
// integer dot product does not depend on the order of its terms).  The
// accumulator is carried in float registers as raw int32 bits.
__device__ __forceinline__ f32x4 mfma_i8(const i32x8 &a, const i32x8 &b, f32x4 c) {
  i32x4 ci = __builtin_bit_cast(i32x4, c);
  ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_shufflevector(a, a, 0, 1, 2, 3),
                                             __builtin_shufflevector(b, b, 0, 1, 2, 3), ci, 0, 0, 0);
  ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_shufflevector(a, a, 4, 5, 6, 7),
                                             __builtin_shufflevector(b, b, 4, 5, 6, 7), ci, 0, 0, 0);
  return __builtin_bit_cast(f32x4, ci);
}
__device__ __forceinline__ f32x4 mfma_bf16(const i32x4 &a, const i32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 ld16(const void *p) {
  return *reinterpret_cast<const i32x4 *>(p);
}


// =============================================================================
// block_m = 16: weight streaming
// =============================================================================
// One persistent workgroup per CU.  Workgroup b handles expert e = b / groups
// and G <= 7 of that expert's 64-column tiles (strided, see below; 4G groups
// of 16 weight rows), with up to 64 of the expert's rows per pass.  Wavefront w
// owns the row groups w, w + 8, w + 16 and w + 24 (those below 4G): every
// wavefront owns whole output elements, so no partial sums meet.
//
// No wavefront reads another's weights, so the weights go straight from HBM
// into the registers that feed the MFMAs, SCfg::kD stages (128 k each) ahead of
// their use: for each of its row groups a lane loads the two 16-byte pieces
// that the MFMA operand placement assigns to it (weight row 16j + (l & 15),
// k = 16g .. 16g + 15 and 64 + 16g .. 64 + 16g + 15 of the stage).  A
// wavefront thus keeps up to kD x 8 KB of weights in flight without any LDS,
// and the HBM stream never drains at a stage boundary.  With the MOE_W_FRAG
// layout every such load is one contiguous 1 KB block.  The activation rows,
// which all wavefronts share, flow into a ring of kD + 1 LDS slots by
// global_load_lds_dwordx4 (direct-to-LDS DMA), also kD stages ahead.  Before
// a stage is read each wavefront waits until its own loads of that stage have
// landed (s_waitcnt vmcnt with the number of loads it has issued since) and
// the workgroup synchronises.
//
// LDS activation rows are XOR-swizzled by 16-byte chunk so that the 16 rows
// one MFMA operand read touches fall on distinct banks.
constexpr int kSMB = 4;          // 16-row blocks per pass (64 rows)
constexpr int kSThreads = 512;   // 8 wavefronts
constexpr int kSWaves = kSThreads / 64;
constexpr int kSMaxTiles = 7;    // tiles per workgroup
constexpr int kSK = 128;         // k per stage
constexpr int kSGroups = 4;      // 16-row weight groups per wavefront
// a buffer offset past the end of the weight tensor (below 4 GiB; a tensor
// within 16 bytes of that size would be read in range, harmlessly): a load
// there reads nothing and returns zeros; its data are never used
constexpr uint32_t kNoLoad = 0xFFFFFFF0u;

template <bool kInt8, int kMB>
struct SCfg {
  // weight stages held in registers per wavefront (loads run up to kD stages
  // ahead of the MFMAs); the bf16 path with 64 rows per pass needs the
  // registers of the third stage for its operands (with three stages and
  // those operands it runs slower, measured)
  static constexpr int kD = (kInt8 && kMB > 2) ? 2 : 3;
  static constexpr int kAS = kD + 1;                        // activation ring slots
  static constexpr int kSub = kInt8 ? 64 : 128;            // k per MFMA sub-step
  static constexpr int kARow = kInt8 ? 2 * kSK : kSK;       // activation bytes per row per stage
  static constexpr int kABytes = 16 * kMB * kARow;          // one ring slot
  static constexpr int kAInstr = kABytes / 1024;            // DMA instructions for the rows
};


// 128-byte rows: 16-byte chunk c of row r sits at chunk c ^ swz(r);
// 256-byte rows: at chunk c ^ (r & 15).  With these, the MFMA fragment reads
// (ds_read_b128, lane group g of 16 rows at one chunk index each) run free of
// LDS bank conflicts on gfx950 (measured with SQ_LDS_BANK_CONFLICT: so does
// c ^ (r & 7) on 128-byte rows, while e.g. c ^ ((r & 7) ^ ((r >> 3) & 1))
// conflicts two ways).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int sw128(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }
__device__ __forceinline__ int sw256(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// stream kernel modes: fp8 W8A8, int8 W8A16 (bf16 activations), int8 W8A8
// (int8 activations with one scale per token), fp8 weight-only (bf16
// activations, e4m3 weights with one scale per channel)
enum { kSFp8 = 0, kSW8A16 = 1, kSI8 = 2, kSF8W16 = 3, kSW4A16 = 4 };

// int4 weights (two per byte, stored as q + 8 in 4-bit fields; each group of
// 8 consecutive k forms one little-endian dword with value j in field
// (j >> 1) + 4 (j & 1)): one dword -> the 8 bf16 values 136 + q of an MFMA
// operand.  OR-ing a field into the bf16 pattern of 128 gives 128 + (q + 8)
// exactly (the significand holds 7 bits), two values per instruction pair;
// the constant 136 times the row sum of the activations is taken off after
// the contraction.
__device__ __forceinline__ i32x4 int4x8_to_bf16x8(uint32_t d) {
  constexpr uint32_t kMask = 0x000F000Fu, kBase = 0x43004300u;   // bf16 128.0 in both halves
  return i32x4{(int)((d & kMask) | kBase), (int)(((d >> 4) & kMask) | kBase),
               (int)(((d >> 8) & kMask) | kBase), (int)(((d >> 12) & kMask) | kBase)};
}
constexpr float kInt4Offset = 136.0f;

template <int kMode, int kLayout, int kMB>
__global__ __launch_bounds__(kSThreads, 1) void stream_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ w, const float *__restrict__ w_scale,
    const int *__restrict__ sorted_ids, const int *__restrict__ expert_ids,
    const int *__restrict__ num_post, const float *__restrict__ topk_w, int M, int K, int N,
    int top_k, int groups, int tiles_per_group, int max_blocks, uint16_t *__restrict__ y,
    uint32_t w_bytes) {
  constexpr bool kInt8 = kMode == kSW8A16 || kMode == kSF8W16 || kMode == kSW4A16;   // bf16 acts
  constexpr bool kI8 = kMode == kSI8;                    // int8 activations and weights
  constexpr bool kW4 = kMode == kSW4A16;                 // int4 weights: 64 bytes per row per stage
  constexpr int kP = kW4 ? 1 : 2;                        // 16-byte weight pieces per group and stage
  using C = SCfg<kInt8, kMB>;
  constexpr int kSD = kW4 ? 3 : C::kD, kSAS = kSD + 1;
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kSAS * C::kABytes];
  __shared__ int s_slot[kMB * 16];
  __shared__ int s_nvalid;
  __shared__ float s_scale[kSMaxTiles * 64];
  __shared__ float s_rw[kMB * 16];
  __shared__ float s_A[kMB * 16];                       // int4: activation row sums

  const int e = blockIdx.x / groups;
  const int grp = blockIdx.x - e * groups;
  const int ntiles = (N + 63) / 64;
  // this workgroup's tiles: grp, grp + groups, grp + 2 groups, ... (strided,
  // so that each workgroup's weight stream spreads over the expert's columns)
  const int G = min(tiles_per_group, (ntiles - grp + groups - 1) / groups);
  auto tile_at = [&](int m) { return grp + groups * m; };
  const int tid = threadIdx.x, lane = tid & 63;
  // the wavefront index, in a scalar register (the compiler cannot tell that
  // tid >> 6 is the same in every lane), so that the per-wavefront group
  // loops below branch on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int S = M * top_k;
  if (G <= 0) return;

  const uint32_t lds_ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_ring;
  const uint32_t a_row_bytes = kInt8 ? (uint32_t)K * 2 : (uint32_t)K;
  const int nst = (K + kSK - 1) / kSK;                      // stages
  const int nsub_last = (K - (nst - 1) * kSK) / C::kSub;    // sub-steps of the last stage
  const int ngr = 4 * G;                                    // row groups of the workgroup

  // ---- this lane's weight pieces.  Group u of this wavefront is row group
  // jg = wave + 8u of the workgroup: weight rows 64 tile_at(jg / 4) +
  // 16 (jg % 4) + 0..15, this lane's row r16 of them.  A wavefront with fewer
  // than four groups still issues four groups' loads per stage (so that every
  // wavefront's wait counts are the same), those of the groups it does not
  // own at an offset past the end of the buffer, which read nothing and
  // return zeros.
  // The loads are buffer loads: a per-lane offset that stays fixed over the
  // stages (the lane's row and k group) plus a wavefront-uniform stage offset
  // in a scalar register, checked against the size of the weight tensor (a
  // piece past its end reads as zero; pieces past the last k of a row are
  // never used).
  // int4 weights are a byte matrix [E, N, K/2] (MOE_W_ROWMAJOR) or its
  // MOE_W_FRAG packing; one stage (128 k) is 64 bytes of a row, one 16-byte
  // piece per lane (k 32g .. 32g + 31).
  const int row_bytes = kW4 ? K / 2 : K;
  const int KB = (row_bytes + 63) / 64;                     // MOE_W_FRAG: 64-byte blocks per row group
  const int N16 = (N + 15) / 16;
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)w, (short)0, (int)w_bytes, 0x00020000);
  uint32_t voff[kSGroups][2];
#pragma unroll
  for (int u = 0; u < kSGroups; ++u) {
    const bool owned = wave + kSWaves * u < ngr;
    const int jg = min(wave + kSWaves * u, ngr - 1);
    const int tile = tile_at(jg >> 2);
    const int n = tile * 64 + 16 * (jg & 3) + r16;          // may be >= N in the last tile
    if constexpr (kLayout == MOE_W_ROWMAJOR) {
      const uint32_t row =
          ((uint32_t)e * (uint32_t)N + (uint32_t)min(n, N - 1)) * (uint32_t)row_bytes;
      voff[u][0] = row + 16u * (uint32_t)g;
      voff[u][1] = row + 64u + 16u * (uint32_t)g;
    } else if constexpr (kLayout == MOE_W_TILED) {
      const uint32_t row = ((uint32_t)e * (uint32_t)ntiles + (uint32_t)tile) * (uint32_t)nst * 8192u +
                           (uint32_t)(16 * (jg & 3) + r16) * 128u;
      voff[u][0] = row + (uint32_t)((g ^ swz(r16)) << 4);         // (swz(16q + r) = swz(r))
      voff[u][1] = row + (uint32_t)(((g + 4) ^ swz(r16)) << 4);
    } else {
      const uint32_t blk = ((uint32_t)e * (uint32_t)KB * (uint32_t)N16 +
                            (uint32_t)min(n >> 4, N16 - 1)) * 1024u + 16u * (uint32_t)lane;
      voff[u][0] = blk;
      voff[u][1] = blk + (uint32_t)N16 * 1024u;
    }
    if (!owned) voff[u][0] = voff[u][1] = kNoLoad;
  }
  // byte offset of stage st, the same for every lane
  auto st_off = [&](int st) -> int {
    if constexpr (kLayout == MOE_W_ROWMAJOR) return (kW4 ? kSK / 2 : kSK) * st;
    else if constexpr (kLayout == MOE_W_TILED) return 8192 * st;
    else return (kW4 ? 1024 : 2048) * N16 * st;
  };
  // The weight loads carry the non-temporal hint (each byte is read once):
  // measured 4-5% faster at int8 W8A16 / int8 W8A8 / fp8 M=64-128 than
  // ordinary loads.  A stage past the last one (issued so that every step
  // has the same loads in flight) reads nothing, as above.
  i32x4 wb[kSD][kSGroups][kP];
  auto load_w = [&](int st, i32x4 (&buf)[kSGroups][kP]) {
    if (st < nst) {
      const int so = st_off(st);
#pragma unroll
      for (int u = 0; u < kSGroups; ++u)
#pragma unroll
        for (int h = 0; h < kP; ++h)
          buf[u][h] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, voff[u][h], so, 2);
    } else {
#pragma unroll
      for (int u = 0; u < kSGroups; ++u)
#pragma unroll
        for (int h = 0; h < kP; ++h)
          buf[u][h] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, kNoLoad, 0, 2);
    }
  };
  constexpr int kLw = kP * kSGroups;                        // weight loads per stage

  // Routing first.  With few blocks (decode) the block labels and the sorted
  // slot ids are copied into LDS by dword DMA ahead of the stage-0 weights:
  // vector-memory requests are served in order, so these small reads are not
  // queued behind the weight stream, and the whole routing costs one memory
  // latency instead of a chain of dependent scalar loads.  They land in ring
  // slots 0 (labels) and 1 (slot ids), which are free until the activation
  // DMA of the first pass.
  // The epilogue's column scales are fetched first (one per thread), so that
  // the epilogue reads only LDS.
  float cs_pre = 0.0f;
  if (tid < G * 64) {
    const int col = min(tile_at(tid >> 6) * 64 + (tid & 63), N - 1);
    cs_pre = kMode == kSFp8 ? a_scale[0] * w_scale[e] : w_scale[(size_t)e * N + col];
  }
  const int n_sorted_dma = (max_blocks * 16 + 63) / 64;   // 256-byte dword DMAs
  const int n_label_dma = (max_blocks + 63) / 64;
  const bool staged = n_sorted_dma * 256 <= C::kABytes && n_label_dma * 256 <= C::kABytes;
  const uint32_t lds_labels = lds_ring;
  const uint32_t lds_sorted = lds_ring + (uint32_t)C::kABytes;
  if (staged) {
    for (int q = wave; q < n_sorted_dma + n_label_dma; q += kSWaves) {
      if (q < n_sorted_dma) {
        const int i = min(q * 64 + lane, max_blocks * 16 - 1);          // clamped: in bounds
        dma4(sorted_ids, 4u * (uint32_t)i, lds_sorted + (uint32_t)(256 * q));
      } else {
        const int qq = q - n_sorted_dma;
        const int i = min(qq * 64 + lane, max_blocks - 1);
        dma4(expert_ids, 4u * (uint32_t)i, lds_labels + (uint32_t)(256 * qq));
      }
    }
  }
  // The weights of stage 0 do not depend on the routing: start them now.  The
  // router weights are read only in the epilogue.
  load_w(0, wb[0]);

  // this expert's blocks [b_begin, b_end) from the ascending block labels
  // (-1 after the last block)
  int b_begin = max_blocks, b_end = max_blocks;
  constexpr int kEndLabel = 1 << 30;                       // -1 sorts after every expert
  if (staged) {
    wait_dma_upto(kLw);                                    // this wave's routing DMAs landed
    __syncthreads();                                       // ... and everyone's
    const int *labels = reinterpret_cast<const int *>(s_ring);
    for (int base = 0; base < max_blocks; base += 64) {   // a wavefront-wide search
      int v = base + lane < max_blocks ? labels[base + lane] : kEndLabel;
      v = v < 0 ? kEndLabel : v;
      const unsigned long long ge = __ballot(v >= e), gt = __ballot(v > e);
      if (b_begin == max_blocks && ge) b_begin = base + __builtin_ctzll(ge);
      if (gt) {
        b_end = base + __builtin_ctzll(gt);
        break;
      }
    }
  } else {
    // every wavefront scans the labels on its scalar unit, 16 per load (the
    // scalar loads count on lgkmcnt, so they do not wait for the weights)
    typedef const __attribute__((address_space(4))) int *cint_ptr;
    typedef int int16v __attribute__((ext_vector_type(16)));
    typedef const __attribute__((address_space(4))) int16v *cint16_ptr;
    const cint_ptr c_expert_ids = (cint_ptr)expert_ids;
    auto visit = [&](int b, int v) {
      v = v < 0 ? kEndLabel : v;
      if (b_begin == max_blocks && v >= e) b_begin = b;
      if (b_end == max_blocks && v > e) b_end = b;
    };
    int b0 = 0;
    for (; b0 + 16 <= max_blocks && b_end == max_blocks; b0 += 16) {
      const int16v v = *(cint16_ptr)(c_expert_ids + b0);
#pragma unroll
      for (int u = 0; u < 16; ++u) visit(b0 + u, v[u]);
    }
    for (; b0 < max_blocks && b_end == max_blocks; ++b0) visit(b0, c_expert_ids[b0]);
  }
  if (b_begin >= b_end) {
    wait_dma_all();                                        // no load may outlive the workgroup
    return;
  }

  for (int bp = b_begin, pass_ = 0; bp < b_end; bp += kMB, ++pass_) {
    const int nmb = min(b_end - bp, kMB);
    __syncthreads();                                       // s_slot / ring reuse across passes
    int nvalid;                                            // rows holding a routed slot
    if (staged && pass_ == 0) {
      // from the staged copy (the activation DMA below overwrites it)
      const int *sorted = reinterpret_cast<const int *>(s_ring + C::kABytes);
      int slot = S;
      if (tid < nmb * 16) slot = sorted[bp * 16 + tid];
      if (tid < kMB * 16) s_slot[tid] = slot;
      nvalid = __syncthreads_count(tid < kMB * 16 && slot < S);
    } else {
      if (wave == 0) {                                     // slot ids, scalar
        typedef int int16v __attribute__((ext_vector_type(16)));
        typedef const __attribute__((address_space(4))) int16v *cint16_ptr;
        const cint16_ptr c_sorted16 = (cint16_ptr)sorted_ids;
        int nv = 0;
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
          int16v sl;
          if (i < nmb) {
            sl = c_sorted16[bp + i];                       // one 64-byte block of slots
          } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) sl[u] = S;
          }
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (lane == u) s_slot[i * 16 + u] = sl[u];
#pragma unroll
          for (int u = 0; u < 16; ++u) nv += sl[u] < S ? 1 : 0;
        }
        if (lane == 0) s_nvalid = nv;
      }
      __syncthreads();
      nvalid = s_nvalid;
    }
    // router weight (x token scale) of each row, fetched now for the epilogue
    float rw_pre = 0.0f;
    if (tid < kMB * 16) {
      const int slot = s_slot[tid];
      if (slot < S) {
        rw_pre = topk_w[slot];
        if constexpr (kI8) rw_pre *= a_scale[slot / top_k];
      }
    }

    // activation DMA of this wavefront (1 KB instructions q = wave + 8j): the
    // row and the swizzled chunk each lane fetches
    constexpr int kAPerWave = (C::kAInstr + kSWaves - 1) / kSWaves;
    // rows that hold a routed slot (padding slots only follow the expert's
    // last routed one, and their rows are never stored, so their LDS rows
    // are left as they are); 1 KB holds 4 (bf16) or 8 (one-byte) rows
    const int a_instr = kInt8 ? (nvalid + 3) / 4 : (nvalid + 7) / 8;
    int n_a = 0;                                           // this wave's DMAs per stage
    uint32_t a_row[kAPerWave], a_chk[kAPerWave];
#pragma unroll
    for (int j = 0; j < kAPerWave; ++j) {
      const int q = wave + kSWaves * j;
      a_row[j] = 0;
      a_chk[j] = 0;
      if (q < a_instr) ++n_a;
      if (q < C::kAInstr) {
        int r, c;
        if constexpr (kInt8) {                             // 4 rows of 256 bytes per KB
          r = 4 * q + (lane >> 4);
          c = lane & 15;
        } else {                                           // 8 rows of 128 bytes per KB
          r = 8 * q + (lane >> 3);
          c = lane & 7;
        }
        const int slot = s_slot[r];
        const uint32_t tok = slot < S ? (uint32_t)(slot / top_k) : 0u;
        a_row[j] = tok * a_row_bytes;
        // the lane at LDS chunk position c fetches source chunk c ^ swizzle(r)
        a_chk[j] = 16u * (uint32_t)(kInt8 ? (c ^ (r & 15)) : (c ^ swz(r)));
      }
    }

    // activation DMA of stage st into ring slot `ring`
    auto issue_a = [&](int st, int ring) {
      const uint32_t amax = (uint32_t)(K - st * kSK) * (kInt8 ? 2u : 1u) - 16u;
#pragma unroll
      for (int j = 0; j < kAPerWave; ++j) {
        const int q = wave + kSWaves * j;
        if (q < a_instr)                                   // only the rows of this pass
          dma16(a + (size_t)st * C::kARow, a_row[j] + min(a_chk[j], amax),
                lds_ring + (uint32_t)(ring * C::kABytes + 1024 * q));
      }
    };

    f32x4 acc[kSGroups][kMB];
#pragma unroll
    for (int u = 0; u < kSGroups; ++u)
#pragma unroll
      for (int i = 0; i < kMB; ++i) acc[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    f32x4 accA = f32x4{0.f, 0.f, 0.f, 0.f};               // int4: row sums of block `wave`
    auto compute = [&](int st, int ring, const i32x4 (&buf)[kSGroups][kP]) {
      const uint8_t *sa = s_ring + ring * C::kABytes;
      if constexpr (kW4) {
        // four MFMA sub-steps of 32 k: lane group g takes k 32g + 8m .. + 7
        // (activation chunk 4g + m, weight dword m); wavefront i < nmb also
        // sums the rows of block i (an MFMA against ones)
        const i32x4 ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          i32x4 av[kMB];
#pragma unroll
          for (int i = 0; i < kMB; ++i) {
            if (i >= nmb) break;
            av[i] = *reinterpret_cast<const i32x4 *>(sa + sw256(16 * i + r16, 4 * g + m));
            if (i == wave) accA = mfma_bf16(av[i], ones, accA);
          }
#pragma unroll
          for (int u = 0; u < kSGroups; ++u) {
            if (wave + kSWaves * u >= ngr) break;          // wave-uniform
            const i32x4 b = int4x8_to_bf16x8((uint32_t)buf[u][0][m]);
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
              if (i >= nmb) break;
              acc[u][i] = mfma_bf16(av[i], b, acc[u][i]);
            }
          }
        }
        return;
      }
      const int nsub = (st == nst - 1) ? nsub_last : kSK / C::kSub;
#pragma unroll
      for (int ss = 0; ss < kSK / C::kSub; ++ss) {
        if (ss >= nsub) break;
        if constexpr (kInt8) {
          const int c0 = 8 * ss + 2 * g;
          i32x4 av[kMB][2];
#pragma unroll
          for (int i = 0; i < kMB; ++i) {
            if (i >= nmb) break;
            const int r = 16 * i + r16;
            av[i][0] = *reinterpret_cast<const i32x4 *>(sa + sw256(r, c0));
            av[i][1] = *reinterpret_cast<const i32x4 *>(sa + sw256(r, c0 + 1));
          }
#pragma unroll
          for (int u = 0; u < kSGroups; ++u) {
            if (wave + kSWaves * u >= ngr) break;          // wave-uniform
            i32x4 b0, b1;
            dequant16w<kMode == kSF8W16>(buf[u][ss], b0, b1);
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
              if (i >= nmb) break;
              acc[u][i] = mfma_bf16(av[i][0], b0, acc[u][i]);
              acc[u][i] = mfma_bf16(av[i][1], b1, acc[u][i]);
            }
          }
        } else {
          i32x8 av[kMB];
#pragma unroll
          for (int i = 0; i < kMB; ++i) {
            if (i >= nmb) break;
            const int r = 16 * i + r16;
            const i32x4 al = *reinterpret_cast<const i32x4 *>(sa + sw128(r, g));
            const i32x4 ah = *reinterpret_cast<const i32x4 *>(sa + sw128(r, g + 4));
            av[i] = __builtin_shufflevector(al, ah, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int u = 0; u < kSGroups; ++u) {
            if (wave + kSWaves * u >= ngr) break;          // wave-uniform
            const i32x8 bv = __builtin_shufflevector(buf[u][0], buf[u][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
              if (i >= nmb) break;
              if constexpr (kI8) acc[u][i] = mfma_i8(av[i], bv, acc[u][i]);
              else acc[u][i] = mfma_fp8(av[i], bv, acc[u][i]);
            }
          }
        }
      }
    };

    // prologue: weights of stages 0..kSD-1 (stage 0 of the first pass is
    // already in flight), then their activations; past the last stage the
    // weight loads read nothing and the activations of the last stage are
    // loaded again (L2 hits), so every iteration below issues the same loads
    // and the wait counts stay exact
    if (pass_ > 0) load_w(0, wb[0]);
#pragma unroll
    for (int j = 1; j < kSD; ++j) load_w(j, wb[j]);
#pragma unroll
    for (int j = 0; j < kSD; ++j) issue_a(min(j, nst - 1), j);

    // one stage: wait for it, free the previous slot, start stage st + kSD
    // (its activations now, its weights once `buf` has been read)
    auto step = [&](int st, i32x4 (&buf)[kSGroups][kP]) {
      // loads issued after this wave's loads of stage st (weights, then
      // activations in the prologue; activations, then weights after it)
      const int younger = st < kSD ? (kSD - 1 - st) * n_a + st * (n_a + kLw)
                                   : (kSD - 1) * (n_a + kLw);
      wait_dma_upto(younger);                              // stage st landed here
      __syncthreads();                                     // ... and everywhere; slot st-1 is free
      issue_a(min(st + kSD, nst - 1), (st + kSD) % kSAS);
      compute(st, st % kSAS, buf);
      load_w(st + kSD, buf);
    };
    // whole rounds of kSD stages with no exit inside, so that the compiler's
    // own wait before each MFMA counts the loads of the later stages as
    // still in flight; then the last nst % kSD stages
    int st0 = 0;
    for (; st0 + kSD <= nst; st0 += kSD) {
#pragma unroll
      for (int j = 0; j < kSD; ++j) step(st0 + j, wb[j]);
    }
#pragma unroll
    for (int j = 0; j + 1 < kSD; ++j)
      if (st0 + j < nst) step(st0 + j, wb[j]);
    wait_dma_all();                                        // the reloads land before ring reuse

    // ---- epilogue: scale x router weight, rounded to bf16, staged one
    // 16-row block at a time in the (now idle) activation ring as [16][64 G]
    // bf16 rows, then written out as whole 16-byte pieces of each routed
    // slot's row
    if (pass_ == 0 && tid < G * 64) s_scale[tid] = cs_pre;   // per-column (or fused) scale
    if (tid < kMB * 16) s_rw[tid] = rw_pre;
    if constexpr (kW4) {
      if (wave < nmb && r16 == 0) {                        // every column holds the row sum
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s_A[16 * wave + 4 * g + rr] = accA[rr];
      }
    }
    __syncthreads();
    uint16_t *stg = reinterpret_cast<uint16_t *>(s_ring);
    const int wcols = 64 * G;                              // columns of this workgroup
    const int pieces = wcols / 8;                          // 16-byte pieces per staged row
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
      if (i >= nmb) break;                                 // wave-uniform
#pragma unroll
      for (int u = 0; u < kSGroups; ++u) {
        const int jg = wave + kSWaves * u;
        if (jg >= ngr) break;                              // wave-uniform
        const int cl = 64 * (jg >> 2) + 16 * (jg & 3) + r16;   // column within the workgroup
        const float cs = s_scale[cl];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int k = 4 * g + rr;                        // row within the block
          float acc_v = acc[u][i][rr];
          if constexpr (kI8) acc_v = (float)__builtin_bit_cast(int, acc_v);
          if constexpr (kW4) acc_v = fmaf(-kInt4Offset, s_A[16 * i + k], acc_v);
          const float v = acc_v * cs * s_rw[16 * i + k];   // x router weight (x token scale)
          stg[k * wcols + cl] = (uint16_t)f32x2_to_bf16x2(v, 0.0f);
        }
      }
      __syncthreads();
      // N is a multiple of 8, so a piece is inside the row or past its end
      for (int q = tid; q < 16 * pieces; q += kSThreads) {
        const int k = q / pieces, c8 = q - k * pieces;
        const int slot = s_slot[16 * i + k];
        const int col = tile_at(c8 >> 3) * 64 + 8 * (c8 & 7);
        if (slot < S && col < N)
          *reinterpret_cast<i32x4 *>(y + (size_t)slot * N + col) =
              *reinterpret_cast<const i32x4 *>(stg + k * wcols + 8 * c8);
      }
      __syncthreads();                                     // the staging area is reused
    }
  }
}



// =============================================================================
// block_m = 128 (fp8 W8A8, int8 W8A16) and MXFP8: DMA-fed MFMA tiles
// =============================================================================
// One workgroup of 8 wavefronts (two per SIMD) per 128-row x 256-column
// output tile of one expert; wavefront w owns the 64 x 64 block at rows
// 64*(w & 1).., columns 64*(w >> 1).. as 4 x 4 MFMA fragments.  Two
// wavefronts per SIMD let one issue MFMAs while the other waits for its LDS
// reads.  Routed formats take the tile's rows from the sorted slots of one
// routing block; MXFP8 from the expert's contiguous row segment.
//
// Every k-stage (128 k) of the tile's activation rows and weight columns is
// copied HBM/L2 -> LDS by global_load_lds_dwordx4 (direct-to-LDS DMA, as in
// the streaming kernel) into a ring of kSlots stages that runs kSlots - 1
// stages ahead of the MFMAs, so loads in flight cost no registers and their
// latency hides behind whole stages of compute.  The wavefront pair of a
// 64-column block DMAs that block (8 KB per stage, one half each) and every
// wavefront an eighth of the activation rows; MXFP8 scale bytes of the stage
// (4 per row and column) follow by global_load_lds_dword.  Before a stage is
// read each wavefront waits for its own DMA and the workgroup synchronises.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that the 16 rows one fragment
// read touches hit distinct banks):
//   fp8 activations, 128-byte rows: chunk c of row r at c ^ swz(r)
//   bf16 activations, 256-byte rows: chunk c of row r at c ^ (r & 15)
//   weights, 64 rows of 128 bytes per column block: chunk c of row r at
//   c ^ swz(r), the MOE_W_TILED block layout, so tiled weights are a plain
//   8 KB copy and row-major weights are swizzled on the source side.
//
// The epilogue goes through LDS as well: each wavefront writes its scaled
// 64 x 64 block there, then stores whole row segments (256 bytes of fp32 per
// routed slot, 128 bytes of bf16 per MXFP8 row) with 16-byte stores.
constexpr int kGBM = 128;
constexpr int kGBN = 256;
constexpr int kGThreads = 512;

template <bool kInt8>
struct GCfg {
  static constexpr int kARow = kInt8 ? 256 : 128;           // activation bytes per row per stage
  static constexpr int kABytes = kGBM * kARow;
  static constexpr int kBBytes = kGBN * 128;
  static constexpr int kStage = kABytes + kBBytes;          // 48 KB (fp8) / 64 KB (int8)
  static constexpr int kSlots = kInt8 ? 2 : 3;              // ring stages (LDS: 144 / 128 KB)
  static constexpr int kAPerWave = kABytes / 1024 / 8;      // activation DMA instructions per wave
  static constexpr int kPerStage = kAPerWave + 4;           // DMA instructions per wave per stage
};
constexpr int kSfStage = 4 * kGBM + 4 * kGBN;                // MXFP8 scale bytes per stage

template <int kFmt, bool kTiled>
__global__ __launch_bounds__(kGThreads, 1) void gemm_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ a_sf, const uint8_t *__restrict__ w,
    const float *__restrict__ w_scale, const uint8_t *__restrict__ w_sf,
    const int *__restrict__ sorted_ids, const int *__restrict__ expert_ids,
    const float *__restrict__ topk_w, const int *__restrict__ m_offsets, int M, int K, int N,
    int E, int top_k, int max_blocks, uint16_t *__restrict__ out) {
  constexpr bool kInt8 = kFmt == kFmtInt8 || kFmt == kFmtF8W16;   // bf16 activations
  constexpr bool kMx = kFmt == kFmtMx;
  using C = GCfg<kInt8>;
  constexpr int kMF = 4, kNF = 4;                       // fragments per wavefront
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[C::kSlots * C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_sf[kMx ? C::kSlots * kSfStage : 16];
  __shared__ int s_row[kGBM];
  __shared__ int s_blk_first[kMaxExperts + 1];
  __shared__ int s_tile_first[kMaxExperts + 1];
  __shared__ int s_mo[kMx ? kMaxExperts + 1 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, r16 = lane & 15;
  const int ntn = (N + kGBN - 1) / kGBN;

  // ---- tile space: expert by expert, column tile by column tile, row block
  // fastest; each XCD takes one contiguous chunk of it
  if constexpr (!kMx) {
    expert_block_starts(expert_ids, max_blocks, E, s_blk_first);
    __syncthreads();
  }
  if (tid == 0) {
    int blk = 0, tiles = 0;
    for (int ee = 0; ee < E; ++ee) {
      int nb;
      if constexpr (kMx) {
        s_mo[ee] = m_offsets[ee];
        s_mo[ee + 1] = m_offsets[ee + 1];
        const int m = s_mo[ee + 1] - s_mo[ee];
        nb = m > 0 ? (m + kGBM - 1) / kGBM : 0;
        s_blk_first[ee] = blk;
        blk += nb;
      } else {
        nb = s_blk_first[ee + 1] - s_blk_first[ee];
      }
      s_tile_first[ee] = tiles;
      tiles += nb * ntn;
    }
    if constexpr (kMx) s_blk_first[E] = blk;
    s_tile_first[E] = tiles;
  }
  __syncthreads();
  const int total = s_tile_first[E];
  const int chunk = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int idx = blockIdx.x / kXcds;
  const int L = xcd * chunk + idx;
  if (idx >= chunk || L >= total) return;
  int e = 0;
  while (s_tile_first[e + 1] <= L) ++e;
  const int nblk = s_blk_first[e + 1] - s_blk_first[e];
  const int local = L - s_tile_first[e];
  const int nt = local / nblk;
  const int mb = local - nt * nblk;
  const int n0 = nt * kGBN;
  const int S = M * top_k;                              // routed: slots; MXFP8: unused
  int row0 = 0, row_end = 0;                            // MXFP8: the tile's rows
  if constexpr (kMx) {
    row0 = s_mo[e] + mb * kGBM;
    row_end = s_mo[e + 1];
    if (tid < kGBM) s_row[tid] = row0 + tid;
  } else {
    if (tid < kGBM) s_row[tid] = sorted_ids[(s_blk_first[e] + mb) * kGBM + tid];
  }
  __syncthreads();
  // source row of tile row r (rows past the tile's end repeat a valid one)
  auto src_row = [&](int r) -> uint32_t {
    const int v = s_row[r];
    if constexpr (kMx) return (uint32_t)(v < row_end ? v : row_end - 1);
    else return (uint32_t)(v < S ? v / top_k : 0);
  };

  // ---- DMA sources of this lane ----------------------------------------------
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_ring;
  const uint32_t a_row_bytes = kInt8 ? (uint32_t)K * 2u : (uint32_t)K;
  const int nst = (K + 127) / 128;
  // activations: instruction q = wave * kAPerWave + u moves 8 fp8 rows (or 4
  // bf16 rows); the lane at LDS chunk position c fetches source chunk
  // c ^ swizzle(row)
  uint32_t a_row[C::kAPerWave], a_chk[C::kAPerWave];
#pragma unroll
  for (int u = 0; u < C::kAPerWave; ++u) {
    const int q = wave * C::kAPerWave + u;
    int r, c;
    if constexpr (kInt8) {
      r = 4 * q + (lane >> 4);
      c = (lane & 15) ^ (r & 15);
    } else {
      r = 8 * q + (lane >> 3);
      c = (lane & 7) ^ swz(r);
    }
    a_row[u] = src_row(r) * a_row_bytes;
    a_chk[u] = 16u * (uint32_t)c;
  }
  // weights: rows 32*wm .. 32*wm + 31 of column block wn (4 instructions)
  uint32_t wblk = 0;                                    // tiled: the packed block of stage 0
  uint32_t b_row[4], b_chk[4];                          // row-major: 8 rows per instruction
  if constexpr (kTiled) {
    const int T = (N + 63) / 64;
    const int pt = min(n0 / 64 + wn, T - 1);
    wblk = ((uint32_t)e * (uint32_t)T + (uint32_t)pt) * (uint32_t)nst * 8192u;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = 8 * (4 * wm + u) + (lane >> 3);
      const int col = min(n0 + wn * 64 + n, N - 1);
      b_row[u] = ((uint32_t)e * (uint32_t)N + (uint32_t)col) * (uint32_t)K;
      b_chk[u] = 16u * (uint32_t)((lane & 7) ^ swz(n));
    }
  }
  // MXFP8 scales: wavefronts 0-1 move the 4 scale bytes of rows 64w + lane,
  // wavefronts 2-5 those of columns 64(w-2) + lane (one dword DMA each)
  const uint32_t kb_row = (uint32_t)K / 32u;            // scale bytes per row
  uint32_t sf_off = 0;
  const int sfn = (kMx && wave < 6) ? 1 : 0;            // scale DMAs of this wave per stage
  if constexpr (kMx) {
    if (wave < 2) {
      int po = 0;                                       // the expert's padded scale rows
      for (int ee = 0; ee < e; ++ee) po += (s_mo[ee + 1] - s_mo[ee] + kMxRowPad - 1) / kMxRowPad * kMxRowPad;
      sf_off = ((uint32_t)po + src_row(64 * wave + lane) - (uint32_t)s_mo[e]) * kb_row;
    } else if (wave < 6) {
      const int col = min(n0 + 64 * (wave - 2) + lane, N - 1);
      sf_off = ((uint32_t)e * (uint32_t)N + (uint32_t)col) * kb_row;
    }
  }
  const uint32_t lds_sf = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_sf;

  auto issue = [&](int st, int slot_i) {
    const uint32_t base = lds_ring + (uint32_t)(slot_i * C::kStage);
    // the last stage of an int8 W8A16 product with K % 128 == 64 holds 64 k:
    // chunks past the row end are clamped (fetched but never used)
    const uint32_t amax = (uint32_t)(K - st * 128) * (kInt8 ? 2u : 1u) - 16u;
    const uint8_t *abase = a + (size_t)st * C::kARow;
#pragma unroll
    for (int u = 0; u < C::kAPerWave; ++u)
      dma16(abase, a_row[u] + min(a_chk[u], amax),
            base + (uint32_t)((wave * C::kAPerWave + u) * 1024));
    const uint32_t bdst = base + (uint32_t)(C::kABytes + wn * 8192 + wm * 4096);
    if constexpr (kTiled) {
      const uint8_t *bbase = w + wblk + (size_t)st * 8192u + wm * 4096;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dma16(bbase, (uint32_t)(u * 1024 + 16 * lane), bdst + (uint32_t)(u * 1024));
    } else {
      const uint32_t kmax = (uint32_t)(K - st * 128) - 16u;
      const uint8_t *bbase = w + (size_t)st * 128u;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dma16(bbase, b_row[u] + min(b_chk[u], kmax), bdst + (uint32_t)(u * 1024));
    }
    if constexpr (kMx) {
      const uint32_t sdst = lds_sf + (uint32_t)(slot_i * kSfStage);
      if (wave < 2) dma4(a_sf + 4 * st, sf_off, sdst + (uint32_t)(256 * wave));
      else if (wave < 6) dma4(w_sf + 4 * st, sf_off, sdst + (uint32_t)(4 * kGBM + 256 * (wave - 2)));
    }
  };

  f32x4 acc[kMF][kNF];
#pragma unroll
  for (int i = 0; i < kMF; ++i)
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets (independent of the fragment index: every swizzle
  // depends on the row modulo 16 only)
  const int sw = swz(r16);
  auto compute = [&](int slot_i, int nh) {
    const uint8_t *As = s_ring + slot_i * C::kStage + wm * 64 * C::kARow;
    const uint8_t *Bs = s_ring + slot_i * C::kStage + C::kABytes + wn * 8192;
    if constexpr (kInt8) {
      for (int h = 0; h < nh; ++h) {
        i32x4 bq[kNF][2];
#pragma unroll
        for (int j = 0; j < kNF; ++j)
          dequant16w<kFmt == kFmtF8W16>(ld16(Bs + (j * 16 + r16) * 128 + (((g + 4 * h) ^ sw) << 4)),
                                        bq[j][0], bq[j][1]);
        const int c0 = ((8 * h + 2 * g) ^ r16) << 4;
        const int c1 = ((8 * h + 2 * g + 1) ^ r16) << 4;
        i32x4 a0[kMF], a1[kMF];
#pragma unroll
        for (int i = 0; i < kMF; ++i) {
          a0[i] = ld16(As + (i * 16 + r16) * 256 + c0);
          a1[i] = ld16(As + (i * 16 + r16) * 256 + c1);
        }
#pragma unroll
        for (int i = 0; i < kMF; ++i)
#pragma unroll
          for (int j = 0; j < kNF; ++j) {
            acc[i][j] = mfma_bf16(a0[i], bq[j][0], acc[i][j]);
            acc[i][j] = mfma_bf16(a1[i], bq[j][1], acc[i][j]);
          }
      }
    } else {
      i32x8 bv[kNF], av[kMF];
#pragma unroll
      for (int j = 0; j < kNF; ++j) {
        const uint8_t *br = Bs + (j * 16 + r16) * 128;
        bv[j] = __builtin_shufflevector(ld16(br + ((g ^ sw) << 4)), ld16(br + (((g + 4) ^ sw) << 4)),
                                        0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < kMF; ++i) {
        const uint8_t *ar = As + (i * 16 + r16) * 128;
        av[i] = __builtin_shufflevector(ld16(ar + ((g ^ sw) << 4)), ld16(ar + (((g + 4) ^ sw) << 4)),
                                        0, 1, 2, 3, 4, 5, 6, 7);
      }
      if constexpr (kMx) {
        // lane (g, r16) supplies the scale of 32-k block g of its row / column
        const uint8_t *sfs = s_sf + slot_i * kSfStage;
        int sa[kMF], sb[kNF];
#pragma unroll
        for (int i = 0; i < kMF; ++i)
          sa[i] = (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * (wm * 64 + i * 16 + r16)) >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < kNF; ++j)
          sb[j] = (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * kGBM + 4 * (wn * 64 + j * 16 + r16)) >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < kMF; ++i)
#pragma unroll
          for (int j = 0; j < kNF; ++j) acc[i][j] = mfma_mx(av[i], bv[j], acc[i][j], sa[i], sb[j]);
      } else {
#pragma unroll
        for (int i = 0; i < kMF; ++i)
#pragma unroll
          for (int j = 0; j < kNF; ++j) acc[i][j] = mfma_fp8(av[i], bv[j], acc[i][j]);
      }
    }
  };

  // ---- the ring: stage st lives in slot st % kSlots --------------------------
  constexpr int D = C::kSlots - 1;                      // stages in flight ahead of compute
  const int per_stage = C::kPerStage + sfn;             // this wave's DMAs per stage
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (st < nst) issue(st, st);
  const int nh_last = kInt8 ? ((K - (nst - 1) * 128) >= 128 ? 2 : 1) : 1;
  int slot_c = 0;                                       // slot of stage st
  int slot_i = D % C::kSlots;                           // slot of stage st + D
  for (int st = 0; st < nst; ++st) {
    // stages st .. min(st + D - 1, nst - 1) are in flight: wait for stage st
    // (loads complete in order, so waiting for stage st leaves the later
    // stage's DMAs in flight)
    if (D == 2 && st + 1 < nst) wait_dma_upto(per_stage);
    else wait_dma_all();
    __syncthreads();                                    // stage st complete; slot_i is free
    if (st + D < nst) issue(st + D, slot_i);
    compute(slot_c, (kInt8 && st == nst - 1) ? nh_last : 2);
    slot_c = slot_c + 1 == C::kSlots ? 0 : slot_c + 1;
    slot_i = slot_i + 1 == C::kSlots ? 0 : slot_i + 1;
  }

  // ---- epilogue: results (routed: scaled by the format's scales and the
  // router weight) as bf16 -> LDS (the ring is free) -> 128-byte row segments
  // of the destination rows (routed: the slots; MXFP8: the expert's rows)
  __syncthreads();                                      // every wavefront is done with the ring
  float cscale = 1.0f;
  if constexpr (kFmt == kFmtFp8) cscale = a_scale[0] * w_scale[e];
  uint16_t *t = reinterpret_cast<uint16_t *>(s_ring) + wave * 64 * 64;   // [64 rows][64 columns]
#pragma unroll
  for (int j = 0; j < kNF; ++j) {
    float cs = cscale;
    if constexpr (kInt8) cs = w_scale[(size_t)e * N + min(n0 + wn * 64 + j * 16 + r16, N - 1)];
#pragma unroll
    for (int i = 0; i < kMF; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = i * 16 + 4 * g + rr;
        float v = acc[i][j][rr];
        if constexpr (!kMx) {
          const int slot = s_row[wm * 64 + r];
          v = v * cs * (slot < S ? topk_w[slot] : 0.0f);
        }
        t[r * 64 + j * 16 + r16] = (uint16_t)(f32x2_to_bf16x2(v, 0.0f) & 0xFFFFu);
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0): the wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  const bool vec = (N & 7) == 0 && ((uintptr_t)out & 15u) == 0;   // 16-byte aligned segments
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = q * 8 + (lane >> 3);                  // row within the wavefront's block
    const int col = n0 + wn * 64 + (lane & 7) * 8;
    int dst_row;
    if constexpr (kMx) {
      dst_row = row0 + wm * 64 + r;
      if (dst_row >= row_end) continue;
    } else {
      dst_row = s_row[wm * 64 + r];
      if (dst_row >= S) continue;
    }
    if (col >= N) continue;
    const uint16_t *src = t + r * 64 + (lane & 7) * 8;
    uint16_t *dst = out + (size_t)dst_row * N + col;
    if (vec && col + 8 <= N) {
      *reinterpret_cast<i32x4 *>(dst) = *reinterpret_cast<const i32x4 *>(src);
    } else {
      for (int c = 0; c < 8 && col + c < N; ++c) dst[c] = src[c];
    }
  }
}

// =============================================================================
// fp8 W8A8 (block_m = 128) and MXFP8: 256 x 256 tiles
// =============================================================================
// A tile covers two consecutive 128-row blocks of one expert (the second may
// be missing: an expert with an odd number of blocks) and 256 columns.  The
// kWaves wavefronts split it as 2 (rows) x kWaves/2 (columns): each owns 128
// rows x 512/kWaves columns as 8 x kFN MFMA fragments.  Against 64 x 64
// wavefront tiles this reads fewer LDS bytes per MFMA (activation fragments
// serve kFN MFMAs each) and moves a third fewer global bytes per flop.
// Operands of stage st + 1 come HBM/L2 -> LDS by direct-to-LDS DMA while
// stage st computes (two 64 KB ring slots); the epilogue stages bf16 results
// in LDS and stores whole row segments.  LDS layouts as in gemm_kernel.
constexpr int kHBM = 256;
constexpr int kHBN = 256;
constexpr int kHABytes = kHBM * 128;                        // 32 KB of fp8 rows per stage
constexpr int kHBBytes = kHBN * 128;                        // 32 KB of weight rows per stage
constexpr int kHStage = kHABytes + kHBBytes;
constexpr int kHSf = 4 * kHBM + 4 * kHBN;                   // MXFP8 scale bytes per stage
constexpr int kHWaves = 8;

template <int kFmt, bool kTiled, int kWaves>
__global__ __launch_bounds__(64 * kWaves, 1) void gemm_big_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ a_sf, const uint8_t *__restrict__ w,
    const float *__restrict__ w_scale, const uint8_t *__restrict__ w_sf,
    const int *__restrict__ sorted_ids, const int *__restrict__ expert_ids,
    const float *__restrict__ topk_w, const int *__restrict__ m_offsets, int M, int K, int N,
    int E, int top_k, int max_blocks, uint16_t *__restrict__ out) {
  constexpr bool kMx = kFmt == kFmtMx;
  static_assert(kFmt != kFmtInt8, "int8 W8A16 uses gemm_kernel");
  static_assert(kWaves == 4 || kWaves == 8, "wavefronts");
  constexpr int kThr = 64 * kWaves;
  constexpr int kFM = 8;                                 // row fragments per wavefront (128 rows)
  constexpr int kCols = 512 / kWaves;                    // columns per wavefront
  constexpr int kFN = kCols / 16;
  constexpr int kDma = 32 / kWaves;                      // activation (and weight) DMAs per wave
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[2 * kHStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_sf[kMx ? 2 * kHSf : 16];
  __shared__ int s_row[kHBM];
  __shared__ int s_blk_first[kMaxExperts + 1];
  __shared__ int s_tile_first[kMaxExperts + 1];
  __shared__ int s_mo[kMx ? kMaxExperts + 1 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, r16 = lane & 15;
  const int ntn = (N + kHBN - 1) / kHBN;

  // ---- tile space: expert by expert, column tile by column tile, block pair
  // fastest; each XCD takes one contiguous chunk of it
  if constexpr (!kMx) {
    expert_block_starts(expert_ids, max_blocks, E, s_blk_first);
    __syncthreads();
  }
  if (tid == 0) {
    int blk = 0, tiles = 0;
    for (int ee = 0; ee < E; ++ee) {
      int nb;
      if constexpr (kMx) {
        s_mo[ee] = m_offsets[ee];
        s_mo[ee + 1] = m_offsets[ee + 1];
        const int m = s_mo[ee + 1] - s_mo[ee];
        nb = m > 0 ? (m + kGBM - 1) / kGBM : 0;
        s_blk_first[ee] = blk;
        blk += nb;
      } else {
        nb = s_blk_first[ee + 1] - s_blk_first[ee];
      }
      s_tile_first[ee] = tiles;
      tiles += (nb + 1) / 2 * ntn;
    }
    if constexpr (kMx) s_blk_first[E] = blk;
    s_tile_first[E] = tiles;
  }
  __syncthreads();
  const int total = s_tile_first[E];
  const int chunk = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int idx = blockIdx.x / kXcds;
  const int L = xcd * chunk + idx;
  if (idx >= chunk || L >= total) return;
  int e = 0;
  while (s_tile_first[e + 1] <= L) ++e;
  const int nblk = s_blk_first[e + 1] - s_blk_first[e];
  const int npair = (nblk + 1) / 2;
  const int local = L - s_tile_first[e];
  const int nt = local / npair;
  const int pr = local - nt * npair;
  const int nb_here = min(2, nblk - 2 * pr);            // 128-row blocks in this tile
  const int n0 = nt * kHBN;
  const int S = M * top_k;
  int row0 = 0, row_end = 0;                            // MXFP8: the tile's rows
  for (int r = tid; r < kHBM; r += kThr) {
    if constexpr (kMx) {
      row0 = s_mo[e] + 2 * pr * kGBM;
      s_row[r] = row0 + r;
    } else {
      s_row[r] = r < nb_here * kGBM ? sorted_ids[(s_blk_first[e] + 2 * pr) * kGBM + r] : S;
    }
  }
  if constexpr (kMx) {
    row0 = s_mo[e] + 2 * pr * kGBM;
    row_end = s_mo[e + 1];
  }
  __syncthreads();
  auto src_row = [&](int r) -> uint32_t {
    const int v = s_row[r];
    if constexpr (kMx) return (uint32_t)(v < row_end ? v : row_end - 1);
    else return (uint32_t)(v < S ? v / top_k : 0);
  };
  // this wave's activation DMA rows (8 kDma rows from 8 kDma wave) exist
  const bool a_dma = (8 * kDma * wave) / kGBM < nb_here;
  const bool busy = wm < nb_here;                       // this wave's 128 output rows exist

  // ---- DMA sources of this lane ----------------------------------------------
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_ring;
  const int nst = K / 128;
  uint32_t a_off[kDma];
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int r = 8 * (kDma * wave + u) + (lane >> 3);
    a_off[u] = src_row(r) * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ swz(r));
  }
  // weights: DMAs q = kDma wave + u, 1 KB each: 64-column block q / 8, piece q % 8
  const int bblk = (kDma * wave) / 8;                   // the same block for all of this wave's
  uint32_t wblk = 0;
  uint32_t b_off[kDma];
  if constexpr (kTiled) {
    const int T = (N + 63) / 64;
    const int pt = min(n0 / 64 + bblk, T - 1);
    wblk = ((uint32_t)e * (uint32_t)T + (uint32_t)pt) * (uint32_t)nst * 8192u;
  } else {
#pragma unroll
    for (int u = 0; u < kDma; ++u) {
      const int n = 8 * ((kDma * wave + u) & 7) + (lane >> 3);
      const int col = min(n0 + bblk * 64 + n, N - 1);
      b_off[u] = ((uint32_t)e * (uint32_t)N + (uint32_t)col) * (uint32_t)K +
                 16u * (uint32_t)((lane & 7) ^ swz(n));
    }
  }
  // MXFP8 scales: 8 dword DMAs per stage (rows 0-255, then columns 0-255, 64
  // per DMA), spread over the wavefronts
  constexpr int kSfPerWave = 8 / kWaves;
  const uint32_t kb_row = (uint32_t)K / 32u;
  uint32_t sf_off[kSfPerWave];
  bool sf_on[kSfPerWave];
  if constexpr (kMx) {
    int po = 0;
    for (int ee = 0; ee < e; ++ee) po += (s_mo[ee + 1] - s_mo[ee] + kMxRowPad - 1) / kMxRowPad * kMxRowPad;
#pragma unroll
    for (int u = 0; u < kSfPerWave; ++u) {
      const int q = kSfPerWave * wave + u;             // 0-3 rows, 4-7 columns
      if (q < 4) {
        sf_off[u] = ((uint32_t)po + src_row(64 * q + lane) - (uint32_t)s_mo[e]) * kb_row;
        sf_on[u] = (64 * q) / kGBM < nb_here;
      } else {
        sf_off[u] = ((uint32_t)e * (uint32_t)N + (uint32_t)min(n0 + 64 * (q - 4) + lane, N - 1)) * kb_row;
        sf_on[u] = true;
      }
    }
  }
  const uint32_t lds_sf = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_sf;

  auto issue = [&](int st, int slot_i) {
    const uint32_t base = lds_ring + (uint32_t)(slot_i * kHStage);
    if (a_dma) {
      const uint8_t *src = a + (size_t)st * 128u;
#pragma unroll
      for (int u = 0; u < kDma; ++u)
        dma16(src, a_off[u], base + (uint32_t)((kDma * wave + u) * 1024));
    }
    const uint32_t bdst = base + (uint32_t)(kHABytes + (kDma * wave) * 1024);
    if constexpr (kTiled) {
      const uint8_t *src = w + wblk + (size_t)st * 8192u + ((kDma * wave) & 7) * 1024;
#pragma unroll
      for (int u = 0; u < kDma; ++u) dma16(src, (uint32_t)(u * 1024 + 16 * lane), bdst + (uint32_t)(u * 1024));
    } else {
      const uint8_t *src = w + (size_t)st * 128u;
#pragma unroll
      for (int u = 0; u < kDma; ++u) dma16(src, b_off[u], bdst + (uint32_t)(u * 1024));
    }
    if constexpr (kMx) {
      const uint32_t sdst = lds_sf + (uint32_t)(slot_i * kHSf);
#pragma unroll
      for (int u = 0; u < kSfPerWave; ++u) {
        const int q = kSfPerWave * wave + u;
        if (sf_on[u]) dma4((q < 4 ? a_sf : w_sf) + 4 * st, sf_off[u], sdst + (uint32_t)(256 * q));
      }
    }
  };

  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int sw = swz(r16);
  auto compute = [&](int slot_i) {
    const uint8_t *As = s_ring + slot_i * kHStage + wm * 128 * 128;
    const uint8_t *Bs = s_ring + slot_i * kHStage + kHABytes + wn * kCols * 128;
    const uint8_t *sfs = s_sf + slot_i * kHSf;
    i32x8 bv[kFN];
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const uint8_t *br = Bs + (j * 16 + r16) * 128;
      bv[j] = __builtin_shufflevector(ld16(br + ((g ^ sw) << 4)), ld16(br + (((g + 4) ^ sw) << 4)),
                                      0, 1, 2, 3, 4, 5, 6, 7);
    }
    int sb[kFN];
    if constexpr (kMx) {
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        sb[j] = (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * kHBM + 4 * (wn * kCols + j * 16 + r16)) >> (8 * g)) & 0xFFu);
    }
    // activation fragment i + 1 is read while the MFMAs of fragment i run
    auto load_a = [&](int i) {
      const uint8_t *ar = As + (i * 16 + r16) * 128;
      return __builtin_shufflevector(ld16(ar + ((g ^ sw) << 4)), ld16(ar + (((g + 4) ^ sw) << 4)),
                                     0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto load_sa = [&](int i) {
      if constexpr (kMx)
        return (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * (wm * 128 + i * 16 + r16)) >> (8 * g)) & 0xFFu);
      else
        return 0;
    };
    i32x8 av = load_a(0);
    int sa = load_sa(0);
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      i32x8 av_next = av;
      int sa_next = sa;
      if (i + 1 < kFM) {
        av_next = load_a(i + 1);
        sa_next = load_sa(i + 1);
      }
      if constexpr (kMx) {
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mfma_mx(av, bv[j], acc[i][j], sa, sb[j]);
      } else {
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mfma_fp8(av, bv[j], acc[i][j]);
      }
      av = av_next;
      sa = sa_next;
    }
  };

  // ---- two-slot ring: stage st in slot st & 1, stage st + 1 in flight ------
  issue(0, 0);
  for (int st = 0; st < nst; ++st) {
    wait_dma_all();                                     // this wave's DMA of stage st landed
    __syncthreads();                                    // ... everyone's; slot (st + 1) & 1 is free
    if (st + 1 < nst) issue(st + 1, (st + 1) & 1);
    if (busy) compute(st & 1);
  }

  // ---- epilogue: bf16 results -> LDS (the ring is free) -> row segments ----
  __syncthreads();
  float cscale = 1.0f;
  if constexpr (!kMx) cscale = a_scale[0] * w_scale[e];
  if (!busy) return;
  uint16_t *t = reinterpret_cast<uint16_t *>(s_ring) + wave * 128 * kCols;   // [128 rows][kCols]
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = i * 16 + 4 * g + rr;
      float rs = 1.0f;
      if constexpr (!kMx) {
        const int slot = s_row[wm * 128 + r];
        rs = cscale * (slot < S ? topk_w[slot] : 0.0f);
      }
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        t[r * kCols + j * 16 + r16] = (uint16_t)(f32x2_to_bf16x2(acc[i][j][rr] * rs, 0.0f) & 0xFFFFu);
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0): the wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  const bool vec = (N & 7) == 0 && ((uintptr_t)out & 15u) == 0;
  constexpr int kLanesPerRow = kCols / 8;               // 16 bytes per lane
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
#pragma unroll 4
  for (int q = 0; q < 128 / kRowsPerStore; ++q) {
    const int r = q * kRowsPerStore + lane / kLanesPerRow;
    const int col = n0 + wn * kCols + (lane % kLanesPerRow) * 8;
    int dst_row;
    if constexpr (kMx) {
      dst_row = row0 + wm * 128 + r;
      if (dst_row >= row_end) continue;
    } else {
      dst_row = s_row[wm * 128 + r];
      if (dst_row >= S) continue;
    }
    if (col >= N) continue;
    const uint16_t *src = t + r * kCols + (lane % kLanesPerRow) * 8;
    uint16_t *dst = out + (size_t)dst_row * N + col;
    if (vec && col + 8 <= N) {
      *reinterpret_cast<i32x4 *>(dst) = *reinterpret_cast<const i32x4 *>(src);
    } else {
      for (int c = 0; c < 8 && col + c < N; ++c) dst[c] = src[c];
    }
  }
}

unsigned tile_grid(long long tiles_bound) {
  long long per = (tiles_bound + kXcds - 1) / kXcds;
  return (unsigned)(per * kXcds);
}

}  // namespace

namespace {
int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
  }
  return n;
}

// Below this many routed rows per expert (on average) most 256-row tiles
// hold a single 128-row block; the eight-wavefront kernels then idle the
// wavefronts of the missing block and give their SIMD time to the others,
// where the four-wavefront tile kernel (one per SIMD) would leave half the
// MFMA units to a block that does not exist.  (Measured: fp8 with a biased
// router at 128 rows per expert runs equally fast on either kernel, at 256
// rows 6.5% faster on the tile kernel.)
constexpr long long kWideMinRowsPerExpert = 256;

// bytes of the weight tensor in the layout the call passes (below 4 GiB)
uint32_t stream_weight_bytes(const RoutedArgs &r) {
  if (r.w_layout == MOE_W_TILED)
    return (uint32_t)r.E * (uint32_t)((r.N + 63) / 64) * (uint32_t)((r.K + 127) / 128) * 8192u;
  if (r.w_layout == MOE_W_FRAG)
    return (uint32_t)r.E * (uint32_t)((r.N + 15) / 16) * (uint32_t)((r.K + 63) / 64) * 1024u;
  return (uint32_t)r.E * (uint32_t)r.N * (uint32_t)r.K;
}

template <int kMode, int kMB>
decltype(&stream_kernel<kMode, MOE_W_ROWMAJOR, kMB>) stream_kernel_l(int layout) {
  if (layout == MOE_W_FRAG) return stream_kernel<kMode, MOE_W_FRAG, kMB>;
  if (layout == MOE_W_TILED) return stream_kernel<kMode, MOE_W_TILED, kMB>;
  return stream_kernel<kMode, MOE_W_ROWMAJOR, kMB>;
}
// The bf16-activation paths take 32 rows per pass when the experts average
// at most 16 routed rows (decode): the registers saved go to a third weight
// stage in flight; an expert with more rows takes further passes.
bool stream_two_blocks(const RoutedArgs &r) {
  return (long long)r.M * r.top_k <= 16ll * r.E;
}
template <int kMode>
decltype(&stream_kernel<kMode, MOE_W_ROWMAJOR, kSMB>) stream_kernel_for(int layout, bool two) {
  return two ? stream_kernel_l<kMode, 2>(layout) : stream_kernel_l<kMode, kSMB>(layout);
}

// persistent decomposition of the weight stream: E * groups workgroups, each
// with up to tiles_per_group 64-column tiles of one expert (taken strided:
// tiles grp, grp + groups, ...)
void stream_grid(int N, int E, int &groups, int &tiles_per_group) {
  const int ntiles = (N + 63) / 64;
  int tpg = (E * ntiles + num_cus() - 1) / num_cus();
  tpg = tpg < 1 ? 1 : (tpg > kSMaxTiles ? kSMaxTiles : tpg);   // LDS holds <= 7 tiles
  tiles_per_group = tpg;
  groups = (ntiles + tpg - 1) / tpg;
}
}  // namespace

namespace {
TileArgs routed_tile_args(const uint8_t *a, const float *a_scale, const uint8_t *w,
                          const float *w_scale, const RoutedArgs &r) {
  TileArgs t{};
  t.a = a;
  t.a_scale = a_scale;
  t.w = w;
  t.w_scale = w_scale;
  t.sorted_ids = r.sorted_ids;
  t.expert_ids = r.expert_ids;
  t.topk_w = r.topk_w;
  t.out = r.y;
  t.out_bytes = (uint32_t)((unsigned long long)r.M * r.top_k * r.N * 2ull);
  t.M = r.M;
  t.K = r.K;
  t.N = r.N;
  t.E = r.E;
  t.top_k = r.top_k;
  t.max_blocks = r.max_blocks;
  return t;
}
}  // namespace

hipError_t launch_gemm_fp8(const uint8_t *a_q, const float *a_scale, const uint8_t *w_q,
                           const float *w_scale, const RoutedArgs &r, hipStream_t s) {
  if (r.block_m == 16) {
    int groups, tpg;
    stream_grid(r.N, r.E, groups, tpg);
    auto k = stream_kernel_for<kSFp8>(r.w_layout, false);
    hipLaunchKernelGGL(k, dim3(r.E * groups), dim3(kSThreads), 0, s, a_q, a_scale, w_q, w_scale,
                       r.sorted_ids, r.expert_ids, r.num_post, r.topk_w, r.M, r.K, r.N, r.top_k,
                       groups, tpg, r.max_blocks, r.y, stream_weight_bytes(r));
  } else {
    const long long tiles = (long long)(r.max_blocks / 2 + r.E) * ((r.N + kHBN - 1) / kHBN);
    if ((long long)r.M * r.top_k >= kWideMinRowsPerExpert * (long long)r.E) {
      return launch_tile_gemm(kFmtFp8, r.w_layout == MOE_W_TILED,
                              routed_tile_args(a_q, a_scale, w_q, w_scale, r), nullptr, tiles, s);
    } else {
      auto k = r.w_layout ? gemm_big_kernel<kFmtFp8, true, kHWaves>
                          : gemm_big_kernel<kFmtFp8, false, kHWaves>;
      hipLaunchKernelGGL(k, dim3(tile_grid(tiles)), dim3(64 * kHWaves), 0, s, a_q, a_scale,
                         nullptr, w_q, w_scale, nullptr, r.sorted_ids, r.expert_ids, r.topk_w,
                         nullptr, r.M, r.K, r.N, r.E, r.top_k, r.max_blocks, r.y);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm_int8w8a8(const int8_t *a_q, const float *a_scale, const int8_t *w_q,
                               const float *w_scale, const RoutedArgs &r, hipStream_t s) {
  const uint8_t *ab = reinterpret_cast<const uint8_t *>(a_q);
  const uint8_t *wb = reinterpret_cast<const uint8_t *>(w_q);
  if (r.block_m == 16) {
    int groups, tpg;
    stream_grid(r.N, r.E, groups, tpg);
    auto k = stream_kernel_for<kSI8>(r.w_layout, false);
    hipLaunchKernelGGL(k, dim3(r.E * groups), dim3(kSThreads), 0, s, ab, a_scale, wb, w_scale,
                       r.sorted_ids, r.expert_ids, r.num_post, r.topk_w, r.M, r.K, r.N, r.top_k,
                       groups, tpg, r.max_blocks, r.y, stream_weight_bytes(r));
  } else {
    const long long tiles = (long long)(r.max_blocks / 2 + r.E) * ((r.N + kHBN - 1) / kHBN);
    return launch_tile_gemm(kFmtI8, r.w_layout == MOE_W_TILED,
                            routed_tile_args(ab, a_scale, wb, w_scale, r), nullptr, tiles, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_fp8w8a16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                                const RoutedArgs &r, hipStream_t s) {
  const uint8_t *ab = reinterpret_cast<const uint8_t *>(a);
  if (r.block_m == 16) {
    int groups, tpg;
    stream_grid(r.N, r.E, groups, tpg);
    auto k = stream_kernel_for<kSF8W16>(r.w_layout, stream_two_blocks(r));
    hipLaunchKernelGGL(k, dim3(r.E * groups), dim3(kSThreads), 0, s, ab, nullptr, w_q, w_scale,
                       r.sorted_ids, r.expert_ids, r.num_post, r.topk_w, r.M, r.K, r.N, r.top_k,
                       groups, tpg, r.max_blocks, r.y, stream_weight_bytes(r));
  } else {
    if ((long long)r.M * r.top_k >= kWideMinRowsPerExpert * (long long)r.E) {
      const long long tt = (long long)(r.max_blocks / 2 + r.E) * ((r.N + kHBN - 1) / kHBN);
      return launch_tile_gemm(kFmtF8W16, r.w_layout == MOE_W_TILED,
                              routed_tile_args(ab, nullptr, w_q, w_scale, r), nullptr, tt, s);
    }
    const long long tiles = (long long)r.max_blocks * ((r.N + kGBN - 1) / kGBN);
    auto k = r.w_layout ? gemm_kernel<kFmtF8W16, true> : gemm_kernel<kFmtF8W16, false>;
    hipLaunchKernelGGL(k, dim3(tile_grid(tiles)), dim3(kGThreads), 0, s, ab, nullptr, nullptr, w_q,
                       w_scale, nullptr, r.sorted_ids, r.expert_ids, r.topk_w, nullptr, r.M, r.K,
                       r.N, r.E, r.top_k, r.max_blocks, r.y);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_int8(const uint16_t *a, const int8_t *w_q, const float *w_scale,
                            const RoutedArgs &r, hipStream_t s) {
  const uint8_t *ab = reinterpret_cast<const uint8_t *>(a);
  const uint8_t *wb = reinterpret_cast<const uint8_t *>(w_q);
  if (r.block_m == 16) {
    int groups, tpg;
    stream_grid(r.N, r.E, groups, tpg);
    auto k = stream_kernel_for<kSW8A16>(r.w_layout, stream_two_blocks(r));
    hipLaunchKernelGGL(k, dim3(r.E * groups), dim3(kSThreads), 0, s, ab, nullptr, wb, w_scale,
                       r.sorted_ids, r.expert_ids, r.num_post, r.topk_w, r.M, r.K, r.N, r.top_k,
                       groups, tpg, r.max_blocks, r.y, stream_weight_bytes(r));
  } else {
    if ((long long)r.M * r.top_k >= kWideMinRowsPerExpert * (long long)r.E) {
      const long long tt = (long long)(r.max_blocks / 2 + r.E) * ((r.N + kHBN - 1) / kHBN);
      return launch_tile_gemm(kFmtInt8, r.w_layout == MOE_W_TILED,
                              routed_tile_args(ab, nullptr, wb, w_scale, r), nullptr, tt, s);
    }
    const long long tiles = (long long)r.max_blocks * ((r.N + kGBN - 1) / kGBN);
    auto k = r.w_layout ? gemm_kernel<kFmtInt8, true> : gemm_kernel<kFmtInt8, false>;
    hipLaunchKernelGGL(k, dim3(tile_grid(tiles)), dim3(kGThreads), 0, s, ab, nullptr, nullptr, wb,
                       w_scale, nullptr, r.sorted_ids, r.expert_ids, r.topk_w, nullptr, r.M, r.K,
                       r.N, r.E, r.top_k, r.max_blocks, r.y);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_int4w16(const uint16_t *a, const uint8_t *w_q, const float *w_scale,
                               const RoutedArgs &r, hipStream_t s) {
  // block_m 16 only (checked by the caller); w_q is the [E, N, K/2] byte matrix
  // or its MOE_W_FRAG packing
  int groups, tpg;
  stream_grid(r.N, r.E, groups, tpg);
  const uint32_t half = (uint32_t)(r.K / 2);
  const uint32_t w_bytes = r.w_layout == MOE_W_FRAG
                               ? (uint32_t)r.E * (uint32_t)((r.N + 15) / 16) * ((half + 63u) / 64u) * 1024u
                               : (uint32_t)r.E * (uint32_t)r.N * half;
  auto k = stream_kernel_for<kSW4A16>(r.w_layout, stream_two_blocks(r));
  hipLaunchKernelGGL(k, dim3(r.E * groups), dim3(kSThreads), 0, s,
                     reinterpret_cast<const uint8_t *>(a), nullptr, w_q, w_scale, r.sorted_ids,
                     r.expert_ids, r.num_post, r.topk_w, r.M, r.K, r.N, r.top_k, groups, tpg,
                     r.max_blocks, r.y, w_bytes);
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp8_wgrad(const uint8_t *dyT_q, const uint8_t *dyT_sf, const uint8_t *xT_q,
                                   const uint8_t *xT_sf, const int *padded_offsets, int E, int N,
                                   int K, uint16_t *dw, hipStream_t s) {
  WgradSeg seg{};
  for (int e = 0; e <= E; ++e) seg.po[e] = padded_offsets[e];
  // per expert ceil(N / 128) row blocks, in pairs, times ceil(K / 256) column tiles
  const long long pairs = (long long)E * (((N + kGBM - 1) / kGBM + 1) / 2);
  const long long tiles = pairs * ((K + kHBN - 1) / kHBN);
  TileArgs a{};
  a.a = dyT_q;
  a.a_sf = dyT_sf;
  a.w = xT_q;
  a.w_sf = xT_sf;
  a.out = dw;
  a.out_bytes = (uint32_t)((unsigned long long)E * N * K * 2ull);
  a.M = N;          // output rows per expert (dW_e is [N, K])
  a.K = 0;          // per expert: the padded row count of its segment
  a.N = K;
  a.E = E;
  a.top_k = 1;
  return launch_tile_gemm(kFmtMxW, false, a, &seg, tiles, s);
}

hipError_t launch_gemm_mxfp8(const uint8_t *a_q, const uint8_t *a_sf, const uint8_t *w_q,
                             const uint8_t *w_sf, const int *m_offsets, int rows, int K, int N,
                             int E, uint16_t *out, hipStream_t s) {
  // block pairs: at most (sum of blocks + E) / 2 + E
  const long long pairs = ((rows + kGBM - 1) / kGBM + E) / 2 + E;
  const long long tiles = pairs * ((N + kHBN - 1) / kHBN);
  TileArgs a{};
  a.a = a_q;
  a.a_sf = a_sf;
  a.w = w_q;
  a.w_sf = w_sf;
  a.m_offsets = m_offsets;
  a.out = out;
  a.out_bytes = (uint32_t)((unsigned long long)rows * N * 2ull);
  a.M = rows;
  a.K = K;
  a.N = N;
  a.E = E;
  a.top_k = 1;
  return launch_tile_gemm(kFmtMx, false, a, nullptr, tiles, s);
}

}  // namespace qmoe
