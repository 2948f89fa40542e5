// The large-M grouped GEMM: 256 x 256 output tiles on four wavefronts (one
// per SIMD, 128 x 128 outputs each in 256 accumulation registers), for fp8
// W8A8, int8 W8A8, int8 W8A16 and fp8 weight-only over routed rows (block_m
// 128) and for MXFP8 (the forward grouped linear and its weight gradient).
//
// Operands.  A tile's rows are two 128-row routing blocks of one expert (the
// sorted slots) or 256 consecutive rows of an expert's segment (MXFP8); its
// columns are 256 output channels of that expert.  Each k-stage is 128 bytes
// of every activation row (128 k of one-byte codes, 64 k of bf16) and the
// same k of every weight column, copied HBM/L2 -> LDS by
// global_load_lds_dwordx4 (direct-to-LDS DMA, whole 128-byte lines, or 64-byte
// halves for the weights of bf16 stages) into a ring of stage slots (two of
// 64 KB; three of 48 KB for bf16 activations).  The contraction is
// v_mfma_*_32x32x64_f8f6f4 (scaled for MXFP8), two v_mfma_i32_32x32x32_i8, or,
// for bf16 activations, two v_mfma_f32_32x32x16_bf16 on weights widened to
// bf16 in registers (exact for int8 and e4m3 values), always with the weight
// fragment as the first operand.
//
// Persistent schedule.  One workgroup per CU.  The tiles are ordered expert
// by expert, column tile by column tile, block pair fastest (an expert with
// more than 8 block pairs: by groups of 8 column tiles, pairs within a
// group, columns fastest), and cut into eight contiguous chunks, one per XCD
// (workgroup b runs on XCD b mod 8, the dispatch order); the workgroups of an
// XCD take its chunk's tiles round robin, so the 32 tiles in flight on one
// XCD at a time are neighbours that share weight columns and activation rows
// in that XCD's L2.  The schedule is static: no device state, no atomics,
// every launch independent.
//
// Pipeline.  A stage is computed as two halves; the fragment reads of the
// next half are spread over the MFMAs of the current one.  Between the halves
// a wavefront waits for the next stage's copy and meets the others at the one
// barrier of the stage, which also frees the stage's slot; the second half
// then issues the DMA of the stage a ring's length ahead into that slot, one
// 1 KB piece per MFMA (per other MFMA for bf16).  The DMA runs across tile
// boundaries: the first stages of a workgroup's next tile (and, for routed
// rows, its sorted slots and router weights, fetched into LDS by dword DMA one
// tile ahead) are loaded while the current tile's last stages are computed,
// so a tile starts without waiting for memory.
//
// Epilogue.  Straight from the accumulators to HBM: the router weight and the
// scales are applied in float32, pairs are packed to bf16, and one
// v_permlane32_swap per register pair turns the MFMA's four-column runs into
// eight-column runs, so each lane stores whole 16-byte pieces.  The stores
// complete while the next tile's first half-stage computes.
//
// LDS rows are 128 bytes with 16-byte chunk c of row r at c ^ ((r >> 1) & 7)
// (the MOE_W_TILED block layout, so tiled weights are a plain copy), or 64
// bytes (bf16-stage weights) with chunk c at c ^ (((r >> 1) ^ (r >> 3)) & 3):
// the fragment reads (32 rows at one chunk per lane group) hit distinct banks.
#include "qmoe_device.h"

namespace qmoe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// every helper lambda of the kernel is inlined (an outlined one would move
// its captured state through scratch memory)
#define QMOE_INLINE __attribute__((always_inline))

constexpr int kTM = 256;                        // tile rows
constexpr int kTN = 256;                        // tile columns
constexpr int kARow = 128;                      // activation bytes per row and stage
constexpr int kASlot = kTM * kARow;             // 32 KB of activation rows per stage
constexpr int kSfSlot = 4 * (kTM + kTN);        // MXFP8: the scale dword of every row and column
constexpr int kMaxPairsTogether = 8;            // tile order: see decode()
constexpr int kColGroup = 8;

// chunk swizzles: 128-byte rows (8 chunks), 64-byte rows (4 chunks)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8 &a, const i32x8 &b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(const i32x4 &a, const i32x4 &b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_mx(const i32x8 &a, const i32x8 &b, f32x16 c, int sa,
                                            int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Fragments of one half-stage.  One-byte formats (64 k per half): for row
// (column) fragment i, lane 32 g + r holds row r, k 16g..16g+15 (lo) and
// 32+16g..32+16g+15 (hi) of the half; MXFP8: the e8m0 scale of 32-k block g
// of the half for row (column) r.  bf16 activations (32 k per half, two
// 32x32x16 MFMAs): lane 32 g + r holds k 16g..16g+7 (lo) and 16g+8..16g+15
// (hi) of activation row r, and the 16 weight bytes k 16g..16g+15 of column r
// in blo (bhi unused); the two MFMAs take the first and the last 8 k of each
// lane, a fixed assignment of k to the MFMA inputs that both operands share.
struct Frags {
  i32x4 alo[4], ahi[4], blo[4], bhi[4];
  int sa[4], sb[4];
};

// Order in which a half-stage's fragment parts are read: by first use in
// the MFMA order.  Part p: kind (0 A lo, 1 A hi, 2 B lo, 3 B hi) and fragment
// index.  One-byte formats, MFMA order (i, j) = (q >> 2, q & 3): 16 parts.
constexpr int kPartKind[16] = {0, 1, 2, 3, 2, 3, 2, 3, 2, 3, 0, 1, 0, 1, 0, 1};
constexpr int kPartFrag[16] = {0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 1, 1, 2, 2, 3, 3};
// bf16 activations, 32 MFMAs per half in the order (j, step, i) = (q >> 3,
// (q >> 2) & 1, q & 3) (four independent accumulators between the two steps
// of one): 12 parts, one read after every other MFMA.
constexpr int kPart16Kind[12] = {2, 0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2};
constexpr int kPart16Frag[12] = {0, 0, 1, 2, 3, 0, 1, 2, 3, 1, 2, 3};

template <int kFmt, bool kTiled>
__global__ __launch_bounds__(256, 1) void tile_kernel(const TileArgs p, const WgradSeg seg) {
  constexpr bool kW = kFmt == kFmtMxW;               // MXFP8 weight gradient
  constexpr bool kMx = kFmt == kFmtMx || kW;
  constexpr bool kRouted = !kMx;
  constexpr bool kI8 = kFmt == kFmtI8;
  // bf16 activations x byte weights (int8 W8A16, fp8 weight-only): weights
  // converted to bf16 in registers, bf16 MFMAs, 64 k per stage (the same 128
  // activation bytes per row), three stage slots
  constexpr bool kB16 = kFmt == kFmtInt8 || kFmt == kFmtF8W16;
  constexpr bool kCS = kI8 || kB16;                  // one weight scale per output column
  constexpr int kTK = kB16 ? 64 : 128;               // k per stage
  constexpr int kBRow = kB16 ? 64 : 128;             // weight bytes per row and stage
  constexpr int kRing = kB16 ? 3 : 2;                // stage slots
  // per-tile routing buffers: with one stage per tile the DMA cursor runs
  // kRing tiles ahead of the tile being computed (and fetches the sorted
  // slots of the tile after that one) while the computed tile's epilogue
  // still needs its own: kRing + 2 buffers of sorted slots, kRing + 1 of the
  // per-row and per-column scales
  constexpr int kInfo = kRing + 2;
  constexpr int kInfoS = kRing + 1;
  constexpr int kSlot = kASlot + kTN * kBRow;        // 48 / 64 KB per stage
  constexpr int kBP = kB16 ? 4 : 8;                  // weight DMA pieces per wavefront and stage
  constexpr int kPieces = 8 + kBP + (kMx ? 2 : 0);   // DMA instructions per wavefront and stage
  static_assert(!(kTiled && kMx), "MXFP8 weights are row-major");

  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kRing * kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s_sf[kMx ? kRing * kSfSlot : 16];
  __shared__ __attribute__((aligned(16))) int s_row[kRouted ? kInfo : 1][kTM];    // sorted slots
  __shared__ __attribute__((aligned(16))) float s_tw[kRouted ? kInfoS : 1][kTM];  // router weights
  __shared__ __attribute__((aligned(16))) float s_ts[kI8 ? kInfoS : 1][kTM];      // token scales
  __shared__ __attribute__((aligned(16))) float s_cs[kCS ? kInfoS : 1][kTN];      // column scales
  __shared__ int s_blk_first[kMaxExperts + 1];
  __shared__ int s_tile_first[kMaxExperts + 1];
  __shared__ int s_mo[kMx ? kMaxExperts + 1 : 1];     // first row of every segment
  __shared__ int s_po[kMx ? kMaxExperts + 1 : 1];     // first padded scale row (forward MXFP8)
  __shared__ float s_wsc[kFmt == kFmtFp8 ? kMaxExperts : 1];   // fp8: a_scale x w_scale[e]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;          // this wave's 128 x 128 block of the tile
  const int g = lane >> 5, r32 = lane & 31;
  const int M = p.M, K = p.K, N = p.N, E = p.E, top_k = p.top_k;
  const int S = M * top_k;
  const int ntn = (N + kTN - 1) / kTN;

  // ---- tile space ------------------------------------------------------------
  if constexpr (kRouted) {
    expert_block_starts(p.expert_ids, p.max_blocks, E, s_blk_first);
    __syncthreads();
  }
  if constexpr (kFmt == kFmtFp8) {
    for (int ee = tid; ee < E; ee += 256) s_wsc[ee] = p.a_scale[0] * p.w_scale[ee];
  }
  if (tid == 0) {
    int blk = 0, tiles = 0, po = 0;
    for (int ee = 0; ee < E; ++ee) {
      int nb;
      if constexpr (kMx) {
        int lo, hi;
        if constexpr (kW) {
          lo = ee * M;
          hi = lo + M;
        } else {
          lo = p.m_offsets ? p.m_offsets[ee] : 0;
          hi = p.m_offsets ? p.m_offsets[ee + 1] : M;
        }
        s_mo[ee] = lo;
        s_po[ee] = po;
        po += (hi - lo + kMxRowPad - 1) / kMxRowPad * kMxRowPad;
        nb = hi > lo ? (hi - lo + 127) / 128 : 0;
        s_blk_first[ee] = blk;
        blk += nb;
        if (ee == E - 1) {
          s_mo[E] = hi;
          s_po[E] = po;
          s_blk_first[E] = blk;
        }
      } else {
        nb = s_blk_first[ee + 1] - s_blk_first[ee];
      }
      s_tile_first[ee] = tiles;
      tiles += (nb + 1) / 2 * ntn;
    }
    s_tile_first[E] = tiles;
  }
  __syncthreads();

  // ---- this workgroup's tiles: XCD xq's chunk, round robin over its workgroups
  const int G = gridDim.x, b = blockIdx.x;
  const int xq = b & (kXcds - 1), wl = b / kXcds;
  const int Gx = (G - xq + kXcds - 1) / kXcds;
  const int total = s_tile_first[E];
  const int chunk = (total + kXcds - 1) / kXcds;
  const int c0 = xq * chunk, c1 = min(c0 + chunk, total);
  const int n_my = c0 + wl < c1 ? (c1 - c0 - wl + Gx - 1) / Gx : 0;
  if (n_my == 0) return;
  auto tile_of = [&](int k) QMOE_INLINE { return c0 + wl + k * Gx; };

  struct Tile {
    int e, nt, pr, nb, nst;
  };
  auto decode = [&](int k) QMOE_INLINE -> Tile {
    const int L = tile_of(k);
    int e = 0;
    while (s_tile_first[e + 1] <= L) ++e;
    e = __builtin_amdgcn_readfirstlane(e);
    const int nblk = __builtin_amdgcn_readfirstlane(s_blk_first[e + 1] - s_blk_first[e]);
    const int npair = (nblk + 1) >> 1;
    const int local = L - __builtin_amdgcn_readfirstlane(s_tile_first[e]);
    int nt, pr;
    if (npair <= kMaxPairsTogether) {
      // column tile by column tile, block pair fastest: every block pair of a
      // column tile is in flight at once, so its weights are read once
      nt = local / npair;
      pr = local - nt * npair;
    } else {
      // many row pairs (MXFP8 segments): groups of kColGroup column tiles,
      // pairs within a group, columns fastest, so that 32 consecutive tiles
      // are 4 pairs x 8 columns rather than 2 columns x 16 pairs
      const int grp = local / (npair * kColGroup);
      const int rem = local - grp * npair * kColGroup;
      const int gc = min(kColGroup, ntn - grp * kColGroup);   // columns in this group
      pr = rem / gc;
      nt = grp * kColGroup + (rem - pr * gc);
    }
    int nst = K / kTK;
    if constexpr (kW) nst = (seg.po[e + 1] - seg.po[e]) / kTK;
    return {e, nt, pr, min(2, nblk - 2 * pr), nst};
  };

  const uint32_t lds_ring = lds_addr(s_ring);
  const uint32_t lds_sf = lds_addr(s_sf);

  // ---- the DMA cursor: the next stage to load is stage cur_st of tile cur_k
  int cur_k = 0, cur_st = 0, cur_nst = 0;
  bool cur_live = true;                              // false once every stage is loaded
  int rl_st = 0;                                     // the last stage loaded (reloaded when done)
  int issued = 0;                                    // loads issued by this wave so far
  int info_mark = 0;                                 // `issued` just after the latest routing-info DMA
  uint32_t a_off[8], b_off[8], sf_off[2];
  const uint8_t *b_src = p.w;

  // routing info of tile k (its 256 sorted slots) into buffer k % kInfo; wave w
  // loads rows 64w .. 64w + 63 (rows of a missing second block repeat the first)
  auto issue_info = [&](int k) QMOE_INLINE {
    int lane_opaque = lane;
    asm volatile("" : "+v"(lane_opaque));
    const int lane = lane_opaque;
    const Tile t = decode(k);
    const int base = (s_blk_first[t.e] + 2 * t.pr) * 128;
    const int r = 64 * wave + lane;
    const int rr = r < t.nb * 128 ? r : (r & 127);
    dma4(p.sorted_ids, (uint32_t)(base + rr) * 4u, lds_addr(&s_row[k % kInfo][64 * wave]));
    info_mark = ++issued;
  };

  // Enter tile k: its DMA offsets (and, for routed rows, the routing info of
  // tile k + 1 and the gathers of tile k's router weights and scales).
  auto enter = [&](int k) QMOE_INLINE {
    // lane-derived values are recomputed here from an opaque copy of the lane
    // index, so that the compiler does not keep them live through the stages
    int lane_opaque = lane;
    asm volatile("" : "+v"(lane_opaque));
    const int lane = lane_opaque;                    // shadows the kernel-wide one
    const Tile t = decode(k);
    cur_k = k;
    cur_st = 0;
    cur_nst = t.nst;
    if (t.nst == 0) return;                          // (weight gradient of an empty expert)
    const int n0 = t.nt * kTN;
    if constexpr (kRouted) {
      const int buf = k % kInfo, bufs = k % kInfoS;
      // this tile's sorted slots have landed (once 64 or more loads follow
      // them they have: at most 63 are outstanding and loads return in order)
      if (k > 0 && issued - info_mark < 64) wait_dma_upto(issued - info_mark);
      if (k + 1 < n_my) issue_info(k + 1);
      const int nvalid = t.nb * 128;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int R = 64 * wave + 8 * u + (lane >> 3);
        const int slot = s_row[buf][R];
        const uint32_t tok = (R < nvalid && slot < S) ? (uint32_t)(slot / top_k) : 0u;
        a_off[u] = tok * (uint32_t)(kB16 ? 2 * K : K) + 16u * (uint32_t)((lane & 7) ^ swz(R));
      }
      {
        const int R = 64 * wave + lane;
        const int slot = s_row[buf][R];
        const int sl = (R < nvalid && slot < S) ? slot : 0;
        dma4(p.topk_w, (uint32_t)sl * 4u, lds_addr(&s_tw[bufs][64 * wave]));
        ++issued;
        if constexpr (kI8) {
          dma4(p.a_scale, (uint32_t)(sl / top_k) * 4u, lds_addr(&s_ts[bufs][64 * wave]));
          ++issued;
        }
        if constexpr (kCS) {
          const int col = min(n0 + 64 * wave + lane, N - 1);
          dma4(p.w_scale + (size_t)t.e * N, (uint32_t)col * 4u, lds_addr(&s_cs[bufs][64 * wave]));
          ++issued;
        }
      }
    } else {
      // MXFP8: the tile's rows are rows row0 .. of segment e (clamped to it)
      const int lo = s_mo[t.e], hi = s_mo[t.e + 1];
      const int row0 = lo + 2 * t.pr * 128;
      const uint32_t Ke = kW ? (uint32_t)(seg.po[t.e + 1] - seg.po[t.e]) : (uint32_t)K;
      const uint32_t pe = kW ? (uint32_t)seg.po[t.e] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int R = 64 * wave + 8 * u + (lane >> 3);
        const uint32_t row = (uint32_t)min(row0 + R, hi - 1);
        const uint32_t chunk = 16u * (uint32_t)((lane & 7) ^ swz(R));
        if constexpr (kW) a_off[u] = (uint32_t)M * pe + (row - (uint32_t)lo) * Ke + chunk;
        else a_off[u] = row * (uint32_t)K + chunk;
      }
      {
        const uint32_t row = (uint32_t)min(row0 + 64 * wave + lane, hi - 1);
        const uint32_t col = (uint32_t)min(n0 + 64 * wave + lane, N - 1);
        if constexpr (kW) {
          sf_off[0] = (uint32_t)M * pe / 32u + (row - (uint32_t)lo) * (Ke / 32u);
          sf_off[1] = (uint32_t)N * pe / 32u + col * (Ke / 32u);
        } else {
          sf_off[0] = ((uint32_t)s_po[t.e] + row - (uint32_t)lo) * ((uint32_t)K / 32u);
          sf_off[1] = ((uint32_t)t.e * (uint32_t)N + col) * ((uint32_t)K / 32u);
        }
      }
    }
    // weight columns: wave w loads columns 64w .. 64w + 63 of the tile
    if constexpr (kTiled) {
      // MOE_W_TILED: 8 KB blocks of 64 rows x 128 k bytes, chunk c of row r
      // at c ^ ((r >> 1) & 7).  One-byte formats: one block per stage, in the
      // LDS row order and swizzle already.  bf16 activations: a 64-k stage is
      // chunks 4h .. 4h + 3 of the rows (h = stage parity), which for row r
      // sit at bit 6 of the offset flipped by h
      const int T = (N + 63) / 64;
      const int S128 = (K + 127) / 128;
      const int tb = min(n0 / 64 + wave, T - 1);
      b_src = p.w + (size_t)((t.e * T + tb) * S128) * 8192u;
      if constexpr (kB16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 16 * u + (lane >> 2);
          const int x = (r >> 1) & 7;
          const int c = (lane & 3) ^ swz64(r);
          b_off[u] = (uint32_t)(r * 128 + 16 * ((c ^ x) & 3) + 64 * ((x >> 2) & 1));
        }
      }
    } else if constexpr (kB16) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int R = 64 * wave + 16 * u + (lane >> 2);
        const uint32_t col = (uint32_t)min(n0 + R, N - 1);
        b_off[u] = ((uint32_t)t.e * (uint32_t)N + col) * (uint32_t)K +
                   16u * (uint32_t)((lane & 3) ^ swz64(R));
      }
      b_src = p.w;
    } else {
      const uint32_t Ke = kW ? (uint32_t)(seg.po[t.e + 1] - seg.po[t.e]) : (uint32_t)K;
      const uint32_t pe = kW ? (uint32_t)seg.po[t.e] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int R = 64 * wave + 8 * u + (lane >> 3);
        const uint32_t col = (uint32_t)min(n0 + R, N - 1);
        const uint32_t chunk = 16u * (uint32_t)((lane & 7) ^ swz(R));
        if constexpr (kW) b_off[u] = (uint32_t)N * pe + col * Ke + chunk;
        else b_off[u] = ((uint32_t)t.e * (uint32_t)N + col) * (uint32_t)K + chunk;
      }
      b_src = p.w;
    }
  };

  // Make (cur_k, cur_st) a stage that exists, entering the next tiles as
  // needed; cur_live turns false once every stage has been loaded.
  auto advance = [&]() QMOE_INLINE {
    while (cur_live && cur_st >= cur_nst) {
      if (cur_k + 1 < n_my) enter(cur_k + 1);
      else cur_live = false;
    }
  };

  // DMA piece q of stage st of the cursor's tile into ring slot `slot`:
  // 0-7 activation rows, 8.. weight rows (1 KB each), then the two MXFP8
  // scale dwords
  auto issue_piece = [&](int q, int slot, uint32_t st) QMOE_INLINE {
    const uint32_t base = lds_ring + (uint32_t)(slot * kSlot);
    if (q < 8) {
      dma16(p.a + st * kARow, a_off[q], base + (uint32_t)((8 * wave + q) * 1024));
    } else if (q < 8 + kBP) {
      const int u = q - 8;
      const uint32_t dst = base + (uint32_t)(kASlot + (kBP * wave + u) * 1024);
      if constexpr (kB16) {
        if constexpr (kTiled) dma16(b_src + (st >> 1) * 8192u, b_off[u] ^ ((st & 1u) << 6), dst);
        else dma16(b_src + st * kBRow, b_off[u], dst);
      } else {
        if constexpr (kTiled) dma16(b_src + st * 8192u, (uint32_t)(u * 1024) + 16u * (uint32_t)lane, dst);
        else dma16(b_src + st * kBRow, b_off[u], dst);
      }
    } else if constexpr (kMx) {
      const uint32_t sbase = lds_sf + (uint32_t)(slot * kSfSlot);
      if (q == 8 + kBP) dma4(p.a_sf + 4u * st, sf_off[0], sbase + (uint32_t)(256 * wave));
      else dma4(p.w_sf + 4u * st, sf_off[1], sbase + (uint32_t)(4 * kTM + 256 * wave));
    }
  };

  // ---- fragments ------------------------------------------------------------
  const int sw = swz(r32);                          // (32i + r32 has the same swizzle)
  const int sw64 = swz64(r32);
  constexpr int kParts = kB16 ? 12 : 16;            // fragment reads per half-stage
  constexpr int kMf = kB16 ? 32 : 16;               // MFMA instructions per half-stage
  auto read_part = [&](int slot, int h, Frags &f, int part) QMOE_INLINE {
    int kind, i;
    const uint8_t *p8;
    if constexpr (kB16) {
      kind = kPart16Kind[part];
      i = kPart16Frag[part];
      if (kind < 2)
        p8 = s_ring + slot * kSlot + wm * 128 * kARow + (32 * i + r32) * kARow +
             (((4 * h + 2 * g + kind) ^ sw) << 4);
      else
        p8 = s_ring + slot * kSlot + kASlot + wn * 128 * kBRow + (32 * i + r32) * kBRow +
             (((2 * h + g) ^ sw64) << 4);
    } else {
      kind = kPartKind[part];
      i = kPartFrag[part];
      p8 = s_ring + slot * kSlot + (kind < 2 ? wm * 128 * kARow : kASlot + wn * 128 * kBRow) +
           (32 * i + r32) * kARow + (((4 * h + g + ((kind & 1) ? 2 : 0)) ^ sw) << 4);
    }
    const i32x4 v = *reinterpret_cast<const i32x4 *>(p8);
    if (kind == 0) f.alo[i] = v;
    else if (kind == 1) f.ahi[i] = v;
    else if (kind == 2) f.blo[i] = v;
    else f.bhi[i] = v;
  };
  // MXFP8 scales of half h: byte 2h + g of the stage's scale dword (part i:
  // row fragment i, part 4 + j: column fragment j)
  auto read_scale_part = [&](int slot, int h, Frags &f, int part) QMOE_INLINE {
    if constexpr (kMx) {
      const uint8_t *sfs = s_sf + slot * kSfSlot;
      const int sh = 8 * (2 * h + g);
      const int i = part & 3;
      if (part < 4)
        f.sa[i] = (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * (wm * 128 + 32 * i + r32)) >> sh) & 0xFFu);
      else
        f.sb[i] = (int)((*reinterpret_cast<const uint32_t *>(sfs + 4 * kTM + 4 * (wn * 128 + 32 * i + r32)) >> sh) & 0xFFu);
    }
  };
  // the reads that follow MFMA q (of kMf) in a half-stage: fragment parts
  // (one-byte formats: part q; bf16 activations: part q / 2 after even q)
  auto reads_after = [&](int q, int slot, int h, Frags &f) QMOE_INLINE {
    if constexpr (kB16) {
      if ((q & 1) == 0 && q / 2 < kParts) read_part(slot, h, f, q / 2);
    } else {
      read_part(slot, h, f, q);
      if (kMx && q >= 8) read_scale_part(slot, h, f, q - 8);
    }
  };
  // the DMA piece issued after MFMA q of a second half-stage (-1: none)
  auto piece_after = [&](int q) QMOE_INLINE -> int {
    if constexpr (kB16) return (q & 1) && q / 2 < kPieces ? q / 2 : -1;
    else return q < 16 ? q : -1;
  };

  f32x16 acc[4][4];
  auto zero_acc = [&]() QMOE_INLINE {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  };
  // bf16 activations: the weights of column fragment j are widened while the
  // MFMAs of fragment j - 1 run, one bf16 word after each MFMA (the first
  // fragment of a half during the last group of the half before), so no MFMA
  // waits for a conversion
  i32x4 wcv[2], wnx[2];                             // widened weights: current, next fragment
  auto widen_part = [&](const i32x4 &src, int m) QMOE_INLINE {
    int *dst = reinterpret_cast<int *>(&wnx[m >> 2]);
    dst[m & 3] = dequant_pair<kFmt == kFmtF8W16>((uint32_t)src[m >> 1], m & 1);
  };
  auto mfma_q = [&](const Frags &f, const Frags &fn, int q) QMOE_INLINE {
    if constexpr (kB16) {
      const int j = q >> 3, m = q & 7, st = m >> 2, i = m & 3;
      if (m == 0) {
        wcv[0] = wnx[0];
        wcv[1] = wnx[1];
      }
      acc[i][j] = mfma32_bf16(wcv[st], st ? f.ahi[i] : f.alo[i], acc[i][j]);
      widen_part(j < 3 ? f.blo[j + 1] : fn.blo[0], m);
      return;
    }
    const int i = q >> 2, j = q & 3;
    const i32x8 av = __builtin_shufflevector(f.alo[i], f.ahi[i], 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 bv = __builtin_shufflevector(f.blo[j], f.bhi[j], 0, 1, 2, 3, 4, 5, 6, 7);
    if constexpr (kMx) {
      acc[i][j] = mfma32_mx(bv, av, acc[i][j], f.sb[j], f.sa[i]);
    } else if constexpr (kI8) {
      // two 32x32x32 int8 MFMAs over the two 16-byte halves (A and B share the
      // k placement); int32 accumulators carried as raw bits
      i32x16 ci = __builtin_bit_cast(i32x16, acc[i][j]);
      ci = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.blo[j], f.alo[i], ci, 0, 0, 0);
      ci = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.bhi[j], f.ahi[i], ci, 0, 0, 0);
      acc[i][j] = __builtin_bit_cast(f32x16, ci);
    } else {
      acc[i][j] = mfma32_fp8(bv, av, acc[i][j]);
    }
  };
  auto pin_acc = [&]() QMOE_INLINE {     // the accumulators are "used" here: no MFMA sinks past
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  };

  // ---- prologue: routing info of the first tile, then kRing stages -------------
  // Every stage issues its kPieces DMA instructions (once the last tile's
  // stages are all loaded, the last one again, into the slot just freed).
  if constexpr (kRouted) {
    issue_info(0);
    wait_dma_all();
  }
  enter(0);
  advance();
  const bool any = cur_live;                         // some tile has stages
  if (any) {
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      if (s > 0) advance();
      const uint32_t st = (uint32_t)(cur_live ? cur_st : rl_st);
#pragma unroll
      for (int q = 0; q < kPieces; ++q) issue_piece(q, s, st);
      issued += kPieces;
      if (cur_live) {
        rl_st = cur_st;
        ++cur_st;
      }
    }
    // stage 0 has landed here (the loads after it: the later stages' pieces
    // and at most a few routing loads before them)
    wait_dma_upto((kRing - 1) * kPieces);
  }
  lds_barrier();
  Frags fa, fb;
#pragma unroll
  for (int part = 0; part < kParts; ++part) read_part(0, 0, fa, part);
#pragma unroll
  for (int part = 0; part < 8; ++part) read_scale_part(0, 0, fa, part);
  wait_lds();
  if constexpr (kB16) {
#pragma unroll
    for (int m = 0; m < 8; ++m) widen_part(fa.blo[0], m);
  }
  zero_acc();

  // One stage (flat index t, ring slot t % kRing): half 0 on `fa` while half
  // 1's fragments are read into `fb`; the wait for stage t + 1 and the
  // barrier; half 1 on `fb` while stage t + kRing is issued into slot
  // t % kRing and half 0 of stage t + 1 is read into `fa`.  With three slots
  // the wait leaves stage t + 2 in flight (vmcnt(kPieces)), except after an
  // epilogue, whose stores may complete out of order with the loads.
  int t = 0;
  bool after_epi = false;
  auto stage = [&]() QMOE_INLINE {
    const int slot = t % kRing, nslot = (t + 1) % kRing;
#pragma unroll
    for (int q = 0; q < kMf; ++q) {
      mfma_q(fa, fb, q);
      reads_after(q, slot, 1, fb);
      __builtin_amdgcn_sched_barrier(0);
    }
    pin_acc();
    wait_lds();                                     // this wave is done with the slot
    if (kRing == 2 || after_epi) wait_dma_all();    // stage t + 1 has landed here ...
    else wait_dma_upto(kPieces);
    after_epi = false;
    lds_barrier();                                  // ... everywhere; the slot is free
    advance();
    const uint32_t st = (uint32_t)(cur_live ? cur_st : rl_st);
#pragma unroll
    for (int q = 0; q < kMf; ++q) {
      mfma_q(fb, fa, q);
      const int pc = piece_after(q);
      if (pc >= 0) issue_piece(pc, slot, st);
      reads_after(q, nslot, 0, fa);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kMx) {
      issue_piece(16, slot, st);
      issue_piece(17, slot, st);
    }
    pin_acc();
    wait_lds();
    issued += kPieces;
    if (cur_live) {
      rl_st = cur_st;
      ++cur_st;
    }
    ++t;
  };

  // ---- epilogue: scale, pack to bf16, store 16-byte pieces -------------------
  auto epilogue = [&](int k) QMOE_INLINE {
    int lane_opaque = lane;
    asm volatile("" : "+v"(lane_opaque));
    const int lane = lane_opaque;
    const int g = lane >> 5, r32 = lane & 31;
    const Tile tl = decode(k);
    const int n0 = tl.nt * kTN;
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.out, (short)0, (int)p.out_bytes, 0x00020000);
    const int buf = k % kInfo, bufs = k % kInfoS;
    const float sc = kFmt == kFmtFp8 ? s_wsc[tl.e] : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = wm * 128 + 32 * i + r32;        // this lane's tile row
      int dst;
      float rs = 1.0f;
      if constexpr (kRouted) {
        const int slot = s_row[buf][R];
        dst = (R < tl.nb * 128 && slot < S) ? slot : -1;
        rs = kI8 ? s_ts[bufs][R] * s_tw[bufs][R] : (kB16 ? s_tw[bufs][R] : sc * s_tw[bufs][R]);
      } else {
        const int row = s_mo[tl.e] + 2 * tl.pr * 128 + R;
        dst = row < s_mo[tl.e + 1] ? row : -1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cb = wn * 128 + 32 * j;             // column of the fragment in the tile
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = acc[i][j][8 * kk + u];
          if constexpr (kCS) {
            // times the column scales (int8 W8A8: int32 -> float first):
            // accumulator 4k + c is column 8k + 4g + c of the fragment
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4 cs =
                  *reinterpret_cast<const f32x4 *>(&s_cs[bufs][cb + 8 * (2 * kk + h) + 4 * g]);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float raw = v[4 * h + c];
                v[4 * h + c] = (kI8 ? (float)__builtin_bit_cast(int, raw) : raw) * cs[c];
              }
            }
          }
          const int x0 = (int)f32x2_to_bf16x2(v[0] * rs, v[1] * rs);
          const int x1 = (int)f32x2_to_bf16x2(v[2] * rs, v[3] * rs);
          const int y0 = (int)f32x2_to_bf16x2(v[4] * rs, v[5] * rs);
          const int y1 = (int)f32x2_to_bf16x2(v[6] * rs, v[7] * rs);
          // lanes 0-31 hold columns 4g.. of runs 2kk and 2kk + 1 (g = 0),
          // lanes 32-63 the others: one swap each leaves 8 columns in a row
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const i32x4 piece = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
          const int col = n0 + cb + 16 * kk + 8 * g;
          // rows that are not outputs and columns past N store out of the
          // buffer's range, which the hardware drops
          const uint32_t off = (dst >= 0 && col < N)
                                   ? ((uint32_t)dst * (uint32_t)N + (uint32_t)col) * 2u
                                   : 0xFFFFFFF0u;
          __builtin_amdgcn_raw_buffer_store_b128(piece, orsrc, off, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // ---- tiles -------------------------------------------------------------------
  for (int k = 0; k < n_my; ++k) {
    const int nst = decode(k).nst;
    for (int s = 0; s < nst; ++s) stage();
    epilogue(k);
    zero_acc();
    after_epi = true;
  }
  wait_dma_all();                                   // no copy into LDS outlives the workgroup
}

}  // namespace

hipError_t launch_tile_gemm(int fmt, bool tiled, const TileArgs &args, const WgradSeg *seg,
                            long long tiles_bound, hipStream_t s) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    ncu = 256;
  const long long grid = tiles_bound < ncu ? (tiles_bound > 0 ? tiles_bound : 1) : ncu;
  const WgradSeg none{};
  const WgradSeg &sg = seg ? *seg : none;
  const dim3 gd((unsigned)grid), bd(256);
  switch (fmt) {
    case kFmtFp8:
      if (tiled) hipLaunchKernelGGL((tile_kernel<kFmtFp8, true>), gd, bd, 0, s, args, sg);
      else hipLaunchKernelGGL((tile_kernel<kFmtFp8, false>), gd, bd, 0, s, args, sg);
      break;
    case kFmtI8:
      if (tiled) hipLaunchKernelGGL((tile_kernel<kFmtI8, true>), gd, bd, 0, s, args, sg);
      else hipLaunchKernelGGL((tile_kernel<kFmtI8, false>), gd, bd, 0, s, args, sg);
      break;
    case kFmtInt8:
      if (tiled) hipLaunchKernelGGL((tile_kernel<kFmtInt8, true>), gd, bd, 0, s, args, sg);
      else hipLaunchKernelGGL((tile_kernel<kFmtInt8, false>), gd, bd, 0, s, args, sg);
      break;
    case kFmtF8W16:
      if (tiled) hipLaunchKernelGGL((tile_kernel<kFmtF8W16, true>), gd, bd, 0, s, args, sg);
      else hipLaunchKernelGGL((tile_kernel<kFmtF8W16, false>), gd, bd, 0, s, args, sg);
      break;
    case kFmtMx:
      hipLaunchKernelGGL((tile_kernel<kFmtMx, false>), gd, bd, 0, s, args, sg);
      break;
    case kFmtMxW:
      hipLaunchKernelGGL((tile_kernel<kFmtMxW, false>), gd, bd, 0, s, args, sg);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmoe
