// Routing (top-k over the router logits) and block alignment of the routed
// slots: one workgroup for both up to 1024 tokens; above that the top-k runs
// on a grid of its own (one token per thread) and the workgroup aligns.
//
// The alignment produces the layout the grouped GEMMs consume: the slots
// i = t*top_k + j grouped by expert, each group padded to a multiple of
// block_m, and the expert of every block of block_m sorted slots.  The sort is
// a stable counting sort with no workgroup barrier inside its loops: each
// wavefront owns a contiguous range of slots.  For 64 slots at a time, one
// ballot per bit of the expert index gives every lane the mask of the lanes
// holding the same expert (its peers); mbcnt over that mask is the lane's rank
// among them, and the lowest peer alone updates the expert's entry in LDS
// (the leaders of one instruction hold distinct experts, so their updates do
// not collide).  A first walk counts each wavefront's slots per expert, a scan
// turns the counts into every wavefront's first position per expert, and a
// second walk hands out the positions.  Slot order inside an expert is
// therefore the ascending slot order.
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int lane_rank(unsigned long long mask) {
  // number of set bits of `mask` in the lanes below this one
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

// Top-k choice and router weights of the tokens t = tid, tid + kThreads, ...
// with top_k = kK known at compile time.
template <int kK>
__device__ __forceinline__ void route_tokens(const float *__restrict__ logits, int M, int E,
                                             int t_first, int t_step, int *__restrict__ topk_ids,
                                             float *__restrict__ topk_w, uint8_t *s_eid) {
  for (int t = t_first; t < M; t += t_step) {
    const float *lg = logits + (size_t)t * E;
    int ids[kK];
    float val[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      ids[j] = 0;
      val[j] = 0.0f;
    }
    int nfill = 0;
    for (int e0 = 0; e0 < E; e0 += 8) {
      float v8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v8[u] = e0 + u < E ? lg[e0 + u] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (e0 + u >= E) break;
        float cv = v8[u];
        int ci = e0 + u;
        // The list is ordered by (value descending, expert ascending).  The
        // new expert has the largest index so far, so it moves in only past
        // strictly smaller values; once it is placed, every entry below moves
        // down one position without another comparison (an entry that is
        // carried down must stay ahead of an equal value below it, which has
        // a larger index).
        bool carry = false;
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          if (carry || j >= nfill || cv > val[j]) {
            const float tv = val[j];
            const int ti = ids[j];
            val[j] = cv;
            ids[j] = ci;
            cv = tv;
            ci = ti;
            carry = true;
          }
        }
        nfill = min(nfill + 1, kK);
      }
    }
    // weights: exp(l_j - l_max) / sum over the chosen experts
    float ex[kK];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      ex[j] = expf(val[j] - val[0]);
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      const int i = t * kK + j;
      topk_ids[i] = ids[j];
      topk_w[i] = ex[j] / sum;
      if (s_eid) s_eid[i] = (uint8_t)ids[j];
    }
  }
}

__device__ __forceinline__ void route_tokens_k(const float *__restrict__ logits, int M, int E,
                                               int top_k, int t_first, int t_step,
                                               int *__restrict__ topk_ids,
                                               float *__restrict__ topk_w, uint8_t *s_eid) {
  switch (top_k) {
    case 1: route_tokens<1>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 2: route_tokens<2>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 3: route_tokens<3>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 4: route_tokens<4>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 5: route_tokens<5>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 6: route_tokens<6>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    case 7: route_tokens<7>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
    default: route_tokens<kMaxTopK>(logits, M, E, t_first, t_step, topk_ids, topk_w, s_eid); break;
  }
}

// Many tokens: the top-k choice runs on its own grid, one token per thread,
// before the one-workgroup alignment (one lone workgroup would take it at a
// few microseconds per 1024 tokens).
constexpr int kRouteThreads = 256;
constexpr int kSplitTokens = 1024;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float *__restrict__ logits,
                                                              int M, int E, int top_k,
                                                              int *__restrict__ topk_ids,
                                                              float *__restrict__ topk_w) {
  route_tokens_k(logits, M, E, top_k, blockIdx.x * kRouteThreads + threadIdx.x, M, topk_ids,
                 topk_w, nullptr);
}

// mask of the lanes whose `e` equals this lane's, among the lanes of `valid`
// (one ballot per bit of an index below 2^nbits)
__device__ __forceinline__ unsigned long long peer_mask(int e, int nbits,
                                                        unsigned long long valid) {
  unsigned long long peers = valid;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const unsigned long long mb = __ballot(bit);
    peers &= bit ? mb : ~mb;
  }
  return peers;
}

__global__ __launch_bounds__(kThreads) void route_align_kernel(
    const float *__restrict__ logits, int M, int E, int top_k, int block_m, int max_padded,
    int routed, int *__restrict__ topk_ids, float *__restrict__ topk_w,
    int *__restrict__ sorted_ids, int *__restrict__ expert_ids, int *__restrict__ num_post) {
  __shared__ uint8_t s_eid[kMaxSlots];            // expert of every slot
  __shared__ int s_cnt[kMaxExperts];              // slots per expert
  __shared__ int s_off[kMaxExperts + 1];          // padded start of every expert
  __shared__ int s_wcnt[kWaves][kMaxExperts];     // slots per wavefront range and expert
  __shared__ int s_wpos[kWaves][kMaxExperts];     // next position per wavefront and expert

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = M * top_k;

  for (int x = tid; x < kWaves * kMaxExperts; x += kThreads) (&s_wcnt[0][0])[x] = 0;

  // ---- 1. top-k choice and router weights of every token -------------------
  // One pass over the token's logits keeps the top_k best (value descending;
  // on equal values the lower expert index first) by insertion; logits are
  // read 8 at a time so their loads overlap.
  if (routed) {                                  // top-k already chosen by route_kernel
    for (int i = tid; i < S; i += kThreads) s_eid[i] = (uint8_t)topk_ids[i];
  } else {
    route_tokens_k(logits, M, E, top_k, tid, kThreads, topk_ids, topk_w, s_eid);
  }
  __syncthreads();

  // ---- 2. slots per wavefront range and expert ---------------------------------
  // Wavefront w owns slots [lo, hi).
  const int per = ((S + kWaves - 1) / kWaves + 63) & ~63;
  const int lo = min(wave * per, S), hi = min(lo + per, S);
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool valid = i < hi;
    const int my_e = valid ? (int)s_eid[i] : 0;
    const unsigned long long peers = peer_mask(my_e, nbits, __ballot(valid));
    if (valid && lane_rank(peers) == 0) atomicAdd(&s_wcnt[wave][my_e], __popcll(peers));
  }
  __syncthreads();

  // ---- 3. padded offsets of every expert and every wavefront's first
  // positions: wavefront 0, lane l holding experts l and l + 64 -------------
  if (wave == 0) {
    int w0[kWaves], w1[kWaves];
    int n0 = 0, n1 = 0;                            // slots of experts lane, lane + 64
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      w0[w] = s_wcnt[w][lane];
      w1[w] = s_wcnt[w][lane + 64];
      n0 += w0[w];
      n1 += w1[w];
    }
    if (lane < E) s_cnt[lane] = n0;
    if (lane + 64 < E) s_cnt[lane + 64] = n1;
    const int c0 = (n0 + block_m - 1) / block_m * block_m;   // zero past the last expert
    const int c1 = (n1 + block_m - 1) / block_m * block_m;
    int x0 = c0, x1 = c1;                          // inclusive scans over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y0 = __shfl_up(x0, d), y1 = __shfl_up(x1, d);
      if (lane >= d) {
        x0 += y0;
        x1 += y1;
      }
    }
    const int tot0 = __shfl(x0, 63);
    int r0 = x0 - c0, r1 = tot0 + x1 - c1;         // padded starts
    if (lane < E) s_off[lane] = r0;
    if (lane + 64 < E) s_off[lane + 64] = r1;
    const int total = tot0 + __shfl(x1, 63);
    if (lane == 0) {
      s_off[E] = total;
      *num_post = total;
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s_wpos[w][lane] = r0;
      s_wpos[w][lane + 64] = r1;
      r0 += w0[w];
      r1 += w1[w];
    }
  }
  __syncthreads();
  const int total = s_off[E];

  // ---- 4. block labels, padding and tail ---------------------------------------
  const int nblocks = max_padded / block_m;
  for (int b = tid; b < nblocks; b += kThreads) {
    const int p = b * block_m;
    int label = -1;
    if (p < total) {
      int e_lo = 0, e_hi = E - 1;                // last e with s_off[e] <= p
      while (e_lo < e_hi) {
        const int mid = (e_lo + e_hi + 1) >> 1;
        if (s_off[mid] <= p) e_lo = mid; else e_hi = mid - 1;
      }
      label = e_lo;
    }
    expert_ids[b] = label;
  }
  for (int e = wave; e < E; e += kWaves) {      // each expert's padding, one wavefront
    const int p1 = s_off[e + 1];
    for (int p = s_off[e] + s_cnt[e] + lane; p < p1; p += 64) sorted_ids[p] = S;
  }
  for (int p = total + tid; p < max_padded; p += kThreads) sorted_ids[p] = S;   // the tail

  // ---- 5. stable scatter of the slots -----------------------------------------
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool valid = i < hi;
    const int my_e = valid ? (int)s_eid[i] : 0;
    const unsigned long long peers = peer_mask(my_e, nbits, __ballot(valid));
    const int rank = lane_rank(peers);
    if (valid) {
      const int pos = s_wpos[wave][my_e];        // read by every lane first ...
      sorted_ids[pos + rank] = i;
      if (rank == 0) s_wpos[wave][my_e] = pos + __popcll(peers);   // ... then one per expert
    }
  }
}

}  // namespace

hipError_t launch_route_align(const float *logits, int M, int E, int top_k, int block_m,
                              int max_padded, int *topk_ids, float *topk_w, int *sorted_ids,
                              int *expert_ids, int *num_post, hipStream_t s) {
  const int routed = M > kSplitTokens;
  if (routed) {
    hipLaunchKernelGGL(route_kernel, dim3((M + kRouteThreads - 1) / kRouteThreads),
                       dim3(kRouteThreads), 0, s, logits, M, E, top_k, topk_ids, topk_w);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(route_align_kernel, dim3(1), dim3(kThreads), 0, s, logits, M, E, top_k,
                     block_m, max_padded, routed, topk_ids, topk_w, sorted_ids, expert_ids,
                     num_post);
  return hipGetLastError();
}

}  // namespace qmoe
