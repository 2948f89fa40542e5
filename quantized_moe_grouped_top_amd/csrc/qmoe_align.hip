// Routing (top-k over the router logits) and block alignment of the routed
// slots, in one workgroup.
//
// The alignment produces the layout the grouped GEMMs consume: the slots
// i = t*top_k + j grouped by expert, each group padded to a multiple of
// block_m, and the expert of every block of block_m sorted slots.  The sort is
// a stable counting sort: per chunk of 1024 slots, one wavefront ballot per
// expert gives each slot its rank among the slots of its expert inside its
// wavefront (mbcnt over the ballot mask), a prefix scan over the 16 wavefront
// counts gives the wavefront offsets, and a running count per expert carries
// the offsets across chunks.  Slot order inside an expert is therefore the
// ascending slot order.
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

__global__ __launch_bounds__(kThreads) void route_align_kernel(
    const float *__restrict__ logits, int M, int E, int top_k, int block_m, int max_padded,
    int *__restrict__ topk_ids, float *__restrict__ topk_w, int *__restrict__ sorted_ids,
    int *__restrict__ expert_ids, int *__restrict__ num_post) {
  __shared__ uint8_t s_eid[kMaxSlots];            // expert of every slot
  __shared__ int s_cnt[kMaxExperts];              // slots per expert
  __shared__ int s_off[kMaxExperts + 1];          // padded start of every expert
  __shared__ int s_run[kMaxExperts];              // slots of each expert already placed
  __shared__ int s_chunk[kMaxExperts];            // slots of each expert in this chunk
  __shared__ int s_wcnt[kWaves][kMaxExperts];     // per-wavefront counts of a chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = M * top_k;

  for (int e = tid; e < E; e += kThreads) {
    s_cnt[e] = 0;
    s_run[e] = 0;
  }
  __syncthreads();

  // ---- 1. top-k choice and router weights of every token -------------------
  // One pass over the token's logits keeps the top_k best (value descending;
  // on equal values the earlier expert stays, as a later one must be strictly
  // larger to move in) by insertion; logits are read 8 at a time so their
  // loads overlap.
  for (int t = tid; t < M; t += kThreads) {
    const float *lg = logits + (size_t)t * E;
    int ids[kMaxTopK];
    float val[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
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
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j < top_k && (j >= nfill || cv > val[j])) {   // place here, carry the old one down
            const float tv = val[j];
            const int ti = ids[j];
            val[j] = cv;
            ids[j] = ci;
            cv = tv;
            ci = ti;
          }
        }
        nfill = min(nfill + 1, top_k);
      }
    }
    // weights: exp(l_j - l_max) / sum over the chosen experts
    float ex[kMaxTopK];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      ex[j] = (j < top_k) ? expf(val[j] - val[0]) : 0.0f;
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < top_k) {
        const int i = t * top_k + j;
        topk_ids[i] = ids[j];
        topk_w[i] = ex[j] / sum;
        s_eid[i] = (uint8_t)ids[j];
        atomicAdd(&s_cnt[ids[j]], 1);
      }
    }
  }
  __syncthreads();

  // ---- 2. padded offsets of every expert --------------------------------------
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = acc;
      acc += (s_cnt[e] + block_m - 1) / block_m * block_m;
    }
    s_off[E] = acc;
    *num_post = acc;
  }
  __syncthreads();
  const int total = s_off[E];

  // ---- 3. block labels, padding and tail ---------------------------------------
  const int nblocks = max_padded / block_m;
  for (int b = tid; b < nblocks; b += kThreads) {
    const int p = b * block_m;
    int label = -1;
    if (p < total) {
      int lo = 0, hi = E - 1;                    // last e with s_off[e] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= p) lo = mid; else hi = mid - 1;
      }
      label = lo;
    }
    expert_ids[b] = label;
  }
  for (int p = tid; p < max_padded; p += kThreads) {
    bool pad = p >= total;
    if (!pad) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= p) lo = mid; else hi = mid - 1;
      }
      pad = p >= s_off[lo] + s_cnt[lo];
    }
    if (pad) sorted_ids[p] = S;                   // the sentinel
  }

  // ---- 4. stable scatter of the slots -----------------------------------------
  for (int base = 0; base < S; base += kThreads) {
    const int i = base + tid;
    const int my_e = (i < S) ? (int)s_eid[i] : -1;
    int my_rank = 0;
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot(my_e == e);
      if (lane == 0) s_wcnt[wave][e] = __popcll(m);
      if (my_e == e) my_rank = lane_rank(m);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {     // exclusive scan over wavefronts
      int acc = 0;
      for (int w = 0; w < kWaves; ++w) {
        const int c = s_wcnt[w][e];
        s_wcnt[w][e] = acc;
        acc += c;
      }
      s_chunk[e] = acc;
    }
    __syncthreads();
    if (my_e >= 0) sorted_ids[s_off[my_e] + s_run[my_e] + s_wcnt[wave][my_e] + my_rank] = i;
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) s_run[e] += s_chunk[e];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route_align(const float *logits, int M, int E, int top_k, int block_m,
                              int max_padded, int *topk_ids, float *topk_w, int *sorted_ids,
                              int *expert_ids, int *num_post, hipStream_t s) {
  hipLaunchKernelGGL(route_align_kernel, dim3(1), dim3(kThreads), 0, s, logits, M, E, top_k,
                     block_m, max_padded, topk_ids, topk_w, sorted_ids, expert_ids, num_post);
  return hipGetLastError();
}

}  // namespace qmoe
