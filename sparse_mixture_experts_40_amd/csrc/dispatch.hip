// dispatch.hip — stable counting sort of the routing pairs by expert.
//
// Replaces the one-hot expert mask and the per-expert torch.where loop of
// [QWEN3-READ] "大模型-qwen3 MoE 详细解读" (cnblogs), forward code, by the token
// permutation (and its inverse) that its §三 describes for production kernels.
//
// Pairs p = t*k + j are cut into chunks of kChunk consecutive ids, one block
// each:
//   hist    : per-chunk LDS histogram (integer LDS atomics: exact, order-free)
//   scan    : one block; per-expert totals, kept counts min(total, capacity),
//             exclusive scan of the kept counts, and the rank inside its expert
//             of the first pair of every (chunk, expert) run
//   scatter : each chunk walks its pairs in ascending order, 256 at a time; a
//             lane's rank among equal experts comes from 8 ballots (one per
//             bit of the expert id), wave counts go through LDS, so pairs of an
//             expert land in ascending pair order (a stable sort).
// With a single chunk (P <= kChunk, the decode case) the three steps run in
// one block and one launch; a second block of the same launch (do_aux) makes
// the same histogram and from it the load-balance statistics, while the
// first one sorts, so they need no launch of their own.
// Capacity ([MOE-128x8] 容量因子设计; [QWEN3-ROUTE] §四, tokens taken in order,
// an expert accepts while below its capacity): the pair of rank r inside its
// expert is kept iff r < capacity, i.e. each expert keeps its first
// `capacity` pairs in pair order; a dropped pair gets pair_pos = -1. A
// capacity of 0 keeps every pair. A negative expert id marks an empty slot (a
// token routed to fewer than k experts): it is not a pair and gets
// pair_pos = -1.
// No device-to-host traffic; everything stays on the stream.
#include "aux_small.h"
#include "dispatch_chunk.h"

namespace moe {

namespace {

constexpr int kChunk = kDispChunk;
constexpr int kThreads = kDispThreads;

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(int P, int E,
                                                                 const int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ hist) {
  __shared__ int s_h[256];
  const int tid = threadIdx.x;
  s_h[tid] = 0;
  __syncthreads();
  hist_chunk(P, E, idx, blockIdx.x * kChunk, s_h);
  __syncthreads();
  if (tid < E) hist[(size_t)blockIdx.x * E + tid] = s_h[tid];
}

__global__ __launch_bounds__(kThreads) void dispatch_scan_kernel(
    int nchunks, int E, int cap, const int32_t* __restrict__ hist, int32_t* __restrict__ rank0,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dropped) {
  __shared__ int s_c[256];
  __shared__ int s_drop;
  const int e = threadIdx.x;
  if (e == 0) s_drop = 0;
  int tot = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = 0; b < nchunks; ++b) tot += hist[(size_t)b * E + e];
  }
  const int kept = (cap > 0 && tot > cap) ? cap : tot;
  s_c[e] = kept;
  __syncthreads();
  if (kept < tot) atomicAdd(&s_drop, tot - kept);  // integer: exact, order-free
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan over the 256 slots
    const int add = (e >= d) ? s_c[e - d] : 0;
    __syncthreads();
    s_c[e] += add;
    __syncthreads();
  }
  const int excl = s_c[e] - kept;
  if (e < E) {
    if (counts) counts[e] = tot;
    if (offsets) offsets[e] = excl;
    if (offsets && e == E - 1) offsets[E] = s_c[e];
    if (rank0) {
      int run = 0;
#pragma unroll 8
      for (int b = 0; b < nchunks; ++b) {
        rank0[(size_t)b * E + e] = run;
        run += hist[(size_t)b * E + e];
      }
    }
  }
  if (dropped && e == 0) *dropped = s_drop;
}

// The global outputs of a scatter: sorted_pair[pos] = p, pair_pos[p] = pos,
// and pair_pos = -1 for a dropped pair or an empty slot.
struct GlobalSink {
  int32_t* sorted_pair;
  int32_t* pair_pos;
  __device__ void operator()(int p, int pos) const {
    sorted_pair[pos] = p;
    pair_pos[p] = pos;
  }
};
struct GlobalDrop {
  int32_t* pair_pos;
  __device__ void operator()(int p) const { pair_pos[p] = -1; }
};

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    int P, int E, int cap, const int32_t* __restrict__ idx, const int32_t* __restrict__ rank0,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int s_rank[256];  // rank inside its expert of this chunk's next pair
  __shared__ int s_off[256];
  __shared__ int s_wc[4][256];
  const int tid = threadIdx.x;
  if (tid < E) {
    s_rank[tid] = rank0[(size_t)blockIdx.x * E + tid];
    s_off[tid] = offsets[tid];
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) s_wc[w][tid] = 0;
  __syncthreads();
  scatter_chunk(P, E, cap, idx, blockIdx.x * kChunk, s_rank, s_off, s_wc,
                GlobalSink{sorted_pair, pair_pos}, GlobalDrop{pair_pos});
}

// One chunk (P <= kChunk): histogram, scan and scatter in one block. Every
// expert's first pair of the chunk has rank 0, so the result is that of the
// three kernels above.
__global__ __launch_bounds__(kThreads) void dispatch_single_kernel(
    int P, int E, int cap, const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dropped, int scatter,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos, int do_aux,
    AuxSmallArgs aux) {
  __shared__ int s_h[256];
  __shared__ int s_c[256];
  __shared__ int s_off[256];
  __shared__ int s_wc[4][256];
  __shared__ int s_drop;
  const int e = threadIdx.x;
  s_h[e] = 0;
  if (e == 0) s_drop = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) s_wc[w][e] = 0;
  __syncthreads();
  hist_chunk(P, E, idx, 0, s_h);
  __syncthreads();
  const int tot = e < E ? s_h[e] : 0;
  if (blockIdx.x == 1) {  // the statistics, next to block 0's sort
    if (do_aux) aux_small_body(aux, e < E ? tot : 0);  // block-uniform
    return;
  }
  const int kept = (cap > 0 && tot > cap) ? cap : tot;
  s_c[e] = kept;
  __syncthreads();
  if (kept < tot) atomicAdd(&s_drop, tot - kept);  // integer: exact, order-free
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan over the 256 slots
    const int add = (e >= d) ? s_c[e - d] : 0;
    __syncthreads();
    s_c[e] += add;
    __syncthreads();
  }
  const int excl = s_c[e] - kept;
  if (e < E) {
    if (counts) counts[e] = tot;
    if (offsets) offsets[e] = excl;
    if (offsets && e == E - 1) offsets[E] = s_c[e];
  }
  if (dropped && e == 0) *dropped = s_drop;
  if (!scatter) return;  // block-uniform
  s_off[e] = excl;
  s_h[e] = 0;  // becomes the running rank of each expert
  __syncthreads();
  scatter_chunk(P, E, cap, idx, 0, s_h, s_off, s_wc, GlobalSink{sorted_pair, pair_pos},
                GlobalDrop{pair_pos});
}

// Least-loaded fallback of a capacity limit ([QWEN3-ROUTE] §四: a token left
// with fewer than fallback_min accepted experts gets the least-loaded ones
// added, and those are not counted as accepted). Input: the dropless
// dispatch of the same routing. Pair p of expert e has rank
// pair_pos[p] - offsets[e] in its expert and is kept iff that rank is below
// the capacity. The load of e that token t sees (its accepted pairs among
// tokens <= t) is min(capacity, pairs of e with an id below (t + 1) k),
// found by binary search in e's segment of sorted_pair (ascending pair ids),
// so tokens do not depend on each other. A short token takes the experts with
// the smallest (load, id), one wave minimum per expert, into its dropped
// slots in slot order, each with that slot's weight; the other dropped slots
// and the empty ones get id -1 and weight 0. One wave per token; E <= 256.
__global__ __launch_bounds__(kThreads) void capacity_fallback_kernel(
    int T, int E, int k, int cap, int fmin, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ dropped) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const size_t p = (size_t)t * k + lane;
  int e = -1;
  float wv = 0.0f;
  bool kept = false, drop = false;
  if (lane < k) {
    e = idx[p];
    wv = w[p];
    if (e >= 0) {  // a pair (a negative id is an empty slot)
      kept = pair_pos[p] - offsets[disp_clamp_expert(e, E)] < cap;
      drop = !kept;
    }
  }
  const unsigned long long dm = __ballot(drop);
  const int nkept = __popcll(__ballot(kept)), ndrop = __popcll(dm);
  int need = fmin - nkept;
  need = need > ndrop ? ndrop : (need < 0 ? 0 : need);
  int out_e = kept ? e : -1;
  float out_w = kept ? wv : 0.0f;
  if (need > 0) {  // wave-uniform
    const int lim = (t + 1) * k;  // pair ids of the tokens up to t
    unsigned long long key[4];    // (load, expert) of experts lane + 64 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane + 64 * i;
      key[i] = ~0ull;
      if (ee < E) {
        const int base = offsets[ee];
        int lo = base, hi = offsets[ee + 1];
        while (lo < hi) {  // first entry with a pair id >= lim
          const int mid = (lo + hi) >> 1;
          if (sorted_pair[mid] < lim) lo = mid + 1; else hi = mid;
        }
        const int load = lo - base < cap ? lo - base : cap;
        key[i] = ((unsigned long long)(unsigned)load << 32) | (unsigned)ee;
      }
    }
    // pick r goes to the dropped slot of rank r (slot order)
    const int rank = __popcll(dm & ((1ull << lane) - 1ull));
    for (int r = 0; r < need; ++r) {
      unsigned long long m = key[0] < key[1] ? key[0] : key[1];
      const unsigned long long m2 = key[2] < key[3] ? key[2] : key[3];
      m = m2 < m ? m2 : m;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(m, off);
        m = o < m ? o : m;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key[i] == m) key[i] = ~0ull;
      if (drop && rank == r) {
        out_e = (int)(unsigned)(m & 0xFFFFFFFFull);
        out_w = wv;
      }
    }
  }
  if (lane < k) {
    idx_out[p] = out_e;
    w_out[p] = out_w;
  }
  if (dropped && lane == 0 && ndrop > need) atomicAdd(dropped, ndrop - need);  // exact
}

__global__ void zero_count_kernel(int32_t* __restrict__ n) {
  if (threadIdx.x == 0) n[0] = 0;
}

}  // namespace

int dispatch_num_chunks(const moe_config& c) {
  const long P = (long)c.num_tokens * c.top_k;
  return (int)((P + kChunk - 1) / kChunk);
}

hipError_t launch_dispatch(const moe_config& c, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* hist, int32_t* rank0, bool scatter, int capacity,
                           int32_t* dropped, hipStream_t s) {
  const int P = c.num_tokens * c.top_k, E = c.num_experts;
  const int nch = dispatch_num_chunks(c);
  if (nch == 1) {
    dispatch_single_kernel<<<1, kThreads, 0, s>>>(P, E, capacity, topk_idx, counts, offsets,
                                                  dropped, scatter ? 1 : 0, sorted_pair, pair_pos,
                                                  0, AuxSmallArgs{});
    return hipGetLastError();
  }
  dispatch_hist_kernel<<<nch, kThreads, 0, s>>>(P, E, topk_idx, hist);
  dispatch_scan_kernel<<<1, kThreads, 0, s>>>(nch, E, capacity, hist, scatter ? rank0 : nullptr,
                                              counts, offsets, dropped);
  if (scatter)
    dispatch_scatter_kernel<<<nch, kThreads, 0, s>>>(P, E, capacity, topk_idx, rank0, offsets,
                                                     sorted_pair, pair_pos);
  return hipGetLastError();
}

hipError_t launch_dispatch_aux(const moe_config& c, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               int32_t* hist, int32_t* rank0, int capacity, int32_t* dropped,
                               const AuxSmallArgs& aux, bool* fused, hipStream_t s) {
  *fused = dispatch_num_chunks(c) == 1;
  if (!*fused)
    return launch_dispatch(c, topk_idx, counts, offsets, sorted_pair, pair_pos, hist, rank0, true,
                           capacity, dropped, s);
  // block 1 computes the statistics while block 0 sorts
  dispatch_single_kernel<<<2, kThreads, 0, s>>>(c.num_tokens * c.top_k, c.num_experts, capacity,
                                                topk_idx, counts, offsets, dropped, 1,
                                                sorted_pair, pair_pos, 1, aux);
  return hipGetLastError();
}

hipError_t launch_capacity_fallback(const moe_config& c, const int32_t* topk_idx,
                                    const float* topk_w, int capacity, int fallback_min,
                                    const int32_t* offsets, const int32_t* sorted_pair,
                                    const int32_t* pair_pos, int32_t* idx_out, float* w_out,
                                    int32_t* dropped, bool dropped_zeroed, hipStream_t s) {
  if (dropped && !dropped_zeroed) zero_count_kernel<<<1, 64, 0, s>>>(dropped);
  const int T = c.num_tokens, per = kThreads / 64;
  capacity_fallback_kernel<<<(T + per - 1) / per, kThreads, 0, s>>>(
      T, c.num_experts, c.top_k, capacity, fallback_min, topk_idx, topk_w, offsets, sorted_pair,
      pair_pos, idx_out, w_out, dropped);
  return hipGetLastError();
}

}  // namespace moe
