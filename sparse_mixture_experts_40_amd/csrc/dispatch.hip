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
// one block and one launch, followed (do_aux) by the load-balance statistics
// from these counts, which then need no launch of their own.
// Capacity ([MOE-128x8] 容量因子设计; [QWEN3-ROUTE] §四, tokens taken in order,
// an expert accepts while below its capacity): the pair of rank r inside its
// expert is kept iff r < capacity, i.e. each expert keeps its first
// `capacity` pairs in pair order; a dropped pair gets pair_pos = -1. A
// capacity of 0 keeps every pair. A negative expert id marks an empty slot (a
// token routed to fewer than k experts): it is not a pair and gets
// pair_pos = -1.
// No device-to-host traffic; everything stays on the stream.
#include "aux_small.h"

namespace moe {

namespace {

constexpr int kChunk = 2048;
constexpr int kThreads = 256;

__device__ __forceinline__ int clamp_expert(int v, int E) { return v < 0 ? 0 : (v >= E ? E - 1 : v); }

// LDS histogram of the chunk starting at pair p0 (s_h zeroed by the caller).
__device__ __forceinline__ void hist_chunk(int P, int E, const int32_t* __restrict__ idx, int p0,
                                           int* s_h) {
  for (int i = threadIdx.x; i < kChunk; i += kThreads) {
    const int p = p0 + i;
    if (p < P) {
      const int v = idx[p];
      if (v >= 0) atomicAdd(&s_h[clamp_expert(v, E)], 1);  // v < 0: empty slot
    }
  }
}

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

// Stable scatter of the chunk starting at pair p0. s_rank[e]: rank inside
// expert e of the chunk's first pair of e; s_off[e]: the expert's first
// sorted row; s_wc zeroed; all three visible to the block (caller syncs).
__device__ __forceinline__ void scatter_chunk(int P, int E, int cap,
                                              const int32_t* __restrict__ idx, int p0,
                                              int* s_rank, const int* s_off, int (*s_wc)[256],
                                              int32_t* __restrict__ sorted_pair,
                                              int32_t* __restrict__ pair_pos) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int it = 0; it < kChunk / kThreads; ++it) {
    if (p0 + it * kThreads >= P) break;  // block-uniform: the rest of the chunk is past P
    const int p = p0 + it * kThreads + tid;
    const int raw = p < P ? idx[p] : -1;
    const bool valid = raw >= 0;  // a negative id is an empty slot: no pair
    if (p < P && !valid) pair_pos[p] = -1;
    const int v = valid ? clamp_expert(raw, E) : 0;
    unsigned long long same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (v >> b) & 1;
      const unsigned long long bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wc[wave][v] = __popcll(same);
    __syncthreads();
    if (valid) {
      int r = s_rank[v] + rank;
      for (int w = 0; w < wave; ++w) r += s_wc[w][v];
      if (cap <= 0 || r < cap) {
        const int pos = s_off[v] + r;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
    }
    __syncthreads();
    if (tid < E) {
      s_rank[tid] += s_wc[0][tid] + s_wc[1][tid] + s_wc[2][tid] + s_wc[3][tid];
#pragma unroll
      for (int w = 0; w < 4; ++w) s_wc[w][tid] = 0;
    }
    __syncthreads();
  }
}

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
  scatter_chunk(P, E, cap, idx, blockIdx.x * kChunk, s_rank, s_off, s_wc, sorted_pair, pair_pos);
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
  if (do_aux) aux_small_body(aux, e < E ? tot : 0);  // block-uniform
  if (!scatter) return;                              // block-uniform
  s_off[e] = excl;
  s_h[e] = 0;  // becomes the running rank of each expert
  __syncthreads();
  scatter_chunk(P, E, cap, idx, 0, s_h, s_off, s_wc, sorted_pair, pair_pos);
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
  dispatch_single_kernel<<<1, kThreads, 0, s>>>(c.num_tokens * c.top_k, c.num_experts, capacity,
                                                topk_idx, counts, offsets, dropped, 1,
                                                sorted_pair, pair_pos, 1, aux);
  return hipGetLastError();
}

}  // namespace moe
