// dispatch_chunk.h — one chunk of the stable counting sort of routing pairs.
//
// Replaces the one-hot expert mask and the per-expert torch.where loop of
// [QWEN3-READ] "大模型-qwen3 MoE 详细解读" (cnblogs), forward code, by the token
// permutation of its §三. Used by the dispatch kernels, and by the
// weight-streaming gate/up kernel, whose blocks each sort a one-chunk
// routing (a decode batch) in their own LDS instead of waiting for a
// dispatch launch.
//
// Pair p = t*k + j of expert v = idx[p]; a negative id is an empty slot (no
// pair). Capacity ([MOE-128x8] 容量因子设计; [QWEN3-ROUTE] §四): the pair of
// rank r inside its expert is kept iff cap <= 0 or r < cap.
#pragma once
#include "moe_internal.h"

namespace moe {

constexpr int kDispChunk = 2048;   // pairs per chunk
constexpr int kDispThreads = 256;  // threads of a sorting block

__device__ __forceinline__ int disp_clamp_expert(int v, int E) {
  return v < 0 ? 0 : (v >= E ? E - 1 : v);
}

// LDS histogram of the chunk starting at pair p0 (s_h zeroed by the caller).
__device__ __forceinline__ void hist_chunk(int P, int E, const int32_t* __restrict__ idx, int p0,
                                           int* s_h) {
  for (int i = threadIdx.x; i < kDispChunk; i += kDispThreads) {
    const int p = p0 + i;
    if (p < P) {
      const int v = idx[p];
      if (v >= 0) atomicAdd(&s_h[disp_clamp_expert(v, E)], 1);  // v < 0: empty slot
    }
  }
}

// Stable scatter of the chunk starting at pair p0: pairs walk in ascending
// order, 256 at a time; a lane's rank among equal experts comes from 8
// ballots (one per bit of the expert id), wave counts go through LDS, so the
// pairs of an expert land in ascending pair order. s_rank[e]: rank inside
// expert e of the chunk's first pair of e; s_off[e]: the expert's first
// sorted row; s_wc zeroed; all three visible to the block (caller syncs).
// emit(p, pos) places kept pair p at sorted row pos; drop(p) marks a pair
// past the capacity or an empty slot.
template <class Emit, class Drop>
__device__ __forceinline__ void scatter_chunk(int P, int E, int cap,
                                              const int32_t* __restrict__ idx, int p0,
                                              int* s_rank, const int* s_off, int (*s_wc)[256],
                                              Emit emit, Drop drop) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int it = 0; it < kDispChunk / kDispThreads; ++it) {
    if (p0 + it * kDispThreads >= P) break;  // block-uniform: the rest of the chunk is past P
    const int p = p0 + it * kDispThreads + tid;
    const int raw = p < P ? idx[p] : -1;
    const bool valid = raw >= 0;  // a negative id is an empty slot: no pair
    if (p < P && !valid) drop(p);
    const int v = valid ? disp_clamp_expert(raw, E) : 0;
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
      if (cap <= 0 || r < cap)
        emit(p, s_off[v] + r);
      else
        drop(p);
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

// LDS of a one-chunk sort in one block.
struct DispLds {
  int h[256];      // histogram, then the running rank of each expert
  int c[256];      // inclusive scan of the kept counts
  int off[256];    // first sorted row of each expert
  int wc[4][256];  // per-wave counts of one scatter round
  int drop;        // pairs past the capacity
};

// First half of a one-chunk sort (P <= kDispChunk; a whole block of 256
// threads, E <= 256): histogram, kept counts min(total, cap), their exclusive
// scan. Returns thread e's total (0 for e >= E); on return L.off[e] is the
// first sorted row of expert e, L.c[255] the number of kept pairs, L.drop the
// pairs past the capacity, L.h and L.wc zeroed for the scatter.
__device__ __forceinline__ int disp_counts(int P, int E, int cap, const int32_t* __restrict__ idx,
                                           DispLds& L) {
  const int e = threadIdx.x;
  L.h[e] = 0;
  if (e == 0) L.drop = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) L.wc[w][e] = 0;
  __syncthreads();
  hist_chunk(P, E, idx, 0, L.h);
  __syncthreads();
  const int tot = e < E ? L.h[e] : 0;
  const int kept = (cap > 0 && tot > cap) ? cap : tot;
  L.c[e] = kept;
  __syncthreads();
  if (kept < tot) atomicAdd(&L.drop, tot - kept);  // integer: exact, order-free
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan over the 256 slots
    const int add = (e >= d) ? L.c[e - d] : 0;
    __syncthreads();
    L.c[e] += add;
    __syncthreads();
  }
  L.off[e] = L.c[e] - kept;
  L.h[e] = 0;  // becomes the running rank of each expert
  __syncthreads();
  return tot;
}

}  // namespace moe
