// aux_small.h — load-balance statistics of few router blocks in one block.
//
// [MOE-128x8] "MoE架构深度解析：128专家与8激活的智能路由" (csdn), load-balancing
// section: f_e = n_e / (T*k), P_e = mean softmax probability,
// aux = E * sum_e f_e P_e; the z-loss mean of (ln sum_e exp l)^2.
// Shared by the aux kernel and the one-block dispatch, which runs it after
// its counts when the layer forward asks for statistics (one launch fewer).
#pragma once
#include "moe_internal.h"

namespace moe {

constexpr int kAuxSmall = 64;  // most router blocks whose partials one block reduces

struct AuxSmallArgs {
  int T, E, want_stats;
  const float* partials;  // [np][E] per router block sums of the softmax probabilities
  int np;
  int32_t* c_out;
  float* f_out;
  float* p_out;
  const float* zpart;  // [nz] per router block sums of (ln sum_e exp l)^2, or null
  int nz;
  float* aux_out;
  float* z_out;
};

// Whole block of exactly 256 threads, E <= 256, np <= kAuxSmall. Thread e
// holds n = n_e (0 for e >= E) and sums expert e's partials in block order
// (fixed order, double); f_e divides by the sum of the counts (an integer LDS
// sum: T*k unless slots are empty); aux and z are fixed-shape tree sums.
__device__ __forceinline__ void aux_small_body(const AuxSmallArgs& a, int n) {
  constexpr int NT = 256;
  __shared__ double s[NT];
  __shared__ int s_routed;
  const int e = threadIdx.x;
  const bool mine = a.want_stats && e < a.E;
  if (e == 0) s_routed = 0;
  __syncthreads();
  if (mine) atomicAdd(&s_routed, n);  // integer: exact, order-free
  double acc = 0.0;
  if (mine) {
    // unconditional loads (row index clamped into [0, np)), so that all of
    // them are in flight together; only rows b < np are added, in order
    float r[kAuxSmall];
#pragma unroll
    for (int b = 0; b < kAuxSmall; ++b) r[b] = a.partials[(size_t)min(b, a.np - 1) * a.E + e];
#pragma unroll
    for (int b = 0; b < kAuxSmall; ++b) acc += b < a.np ? (double)r[b] : 0.0;
  }
  __syncthreads();
  double fp = 0.0;
  if (mine) {
    const double f = s_routed > 0 ? (double)n / (double)s_routed : 0.0;
    const double P = acc / (double)a.T;
    if (a.c_out) a.c_out[e] = n;
    if (a.f_out) a.f_out[e] = (float)f;
    if (a.p_out) a.p_out[e] = (float)P;
    fp = f * P;
  }
  if (a.aux_out) {
    s[e] = fp;
    __syncthreads();
    for (int d = NT / 2; d > 0; d >>= 1) {
      if (e < d) s[e] += s[e + d];
      __syncthreads();
    }
    if (e == 0) a.aux_out[0] = (float)((double)a.E * s[0]);
    __syncthreads();
  }
  if (a.z_out) {
    double z = 0.0;
    for (int b = e; b < a.nz; b += NT) z += (double)a.zpart[b];
    s[e] = z;
    __syncthreads();
    for (int d = NT / 2; d > 0; d >>= 1) {
      if (e < d) s[e] += s[e + d];
      __syncthreads();
    }
    if (e == 0) a.z_out[0] = (float)(s[0] / (double)a.T);
  }
}

// Host: the statistics of `out` from n_partials router blocks fit one block
// (then launch_dispatch_aux may produce them with a one-chunk dispatch).
bool aux_small_fits(const moe_config& c, int n_partials);
AuxSmallArgs aux_small_args(const moe_config& c, const float* prob_partials, int n_partials,
                            const AuxOut& out, const float* zpart, int n_zpart);

// launch_dispatch, and for a one-chunk dispatch the statistics in the same
// block (*fused = true); otherwise only the dispatch (*fused = false).
hipError_t launch_dispatch_aux(const moe_config& c, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               int32_t* hist, int32_t* rank0, int capacity, int32_t* dropped,
                               const AuxSmallArgs& aux, bool* fused, hipStream_t s);

// Decode-sized bf16 gate/up of a one-chunk routing with the dispatch inside
// it (gate_up_sorts_itself): each block of the weight-streaming kernel sorts
// topk_idx in its LDS like the one-chunk dispatch (same capacity rule);
// block 0 writes counts (nullable), offsets, sorted_pair, pair_pos and
// *dropped (nullable), block 1 the statistics *aux (nullable: none).
bool gate_up_sorts_itself(const moe_config& c);
hipError_t launch_gate_up_sorting(const moe_config& c, const void* x, const int32_t* topk_idx,
                                  int capacity, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_pair, int32_t* pair_pos, int32_t* dropped,
                                  const AuxSmallArgs* aux, const void* w_gate, const void* w_up,
                                  void* h, hipStream_t s);

}  // namespace moe
