// router.hip — router linear + fp32 softmax + wavefront top-k + weights.
//
// [QWEN3-READ] "大模型-qwen3 MoE 详细解读" (cnblogs), forward code: gate linear
// without bias, softmax over the experts in fp32, top-k, and (Qwen3 only)
// division of the k weights by their sum. [LAB17] 第二阶段 实现流程 steps 1-3.
//
// One block of 256 threads (4 wave64) owns 64 tokens (fewer when it starts
// from given or split-K partial logits and T is small):
//  1. logits tile [64 tokens x E] — bf16: MFMA 32x32x16 with the router rows
//     as the A operand and the tokens as B, K staged through swizzled LDS;
//     fp32: plain FMA dot products. (x == nullptr: the tile is read, or
//     summed from split-K partials.)
//  2. four lanes per token (each wave takes up to 16 tokens): lane part q
//     holds experts e = 4j + q. Softmax max and sum: over the lane's experts,
//     then over the four lanes (two DPP exchanges; a + b == b + a, so all four
//     lanes hold the same bits). Top-k: each lane keeps its k best experts in
//     registers, sorted, inserting its experts in ascending index order with a
//     strict greater-than (an equal logit never displaces an earlier, lower
//     index); then two bitonic merges with the partner lanes (xor 1, xor 2)
//     under the total order (logit descending, index ascending) leave the
//     token's k best in every one of its lanes. Plain fp32 compares, so
//     -0.0 == +0.0. No cross-lane dependency chain runs through the k
//     selections (the former k rounds of a wave-wide max did).
//  3. per-block sums of the full softmax over the block's tokens (fixed
//     token order) for the load-balance statistic P_e, and of
//     (ln sum_e exp l)^2 for the router z-loss.
// Variants: noisy logits l + n * softplus(x W_noise) ([MOE-128x8] router
// pseudocode, [LAB17] noisy top-k gating; the noise logits are a second
// logits pass, the noise values an input) are formed when the logits are read;
// a selection-only bias ([LAB17], DeepSeek-V3 balancing without an auxiliary
// loss) is added to the top-k keys only, the weights use the unbiased logits;
// entropy-driven k ([QWEN3-ROUTE] §二 dynamic TopK) keeps the first k_t slots
// and marks the others empty (-1, weight 0).
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {

constexpr int kTok = 64;       // tokens per block

// Row stride (floats) of the block's logits in LDS: = LPT (mod 64), so the
// LPT lanes of each of a wave's 64 / LPT tokens (experts LPT j + q of row t)
// read 64 different banks.
__host__ __device__ constexpr int router_ls(int E, int lpt) { return ((E + 63) & ~63) + lpt; }
constexpr int kThreads = 256;  // 4 waves
constexpr int kBK = 64;        // K step (elements)

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0.0 -> +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Reductions over the 64 lanes of N tokens at once (independent chains).
// Wave-wide reductions whose result every lane receives. Inside each row of
// 16 lanes four DPP exchanges (xor 1, xor 2, mirror within 8, mirror within
// 16) combine all 16 values without LDS traffic; the four row results are
// then read with readlane and combined in row order 0..3.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int N>
__device__ __forceinline__ void wave_max_n(float (&v)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    float x = v[u];
    x = fmaxf(x, dpp_f32<kDppXor1>(x));
    x = fmaxf(x, dpp_f32<kDppXor2>(x));
    x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppMirror>(x));
    v[u] = fmaxf(fmaxf(lane_f32(x, 0), lane_f32(x, 16)), fmaxf(lane_f32(x, 32), lane_f32(x, 48)));
  }
}

template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    float x = v[u];
    x += dpp_f32<kDppXor1>(x);
    x += dpp_f32<kDppXor2>(x);
    x += dpp_f32<kDppHalfMirror>(x);
    x += dpp_f32<kDppMirror>(x);
    v[u] = ((lane_f32(x, 0) + lane_f32(x, 16)) + lane_f32(x, 32)) + lane_f32(x, 48);
  }
}

template <int N>
__device__ __forceinline__ void wave_max_u64_n(unsigned long long (&v)[N]) {
  auto step = [](unsigned long long x, auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const unsigned long long o =
        (static_cast<unsigned long long>(dpp_u32<C>((uint32_t)(x >> 32))) << 32) |
        dpp_u32<C>((uint32_t)x);
    return o > x ? o : x;
  };
  auto lane64 = [](unsigned long long x, int l) {
    return (static_cast<unsigned long long>(
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l)) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  };
#pragma unroll
  for (int u = 0; u < N; ++u) {
    unsigned long long x = v[u];
    x = step(x, std::integral_constant<int, kDppXor1>{});
    x = step(x, std::integral_constant<int, kDppXor2>{});
    x = step(x, std::integral_constant<int, kDppHalfMirror>{});
    x = step(x, std::integral_constant<int, kDppMirror>{});
    const unsigned long long a = lane64(x, 0), b = lane64(x, 16), c = lane64(x, 32),
                             d = lane64(x, 48);
    const unsigned long long ab = a > b ? a : b, cd = c > d ? c : d;
    v[u] = ab > cd ? ab : cd;
  }
}

// swizzled [rows][64] bf16 tile: 16-byte chunk c of row r lives at chunk c ^ (r & 7)
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

// Router rows of one K stage in LDS: the power of two (times 32) at or above
// E rounded to 32, so that each of the 4 waves issues the same number of
// 8-row LDS-DMA loads.
__host__ __device__ constexpr int router_wrows(int E) {
  return (E + 31) / 32 <= 1 ? 32 : (E + 31) / 32 <= 2 ? 64 : (E + 31) / 32 <= 4 ? 128 : 256;
}
constexpr int kStages = 3;  // LDS stages of the logits pipeline
// LDS bytes of the logits pipeline: kStages x ([64] token rows + router rows) x 64
__host__ __device__ constexpr size_t router_tile_lds(int E) {
  return (size_t)kStages * (kTok + router_wrows(E)) * kBK * sizeof(uint16_t);
}

// One K step of the logits tile: issue the LDS-DMA loads of a later stage
// into dst (if issue), then the MFMAs of the stage in src. dst and src are
// distinct __restrict__ pointers, so the compiler gives the DMA writes and
// the fragment reads disjoint alias scopes and does not drain the loads in
// flight before every fragment read; wait_vmcnt + lds_barrier order them.
// Each DMA instruction fills 8 consecutive tile rows (lane l: row l / 8,
// slot l % 8); the lane's source chunk is (l % 8) ^ (l / 8), which is the
// swz layout. Waves own x row groups 2w, 2w + 1 and router row groups
// NW w .. NW w + NW - 1.
template <int NQ, int NW>
__device__ __forceinline__ void router_step(uint16_t* __restrict__ dst,
                                            const uint16_t* __restrict__ src, bool issue,
                                            __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                            const uint32_t (&xo)[2], const uint32_t (&wo)[NW],
                                            uint32_t kb, f32x16_t (&acc)[NQ > 0 ? NQ : 1],
                                            int wave, int lane) {
  if (issue) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + (2 * wave + i) * 8 * kBK),
                                               16, xo[i], kb, 0, 0);
#pragma unroll
    for (int i = 0; i < NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_void_t*)(dst + (kTok + (NW * wave + i) * 8) * kBK), 16, wo[i], kb, 0, 0);
  }
  // all fragments of the stage first (the token block, wave & 1, is the same
  // for every tile of the wave), then the MFMAs: the reads' latency overlaps
  // the MFMA pipe instead of stalling each MFMA on its own reads
  if constexpr (NQ > 0) {
    constexpr int KK = kBK / 16;
    const uint16_t* s_w = src + kTok * kBK;
    const int tr = (wave & 1) * 32 + (lane & 31);
    bf16x8_t fb[KK], fa[KK][NQ];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      fb[kk] = *reinterpret_cast<const bf16x8_t*>(src + swz(tr, ch));
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int er = (q * 2 + (wave >> 1)) * 32 + (lane & 31);  // expert block (q 4 + wave) / 2
        fa[kk][q] = *reinterpret_cast<const bf16x8_t*>(s_w + swz(er, ch));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][q], fb[kk], acc[q], 0, 0, 0);
  }
}

// Logits tile by bf16 MFMA into s_log[t * ls + e] (+ bias): tokens t0 ..
// t0 + 63 over K range [kbeg, kend), through a kStages LDS ring filled by
// LDS-DMA (no register staging, no LDS store instructions), one wait and one
// barrier per K step. A stage buffer is refilled two steps after it was read,
// and every wave has passed the barrier between. Rows past T and past E are
// clamped to valid rows on load and never stored. Needs T H and E H below
// 2^31 elements (32-bit buffer offsets).
__device__ __forceinline__ void router_logits_mfma(int T, int H, int E, int t0, int kbeg, int kend,
                                   const uint16_t* __restrict__ x,
                                   const uint16_t* __restrict__ wr, const float* __restrict__ bias,
                                   char* smem, float* s_log, int ls) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int EP = (E + 31) & ~31;
  uint16_t* s_ring = reinterpret_cast<uint16_t*>(smem);
  const int ntiles = (EP / 32) * 2;                     // (expert block, token block)

  // tiles of this wave: (expert block, token block) q * 4 + wave for q < nq
  const int nq = ntiles > wave ? (ntiles - wave + 3) / 4 : 0;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0,
                                        (int)((uint32_t)T * (uint32_t)H * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wr), (short)0,
                                        (int)((uint32_t)E * (uint32_t)H * 2u), 0x00020000);
  const int r_in = lane >> 3, chunk = (lane & 7) ^ r_in;

  auto kloop = [&](auto nq_c, auto nw_c) __attribute__((always_inline)) {
    constexpr int NQ = decltype(nq_c)::value;
    constexpr int NW = decltype(nw_c)::value;
    constexpr int NL = 2 + NW;  // DMA loads per wave and stage
    const int stage_elems = (kTok + 32 * NW) * kBK;
    uint32_t xo[2], wo[NW];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = t0 + (2 * wave + i) * 8 + r_in;
      xo[i] = (uint32_t)(r < T ? r : T - 1) * (uint32_t)H * 2u + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int r = (NW * wave + i) * 8 + r_in;
      wo[i] = (uint32_t)(r < E ? r : E - 1) * (uint32_t)H * 2u + chunk * 16;
    }
    f32x16_t acc[NQ > 0 ? NQ : 1];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    const int nk = (kend - kbeg) / kBK;
    // prologue: stages 0 and 1 in flight (no MFMAs)
    f32x16_t none[1];
    router_step<0, NW>(s_ring, s_ring, nk > 0, rx, rw, xo, wo, (uint32_t)kbeg * 2u, none, wave,
                       lane);
    router_step<0, NW>(s_ring + stage_elems, s_ring, nk > 1, rx, rw, xo, wo,
                       (uint32_t)(kbeg + kBK) * 2u, none, wave, lane);
    int cur = 0;  // ring buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk)
        wait_vmcnt(NL);  // stage kt landed; stage kt + 1 may still be in flight
      else
        wait_vmcnt(0);
      lds_barrier();
      const int nxt = cur == 0 ? 2 : cur - 1;  // (kt + 2) mod kStages
      router_step<NQ, NW>(s_ring + nxt * stage_elems, s_ring + cur * stage_elems, kt + 2 < nk,
                          rx, rw, xo, wo, (uint32_t)(kbeg + (kt + 2) * kBK) * 2u, acc, wave,
                          lane);
      cur = cur == 2 ? 0 : cur + 1;
    }
    __syncthreads();  // ring dead; s_log aliases it
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int tile = q * 4 + wave;
      const int eb = tile >> 1, tb = tile & 1;
      const int t = tb * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = eb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (e < E) s_log[t * ls + e] = acc[q][r] + (bias ? bias[e] : 0.0f);
      }
    }
  };
  auto by_nq = [&](auto nw_c) __attribute__((always_inline)) {
    switch (nq) {  // wave-uniform
      case 0: kloop(std::integral_constant<int, 0>{}, nw_c); break;
      case 1: kloop(std::integral_constant<int, 1>{}, nw_c); break;
      case 2: kloop(std::integral_constant<int, 2>{}, nw_c); break;
      case 3: kloop(std::integral_constant<int, 3>{}, nw_c); break;
      default: kloop(std::integral_constant<int, 4>{}, nw_c); break;
    }
  };
  switch (router_wrows(E)) {
    case 32: by_nq(std::integral_constant<int, 1>{}); break;
    case 64: by_nq(std::integral_constant<int, 2>{}); break;
    case 128: by_nq(std::integral_constant<int, 4>{}); break;
    default: by_nq(std::integral_constant<int, 8>{}); break;
  }
}

// A value of the aligned M-lane group next to this lane's (inside the
// aligned 2M-lane group): lane ^ 1 and lane ^ 2 by DPP quad permutes; for
// M = 4 and 8 the mirrored lane inside 8 or 16 lanes (DPP row half mirror,
// row mirror), which lies in the other group; for 16 and 32 lane ^ M, by the
// gfx950 permlane swaps (v_permlane16_swap: odd rows receive the even row's
// values in the first result, even rows the odd row's in the second; likewise
// for halves with v_permlane32_swap). Used where every lane of each M-lane
// group holds the same value, so which lane of the other group answers does
// not matter.
template <int M>
__device__ __forceinline__ uint32_t xchg_u32(uint32_t v) {
  if constexpr (M == 1) return dpp_u32<kDppXor1>(v);
  else if constexpr (M == 2) return dpp_u32<kDppXor2>(v);
  else if constexpr (M == 4) return dpp_u32<kDppHalfMirror>(v);
  else if constexpr (M == 8) return dpp_u32<kDppMirror>(v);
  else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "group size");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int M>
__device__ __forceinline__ float xchg_f32(float v) {
  return __uint_as_float(xchg_u32<M>(__float_as_uint(v)));
}

// Max and sum over the L lanes of a token (aligned groups of L lanes),
// butterflies over xchg_u32: after each step every lane of the group formed
// so far holds the same bits (a + b == b + a).
template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, xchg_f32<1>(v));
  if constexpr (L >= 4) v = fmaxf(v, xchg_f32<2>(v));
  if constexpr (L >= 8) v = fmaxf(v, xchg_f32<4>(v));
  if constexpr (L >= 16) v = fmaxf(v, xchg_f32<8>(v));
  if constexpr (L >= 32) v = fmaxf(v, xchg_f32<16>(v));
  if constexpr (L >= 64) v = fmaxf(v, xchg_f32<32>(v));
  return v;
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += xchg_f32<1>(v);
  if constexpr (L >= 4) v += xchg_f32<2>(v);
  if constexpr (L >= 8) v += xchg_f32<4>(v);
  if constexpr (L >= 16) v += xchg_f32<8>(v);
  if constexpr (L >= 32) v += xchg_f32<16>(v);
  if constexpr (L >= 64) v += xchg_f32<32>(v);
  return v;
}

// Total order of the top-k: larger key first, equal keys by lower index.
__device__ __forceinline__ bool topk_better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Bitonic merge of this lane's sorted (descending) list with the one of the
// neighbouring M-lane group (xchg_u32; the lanes of each group hold the same
// list): the best KM of both, sorted, in every lane of both groups.
template <int KM, int M>
__device__ __forceinline__ void topk_merge(float (&tv)[KM], int (&ti)[KM]) {
  float bv[KM];
  int bi[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    bv[s] = xchg_f32<M>(tv[s]);
    bi[s] = (int)xchg_u32<M>((uint32_t)ti[s]);
  }
  // the better of a[s] and b[KM-1-s]: the KM best, as a bitonic sequence
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    const float ob = bv[KM - 1 - s];
    const int oi = bi[KM - 1 - s];
    if (!topk_better(tv[s], ti[s], ob, oi)) {
      tv[s] = ob;
      ti[s] = oi;
    }
  }
  // bitonic sorter, descending
#pragma unroll
  for (int d = KM / 2; d > 0; d >>= 1)
#pragma unroll
    for (int s = 0; s < KM; ++s)
      if ((s & d) == 0) {
        const int u = s + d;
        if (topk_better(tv[u], ti[u], tv[s], ti[s])) {
          const float fv = tv[s];
          const int fi = ti[s];
          tv[s] = tv[u];
          ti[s] = ti[u];
          tv[u] = fv;
          ti[u] = fi;
        }
      }
}

// All merges of an L-lane token group.
template <int KM, int L>
__device__ __forceinline__ void topk_merge_group(float (&tv)[KM], int (&ti)[KM]) {
  if constexpr (L >= 2) topk_merge<KM, 1>(tv, ti);
  if constexpr (L >= 4) topk_merge<KM, 2>(tv, ti);
  if constexpr (L >= 8) topk_merge<KM, 4>(tv, ti);
  if constexpr (L >= 16) topk_merge<KM, 8>(tv, ti);
  if constexpr (L >= 32) topk_merge<KM, 16>(tv, ti);
  if constexpr (L >= 64) topk_merge<KM, 32>(tv, ti);
}

// KM: the top-k list length, a power of two >= k (1 <= k <= 16).
// LPT: lanes per token (4, 16 or 64): 256 / tokens per block.
template <bool BF16, int KM, int LPT>
__global__ __launch_bounds__(kThreads) void router_kernel(
    int T, int H, int E, int k, int norm, const void* __restrict__ x, const void* __restrict__ wr,
    const float* __restrict__ bias, const float* __restrict__ logits_in, float* __restrict__ logits_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ partials,
    int do_select, int tpb, const float* __restrict__ noise, const float* __restrict__ nlogits,
    const float* __restrict__ sel_bias, float* __restrict__ zpart, int k_min,
    int32_t* __restrict__ kt_out, const float* __restrict__ part, int nsplit) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * tpb;  // tpb = 64 when the logits are computed here
  const int ls = router_ls(E, LPT);
  float* s_log = reinterpret_cast<float*>(smem);  // [64][ls]

  if (part) {  // split-K partial logits: sum in split order, then the bias
    // The loads of 16 splits are issued before the first add (one memory
    // round trip per 16 splits instead of one per split); the adds keep the
    // split order.
    const size_t stride = (size_t)T * E;
    for (int i = tid; i < tpb * E; i += kThreads) {
      const int t = i / E, e = i - t * E;
      float l = 0.0f;
      if (t0 + t < T) {
        const float* p = part + (size_t)(t0 + t) * E + e;
        int ks = 0;
        for (; ks + 16 <= nsplit; ks += 16) {
          float r[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) r[j] = p[(size_t)(ks + j) * stride];
#pragma unroll
          for (int j = 0; j < 16; ++j) l += r[j];
        }
        for (; ks < nsplit; ++ks) l += p[(size_t)ks * stride];
        if (bias) l += bias[e];
      }
      s_log[t * ls + e] = l;
    }
  } else if (logits_in) {
    for (int i = tid; i < tpb * E; i += kThreads) {
      const int t = i / E, e = i - t * E;
      float l = 0.0f;
      if (t0 + t < T) {
        const size_t g = (size_t)(t0 + t) * E + e;
        l = logits_in[g];
        if (noise) {  // l + n * softplus(nl), softplus(z) = ln(1 + e^z)
          const float z = nlogits[g];
          const float sp = z > 0.0f ? z + log1pf(expf(-z)) : log1pf(expf(z));
          l = fmaf(noise[g], sp, l);
        }
      }
      s_log[t * ls + e] = l;
    }
  } else if constexpr (BF16 && LPT == 4) {  // logits computed here: 64-token blocks
    router_logits_mfma(T, H, E, t0, 0, H, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(wr), bias, smem, s_log, ls);
  } else if constexpr (!BF16 && LPT == 4) {
    const float* xf = static_cast<const float*>(x);
    const float* wf = static_cast<const float*>(wr);
    for (int i = tid; i < kTok * E; i += kThreads) {
      const int t = i / E, e = i - t * E;
      float s = 0.0f;
      if (t0 + t < T) {
        for (int h = 0; h < H; ++h) s = fmaf(xf[(size_t)(t0 + t) * H + h], wf[(size_t)e * H + h], s);
        if (bias) s += bias[e];
      }
      s_log[t * ls + e] = s;
    }
  }
  __syncthreads();

  // the logits the softmax uses, written out coalesced from LDS
  if (logits_out)
    for (int i = tid; i < tpb * E; i += kThreads) {
      const int t = i / E, e = i - t * E;
      if (t0 + t < T) logits_out[(size_t)(t0 + t) * E + e] = s_log[t * ls + e];
    }

  // LPT lanes per token: token slot tl of this wave, part q
  constexpr int TPW = 64 / LPT;                  // token slots per wave
  const int q = lane & (LPT - 1), tl = lane / LPT;
  const int tpw = tpb / 4;                       // tokens of this wave (<= TPW)
  const int tb = wave * tpw + (tl < tpw ? tl : tpw - 1);  // its row in s_log
  const bool ok = tl < tpw && t0 + tb < T;       // a real token of this lane
  const float* row = s_log + tb * ls;
  const int EQ = (E + LPT - 1) / LPT;            // experts per lane (e = LPT j + q)
  static_assert(TPW * LPT == 64, "lanes per token");

  float m = -INFINITY;
  for (int j = 0; j < EQ; ++j) {
    const int e = LPT * j + q;
    if (e < E) m = fmaxf(m, row[e]);
  }
  m = group_max<LPT>(m);
  float ssum = 0.0f;
  for (int j = 0; j < EQ; ++j) {
    const int e = LPT * j + q;
    if (e < E) ssum += expf(row[e] - m);
  }
  ssum = group_sum<LPT>(ssum);
  const float inv = 1.0f / ssum;

  // entropy-driven number of experts ([QWEN3-ROUTE] §二 dynamic TopK):
  // k_t = clamp(floor(k_min + (k - k_min) H_t / ln E)), H_t = -sum p ln max(p, 1e-10)
  int kt = k;
  if (k_min > 0) {
    float hs = 0.0f;
    for (int j = 0; j < EQ; ++j) {
      const int e = LPT * j + q;
      if (e < E) {
        const float pe = expf(row[e] - m) * inv;
        hs = fmaf(pe, logf(fmaxf(pe, 1e-10f)), hs);
      }
    }
    hs = group_sum<LPT>(hs);
    const float span = (float)(k - k_min) / logf((float)E);
    const int kk = (int)floorf(fmaf(-hs, span, (float)k_min));
    kt = kk < k_min ? k_min : (kk > k ? k : kk);
    if (kt_out && ok && q == 0) kt_out[t0 + tb] = kt;
  }

  if (do_select) {
    float tv[KM];
    int ti[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      tv[s] = -INFINITY;
      ti[s] = 0x7FFF;
    }
    for (int j = 0; j < EQ; ++j) {
      const int e = LPT * j + q;
      if (e >= E) break;
      const float c = sel_bias ? row[e] + sel_bias[e] : row[e];
      // sorted insertion, strict: c goes below every entry it does not beat
#pragma unroll
      for (int s = KM - 1; s >= 0; --s) {
        const bool gt = c > tv[s];
        const bool gtp = s > 0 ? c > tv[s > 0 ? s - 1 : 0] : false;
        const float pv = tv[s > 0 ? s - 1 : 0];
        const int pi = ti[s > 0 ? s - 1 : 0];
        tv[s] = gt ? (gtp ? pv : c) : tv[s];
        ti[s] = gt ? (gtp ? pi : e) : ti[s];
      }
    }
    topk_merge_group<KM, LPT>(tv, ti);
    // weights from the unbiased logits: p_j = e^(l_j - m) / s, renormalised
    // over the first k_t slots iff norm; slots past k_t are empty
    float pj[KM], psum = 0.0f;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      const float lj = sel_bias ? row[ti[s] < E ? ti[s] : 0] : tv[s];
      pj[s] = expf(lj - m) * inv;
      if (s < kt) psum += pj[s];
    }
    if (ok) {
      const size_t o = (size_t)(t0 + tb) * k;
#pragma unroll
      for (int s = 0; s < KM; ++s)
        if (s < k && (s & (LPT - 1)) == q) {
          const bool live = s < kt;
          topk_idx[o + s] = live ? ti[s] : -1;
          topk_w[o + s] = live ? (norm ? pj[s] / psum : pj[s]) : 0.0f;
        }
    }
  }

  // statistics: per token (ln s)^2 + m-shifted, and the full softmax written
  // back over the block's logits; then fixed-order sums over the tokens
  __shared__ float s_z[kTok];
  if (zpart && q == 0 && tl < tpw) {
    const float lse = m + logf(ssum);
    s_z[tb] = ok ? lse * lse : 0.0f;
  }
  if (partials) {
    __syncthreads();  // every lane's top-k reads of its row are done
    if (tl < tpw)
      for (int j = 0; j < EQ; ++j) {
        const int e = LPT * j + q;
        if (e < E) s_log[tb * ls + e] = ok ? expf(row[e] - m) * inv : 0.0f;
      }
  }
  if (zpart || partials) __syncthreads();
  if (zpart && tid == 0) {
    float z = 0.0f;
    for (int t = 0; t < tpb; ++t) z += s_z[t];  // token order
    zpart[blockIdx.x] = z;
  }
  if (partials)
    for (int e = tid; e < E; e += kThreads) {
      float a = 0.0f;
      for (int t = 0; t < tpb; ++t) a += s_log[t * ls + e];  // token order
      partials[(size_t)blockIdx.x * E + e] = a;
    }
}

// Split-K router logits for small token counts (a single 64-token block
// would stream the whole router matrix through one CU): block (tile, ks)
// computes the partial logits of its 64 tokens over K range ks, written to
// part[ks][t][e]. The top-k pass (router_kernel) sums the partials in ks order
// and adds the bias as it reads them; router_reduce_kernel does the same sum
// where only the logits are wanted.
__global__ __launch_bounds__(kThreads) void router_partial_kernel(
    int T, int H, int E, int kchunk, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, float* __restrict__ part) {
  extern __shared__ __align__(16) char smem[];
  const int t0 = blockIdx.x * kTok, ks = blockIdx.y;
  const int ls = ((E + 31) & ~31) + 1;
  float* s_log = reinterpret_cast<float*>(smem);
  router_logits_mfma(T, H, E, t0, ks * kchunk, ks * kchunk + kchunk, x, wr, nullptr, smem, s_log,
                     ls);
  __syncthreads();
  for (int i = threadIdx.x; i < kTok * E; i += kThreads) {
    const int t = i / E, e = i - t * E;
    if (t0 + t < T) part[((size_t)ks * T + t0 + t) * E + e] = s_log[t * ls + e];
  }
}

__global__ __launch_bounds__(kThreads) void router_reduce_kernel(int T, int E, int nsplit,
                                                                 const float* __restrict__ part,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ logits,
                                                                 float* __restrict__ logits_out) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= T * E) return;
  float s = 0.0f;
  const size_t stride = (size_t)T * E;
  int ks = 0;
  for (; ks + 16 <= nsplit; ks += 16) {  // 16 loads in flight, adds in split order
    float r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = part[(size_t)(ks + j) * stride + i];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += r[j];
  }
  for (; ks < nsplit; ++ks) s += part[(size_t)ks * stride + i];
  if (bias) s += bias[i % E];
  logits[i] = s;
  if (logits_out) logits_out[i] = s;
}

// Small-T router logits in one launch, without split-K partials (a decode
// batch): block (tg, eg) computes tokens [4 tg, 4 tg + 4) x 4 kRlEpw experts,
// wave w the kRlEpw experts from (4 eg + w) kRlEpw on. Lane l holds the K
// elements (64 c + l) 8 .. + 7 for c < H / 512, so each load instruction
// reads 1 KB of consecutive elements; it sums them in c order with fp32 FMA,
// the wave adds its lanes by a fixed butterfly (deterministic), then the
// bias is added. H % 512 == 0.
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
    acc = fmaf(__uint_as_float(av[i] & 0xFFFF0000u), __uint_as_float(bv[i] & 0xFFFF0000u), acc);
  }
  return acc;
}

#ifndef MOE_RL_EPW
#define MOE_RL_EPW 1
#endif
constexpr int kRlEpw = MOE_RL_EPW;  // experts per wave

__global__ __launch_bounds__(kThreads) void router_logits_direct_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 4, e0 = blockIdx.y * (4 * kRlEpw) + wave * kRlEpw;
  const uint16_t* xr[4];
  const uint16_t* wrow[kRlEpw];
#pragma unroll
  for (int i = 0; i < 4; ++i) xr[i] = x + (size_t)min(t0 + i, T - 1) * H;
#pragma unroll
  for (int j = 0; j < kRlEpw; ++j) wrow[j] = wr + (size_t)min(e0 + j, E - 1) * H;
  float acc[4][kRlEpw];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kRlEpw; ++j) acc[i][j] = 0.0f;
  const int nc = H / 512;
#pragma unroll 4
  for (int c = 0; c < nc; ++c) {
    const int off = (c * 64 + lane) * 8;
    uint4 xv[4], wv[kRlEpw];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const uint4*>(xr[i] + off);
#pragma unroll
    for (int j = 0; j < kRlEpw; ++j) wv[j] = *reinterpret_cast<const uint4*>(wrow[j] + off);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kRlEpw; ++j) acc[i][j] = dot8_bf16(xv[i], wv[j], acc[i][j]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kRlEpw; ++j) acc[i][j] += __shfl_xor(acc[i][j], d);
  if (lane < 4 * kRlEpw) {  // lane kRlEpw i + j writes (token t0 + i, expert e0 + j)
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kRlEpw; ++j)
        if (lane == kRlEpw * i + j) v = acc[i][j];
    const int t = t0 + lane / kRlEpw, e = e0 + lane % kRlEpw;
    if (t < T && e < E) out[(size_t)t * E + e] = bias ? v + bias[e] : v;
  }
}

}  // namespace

// Small-T logits in one launch (router_logits_direct_kernel) instead of
// split-K partials and their sum: decode batches (T <= 256). Larger split
// grids keep the MFMA partials, since every expert group of the direct
// kernel reads all of x again.
static bool router_direct(const moe_config& c) {
  return c.dtype == MOE_DTYPE_BF16 && c.hidden % 512 == 0 && c.num_tokens <= 256;
}

static void launch_logits_direct(const moe_config& c, const void* x, const void* w,
                                 const float* bias, float* out, hipStream_t s) {
  const dim3 grid((c.num_tokens + 3) / 4, (c.num_experts + 4 * kRlEpw - 1) / (4 * kRlEpw));
  router_logits_direct_kernel<<<grid, kThreads, 0, s>>>(c.num_tokens, c.hidden, c.num_experts,
                                                        static_cast<const uint16_t*>(x),
                                                        static_cast<const uint16_t*>(w), bias,
                                                        out);
}

// Tokens per router block: 64 when the block computes its logits (one MFMA
// tile); fewer when it starts from logits and T is small, so that the tokens
// spread over more waves (each wave's top-k time is one pass over its
// lanes' experts, whatever the number of its tokens).
int router_tpb(const moe_config& c, bool from_logits) {
  if (!from_logits) return kTok;
  return c.num_tokens <= 256 ? 4 : c.num_tokens <= 4096 ? 16 : kTok;
}

int router_num_blocks(const moe_config& c, bool from_logits) {
  const int tpb = router_tpb(c, from_logits);
  return (c.num_tokens + tpb - 1) / tpb;
}

int router_k_splits(const moe_config& c) {
  if (c.dtype != MOE_DTYPE_BF16) return 1;
  // Split only grids below one block per CU: above that the fused kernel (logits
  // and top-k in one pass) is faster than split + reduce + a top-k pass.
  int ks = 1;
  while (router_num_blocks(c, false) * ks * 2 <= 256 && c.hidden % (ks * 2 * kBK) == 0 &&
         c.hidden / (ks * 2) >= 2 * kBK)
    ks *= 2;
  return ks;
}

namespace {

void launch_partial(const moe_config& c, const void* x, const void* w, float* part,
                    hipStream_t s) {
  const int ks = router_k_splits(c), E = c.num_experts;
  const int EP = (E + 31) & ~31;
  size_t lds = (size_t)kTok * (EP + 1) * sizeof(float);
  const size_t tiles = router_tile_lds(E);
  if (tiles > lds) lds = tiles;
  router_partial_kernel<<<dim3(router_num_blocks(c, false), ks), kThreads, lds, s>>>(
      c.num_tokens, c.hidden, E, c.hidden / ks, static_cast<const uint16_t*>(x),
      static_cast<const uint16_t*>(w), part);
}

}  // namespace

hipError_t launch_router_split(const moe_config& c, const void* x, const void* w_router,
                               const float* bias, float* logits_out, float* part,
                               int32_t* topk_idx, float* topk_w, float* prob_partials,
                               hipStream_t s, const RouterExtras& ex) {
  if (router_direct(c)) {  // the logits in one launch, then the top-k pass from them
    float* lg = logits_out ? logits_out : part;
    launch_logits_direct(c, x, w_router, bias, lg, s);
    RouterExtras e2 = ex;
    e2.noise = nullptr;
    e2.nlogits = nullptr;
    e2.logits_final = nullptr;
    e2.part = nullptr;
    e2.nsplit = 0;
    return launch_router(c, nullptr, nullptr, nullptr, lg, false, topk_idx, topk_w,
                         prob_partials, true, s, e2);
  }
  launch_partial(c, x, w_router, part, s);
  RouterExtras e2 = ex;
  e2.noise = nullptr;  // the split path serves the plain logits
  e2.nlogits = nullptr;
  e2.logits_final = logits_out;
  e2.part = part;
  e2.nsplit = router_k_splits(c);
  return launch_router(c, nullptr, nullptr, bias, nullptr, false, topk_idx, topk_w,
                       prob_partials, true, s, e2);
}

hipError_t launch_logits_split(const moe_config& c, const void* x, const void* w,
                               const float* bias, float* out, float* part, hipStream_t s) {
  if (router_direct(c)) {
    launch_logits_direct(c, x, w, bias, out, s);
    return hipGetLastError();
  }
  launch_partial(c, x, w, part, s);
  const int n = c.num_tokens * c.num_experts;
  router_reduce_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(
      c.num_tokens, c.num_experts, router_k_splits(c), part, bias, out, nullptr);
  return hipGetLastError();
}

hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const float* bias, float* logits, bool logits_out, int32_t* topk_idx,
                         float* topk_w, float* prob_partials, bool do_select, hipStream_t s,
                         const RouterExtras& ex) {
  const int E = c.num_experts;
  size_t lds = (size_t)kTok * router_ls(E, 64) * sizeof(float);
  if (x && c.dtype == MOE_DTYPE_BF16) {
    const size_t tiles = router_tile_lds(E);
    if (tiles > lds) lds = tiles;
  }
  if (lds < 4 * 256 * sizeof(float)) lds = 4 * 256 * sizeof(float);
  const bool from_logits = (x == nullptr);
  const int tpb = router_tpb(c, from_logits);
  const dim3 grid(router_num_blocks(c, from_logits)), block(kThreads);
  const float* lin = x ? nullptr : logits;
  float* lout = x ? (logits_out ? logits : nullptr) : ex.logits_final;
  const float* noise = x ? nullptr : ex.noise;
#define MOE_ROUTER_LAUNCH(BF, KM_, LPT_)                                                      \
  router_kernel<BF, KM_, LPT_><<<grid, block, lds, s>>>(                                        \
      c.num_tokens, c.hidden, E, c.top_k, c.norm_topk_prob, x, w_router, bias, lin, lout,       \
      topk_idx, topk_w, prob_partials, do_select, tpb, noise, ex.nlogits, ex.sel_bias, ex.zpart, \
      ex.k_min, ex.kt_out, ex.part, ex.nsplit)
#define MOE_ROUTER_KM(BF, LPT_)                             \
  do {                                                      \
    const int k = c.top_k;                                  \
    if (k <= 1) MOE_ROUTER_LAUNCH(BF, 1, LPT_);             \
    else if (k <= 2) MOE_ROUTER_LAUNCH(BF, 2, LPT_);        \
    else if (k <= 4) MOE_ROUTER_LAUNCH(BF, 4, LPT_);        \
    else if (k <= 8) MOE_ROUTER_LAUNCH(BF, 8, LPT_);        \
    else MOE_ROUTER_LAUNCH(BF, 16, LPT_);                   \
  } while (0)
#define MOE_ROUTER_LPT(BF)                                  \
  do {                                                      \
    if (tpb == kTok) MOE_ROUTER_KM(BF, 4);                  \
    else if (tpb == 16) MOE_ROUTER_KM(BF, 16);              \
    else MOE_ROUTER_KM(BF, 64);                             \
  } while (0)
  // the top-k list length: the power of two at or above k; lanes per token:
  // 256 / tokens per block (64-token blocks, which compute logits, use 4)
  if (c.dtype == MOE_DTYPE_BF16)
    MOE_ROUTER_LPT(true);
  else
    MOE_ROUTER_LPT(false);
#undef MOE_ROUTER_LPT
#undef MOE_ROUTER_KM
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

hipError_t launch_logits(const moe_config& c, const void* x, const void* w, const float* bias,
                         float* out, hipStream_t s) {
  return launch_router(c, x, w, bias, out, true, nullptr, nullptr, nullptr, false, s, {});
}

}  // namespace moe
