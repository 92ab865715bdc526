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
//  2. each wave takes a quarter of the tokens, up to 4 at a time (their
//     reductions interleave); lanes hold experts e = lane + 64q. Softmax
//     max/sum are xor-butterfly reductions (every lane ends with the same
//     bits). Top-k is k rounds of a wave max over 64-bit keys (order-preserving
//     fp32 bits, then 0xFFFF - e), so equal logits go to the lower expert
//     index; -0.0 is folded into +0.0 first.
//  3. per-block sums of the full softmax over the block's tokens (fixed order)
//     for the load-balance statistic P_e, and of (ln sum_e exp l)^2 for the
//     router z-loss.
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

// Logits tile by bf16 MFMA into s_log[t * ls + e] (+ bias).
__device__ __forceinline__ void router_logits_mfma(int T, int H, int E, int t0, int kbeg, int kend,
                                   const uint16_t* __restrict__ x,
                                   const uint16_t* __restrict__ wr, const float* __restrict__ bias,
                                   char* smem, float* s_log, int ls) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int EP = (E + 31) & ~31;
  uint16_t* s_x = reinterpret_cast<uint16_t*>(smem);  // [64][64]
  uint16_t* s_w = s_x + kTok * kBK;                     // [EP][64]
  const int ntiles = (EP / 32) * 2;                     // (expert block, token block)

  // tiles of this wave: (expert block, token block) q * 4 + wave for q < nq
  const int nq = ntiles > wave ? (ntiles - wave + 3) / 4 : 0;

  // Two register sets: the loads of steps kt + 1 and kt + 2 are in flight
  // while step kt is multiplied. The loads are unconditional (rows clamped)
  // and the tile count is a compile-time constant of the loop, so the
  // compiler's load counting stays exact and each set is waited for only
  // where it is stored. Barriers order LDS only.
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // 16 bytes in registers
  auto gload = [&](int k0, v4u (&rx)[2], v4u (&rw)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      const int gt = t0 + row < T ? t0 + row : T - 1;  // rows past T are never stored
      rx[i] = *reinterpret_cast<const v4u*>(x + (size_t)gt * H + k0 + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      const int gr = row < E ? row : E - 1;  // slots past E re-read row E-1 (one line)
      rw[i] = *reinterpret_cast<const v4u*>(wr + (size_t)gr * H + k0 + ch * 8);
    }
  };
  auto sstore = [&](const v4u (&rx)[2], const v4u (&rw)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      *reinterpret_cast<v4u*>(s_x + swz(row, ch)) = rx[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      if (32 * i < EP) *reinterpret_cast<v4u*>(s_w + swz(row, ch)) = rw[i];
    }
  };
  auto kloop = [&](auto nq_c) __attribute__((always_inline)) {
    constexpr int NQ = decltype(nq_c)::value;
    f32x16_t acc[NQ > 0 ? NQ : 1];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int tile = q * 4 + wave;
          const int eb = tile >> 1, tb = tile & 1;
          const int er = eb * 32 + (lane & 31), tr = tb * 32 + (lane & 31);
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(s_w + swz(er, ch));
          const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(s_x + swz(tr, ch));
          acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
        }
      }
    };
    const int nk = (kend - kbeg) / kBK;
    v4u rxa[2], rwa[8], rxb[2], rwb[8];  // the two load sets
    gload(kbeg, rxa, rwa);
    if (nk > 1) gload(kbeg + kBK, rxb, rwb);
    for (int kt = 0; kt < nk; kt += 2) {
      lds_barrier();  // previous compute done with the tile
      sstore(rxa, rwa);
      lds_barrier();
      if (kt + 2 < nk) gload(kbeg + (kt + 2) * kBK, rxa, rwa);
      compute();
      if (kt + 1 < nk) {
        lds_barrier();
        sstore(rxb, rwb);
        lds_barrier();
        if (kt + 3 < nk) gload(kbeg + (kt + 3) * kBK, rxb, rwb);
        compute();
      }
    }
    __syncthreads();  // tiles dead; s_log aliases them
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
  switch (nq) {  // wave-uniform
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    default: kloop(std::integral_constant<int, 4>{}); break;
  }
}

// NT: tokens a wave reduces together (1 when a wave owns a single token).
template <bool BF16, int NT>
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
  const int ls = ((E + 31) & ~31) + 1;
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
  } else if constexpr (BF16) {
    router_logits_mfma(T, H, E, t0, 0, H, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(wr), bias, smem, s_log, ls);
  } else {
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

  const int EQ = (E + 63) >> 6;  // <= 4 experts per lane
  float pacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float zacc = 0.0f;  // this wave's sum of (ln sum_e exp l)^2 over its tokens
  // Each wave owns tpb / 4 tokens, taken NT at a time: their cross-lane
  // reductions are independent chains, so the shuffle latencies overlap.
  const int tpw = tpb / 4;
  for (int tt = 0; tt < tpw; tt += NT) {
    const int tb0 = wave * tpw + tt;
    if (t0 + tb0 >= T) break;  // wave-uniform
    bool ok[NT];
    float v[NT][4], m[NT], ex[NT][4], ssum[NT], inv[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int t = tb0 + u, gt = t0 + t;
      const bool mine = tt + u < tpw;  // a row of this wave (and of this block)
      ok[u] = mine && gt < T;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        v[u][q] = (q < EQ && e < E) ? (mine ? s_log[t * ls + e] : 0.0f) : -INFINITY;
        if (logits_out && ok[u] && q < EQ && e < E) logits_out[(size_t)gt * E + e] = v[u][q];
      }
      m[u] = fmaxf(fmaxf(v[u][0], v[u][1]), fmaxf(v[u][2], v[u][3]));
    }
    wave_max_n(m);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      ssum[u] = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        ex[u][q] = (q < EQ && e < E) ? expf(v[u][q] - m[u]) : 0.0f;
        ssum[u] += ex[u][q];
      }
    }
    wave_sum_n(ssum);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      inv[u] = 1.0f / ssum[u];
      if (ok[u]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pacc[q] += ex[u][q] * inv[u];
        const float lse = m[u] + logf(ssum[u]);
        zacc = fmaf(lse, lse, zacc);
      }
    }

    // entropy-driven number of experts ([QWEN3-ROUTE] §二 dynamic TopK):
    // k_t = clamp(floor(k_min + (k - k_min) H_t / ln E)), H_t = -sum p ln max(p, 1e-10)
    int kt[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) kt[u] = k;
    if (k_min > 0) {
      float hs[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        hs[u] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float pe = ex[u][q] * inv[u];
          if (q < EQ && lane + 64 * q < E) hs[u] = fmaf(pe, logf(fmaxf(pe, 1e-10f)), hs[u]);
        }
      }
      wave_sum_n(hs);
      const float span = (float)(k - k_min) / logf((float)E);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int kk = (int)floorf(fmaf(-hs[u], span, (float)k_min));
        kt[u] = kk < k_min ? k_min : (kk > k ? k : kk);
        if (kt_out && ok[u] && lane == 0) kt_out[t0 + tb0 + u] = kt[u];
      }
    }

    if (do_select) {
      uint32_t key[NT][4];
      int my_e[NT];
      float my_p[NT], psum[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        my_e[u] = 0;
        my_p[u] = 0.0f;
        psum[u] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = lane + 64 * q;
          const bool live = q < EQ && e < E;
          key[u][q] = live ? order_key(sel_bias ? v[u][q] + sel_bias[e] : v[u][q]) : 0u;
        }
      }
      for (int j = 0; j < k; ++j) {
        unsigned long long best[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          best[u] = 0ull;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const unsigned long long cand = (static_cast<unsigned long long>(key[u][q]) << 32) |
                                            (0xFFFFu - (unsigned)(lane + 64 * q));
            best[u] = (key[u][q] != 0u && cand > best[u]) ? cand : best[u];
          }
        }
        wave_max_u64_n(best);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const int ej = 0xFFFF - static_cast<int>(best[u] & 0xFFFFull);
          if ((ej & 63) == lane) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (q == (ej >> 6)) key[u][q] = 0u;
          }
          // with a selection bias the key is not the logit: read the logit back
          const float lj = sel_bias ? s_log[(tb0 + u) * ls + ej]
                                    : key_value(static_cast<uint32_t>(best[u] >> 32));
          const float pj = expf(lj - m[u]) * inv[u];
          if (j < kt[u]) psum[u] += pj;
          if (lane == j) {
            my_e[u] = ej;
            my_p[u] = pj;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int gt = t0 + tb0 + u;
        if (ok[u] && lane < k) {  // slots past k_t are empty (dynamic k)
          const bool live = lane < kt[u];
          topk_idx[(size_t)gt * k + lane] = live ? my_e[u] : -1;
          topk_w[(size_t)gt * k + lane] = live ? (norm ? my_p[u] / psum[u] : my_p[u]) : 0.0f;
        }
      }
    }
  }

  if (zpart) {  // fixed order: waves 0..3, each in its token order
    __shared__ float s_z[4];
    __syncthreads();
    if (lane == 0) s_z[wave] = zacc;
    __syncthreads();
    if (tid == 0) zpart[blockIdx.x] = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
  }
  if (partials) {
    __syncthreads();  // every wave is done with s_log
    float* s_part = reinterpret_cast<float*>(smem);  // [4][256]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < 256) s_part[wave * 256 + e] = pacc[q];
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads)
      partials[(size_t)blockIdx.x * E + e] =
          ((s_part[e] + s_part[256 + e]) + s_part[512 + e]) + s_part[768 + e];
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

}  // namespace

// Tokens per router block: 64 when the block computes its logits (one MFMA
// tile); fewer when it starts from logits and T is small, so that more waves
// share the top-k work (its cost is the serial reduction chain of each wave).
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
  const size_t tiles = (size_t)(kTok + EP) * kBK * sizeof(uint16_t);
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
  const int EP = (E + 31) & ~31;
  size_t lds = (size_t)kTok * (EP + 1) * sizeof(float);
  if (x && c.dtype == MOE_DTYPE_BF16) {
    const size_t tiles = (size_t)(kTok + EP) * kBK * sizeof(uint16_t);
    if (tiles > lds) lds = tiles;
  }
  if (lds < 4 * 256 * sizeof(float)) lds = 4 * 256 * sizeof(float);
  const bool from_logits = (x == nullptr);
  const int tpb = router_tpb(c, from_logits);
  const dim3 grid(router_num_blocks(c, from_logits)), block(kThreads);
  const float* lin = x ? nullptr : logits;
  float* lout = x ? (logits_out ? logits : nullptr) : ex.logits_final;
  const float* noise = x ? nullptr : ex.noise;
#define MOE_ROUTER_LAUNCH(BF, NT_)                                                            \
  router_kernel<BF, NT_><<<grid, block, lds, s>>>(                                              \
      c.num_tokens, c.hidden, E, c.top_k, c.norm_topk_prob, x, w_router, bias, lin, lout,       \
      topk_idx, topk_w, prob_partials, do_select, tpb, noise, ex.nlogits, ex.sel_bias, ex.zpart, \
      ex.k_min, ex.kt_out, ex.part, ex.nsplit)
  const bool one = tpb / 4 == 1;  // one token per wave
  if (c.dtype == MOE_DTYPE_BF16) {
    // With the logits computed here (64 tokens per block, one block per 64
    // tokens) a wave's 16 tokens go through the top-k as one interleaved
    // group: 16 independent reduction chains hide each other's latency at one
    // wave per SIMD (router 116 -> 105 us at 16K tokens x 128 experts).
    if (one) MOE_ROUTER_LAUNCH(true, 1);
    else if (x) MOE_ROUTER_LAUNCH(true, 16);
    else MOE_ROUTER_LAUNCH(true, 4);
  } else {
    if (one) MOE_ROUTER_LAUNCH(false, 1); else MOE_ROUTER_LAUNCH(false, 4);
  }
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

hipError_t launch_logits(const moe_config& c, const void* x, const void* w, const float* bias,
                         float* out, hipStream_t s) {
  return launch_router(c, x, w, bias, out, true, nullptr, nullptr, nullptr, false, s, {});
}

}  // namespace moe
