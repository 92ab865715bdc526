/*
 * moe_oracle.c — plain CPU oracle of the sparse MoE block forward.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library. The GPU product path shares no
 * code with it and never calls it.
 *
 * Every function is the written-out definition of one step, as scalar loops
 * with fp64 accumulation; no blocking, fusion or reordering beyond what the
 * definition states. OpenMP only splits independent tokens / rows.
 *
 * Sources (web pages, cited by title and section):
 *   [QWEN3-READ]  "大模型-qwen3 MoE 详细解读" (cnblogs), Qwen3MoeSparseMoeBlock
 *                 forward code and §三 (Mixtral difference).
 *   [MOE-128x8]   "MoE架构深度解析：128专家与8激活的智能路由" (csdn), load-balancing
 *                 section and the expert parameter table.
 *   [LAB17]       "项目 17：稀疏性的调度艺术：实现双专家 MoE 路由" (sshipanoo),
 *                 第二阶段 实现流程.
 *
 * Parity unpinned: orc_z_loss (the page names the statistic without a
 * formula; see there). Every other function is pinned by the CPU tests to
 * something outside itself.
 *
 * Element types: dtype 0 = fp32 array, dtype 1 = bf16 array given as the
 * 16-bit patterns (widened to double exactly).
 * All functions return 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact widening of one element to double. */
static double elem(const void* p, int dtype, size_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static void round_bf16_inplace(double* v) {
  /* round-to-nearest-even of the fp32 value to bf16, back to double */
  float f = (float)*v;
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  uint32_t lsb = (b >> 16) & 1u;
  b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;
  memcpy(&f, &b, sizeof f);
  *v = (double)f;
}

/* Router logits, [QWEN3-READ] forward code (gate = Linear(H, E, bias=False)):
 *   l[t,e] = fp32( sum_{h ascending} x[t,h] * Wr[e,h]  (+ bias[e]) )
 * bias is an optional additive per-expert logit offset (NULL: none). */
int orc_logits(int T, int H, int E, int dtype, const void* x, const void* wr,
               const float* bias, float* logits) {
  if (T < 0 || H < 1 || E < 1 || !x || !wr || !logits) return -1;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += elem(x, dtype, (size_t)t * H + h) * elem(wr, dtype, (size_t)e * H + h);
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  }
  return 0;
}

/* Softmax over the experts and top-k selection, [QWEN3-READ] forward code:
 *   p[t,e] = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t),  m_t = max_e l[t,e]
 *   slots j = 0..k-1 hold the k experts with the largest logits, in descending
 *   order of the fp32 logit; equal logits are ordered by ascending expert index
 *   (C float comparison, so +0.0 == -0.0). Selecting on logits is selecting on
 *   p, since softmax is strictly increasing.
 *   w[t,j] = p[t,e_j] / sum_j' p[t,e_j']  if norm (Qwen3), else p[t,e_j]
 *   (Mixtral keeps the unrenormalised probabilities, [QWEN3-READ] §三).
 * forced_idx (nullable): use these experts instead of selecting (weights are
 * computed the same way from them). A negative forced id is an empty slot,
 * as entropy-driven k leaves them ([QWEN3-ROUTE] §二): weight 0, and the
 * renormalisation runs over the slots that hold an expert.
 * probs (nullable) receives the full softmax [T,E]. */
int orc_route_sel(int T, int E, int k, int norm, const float* logits, const float* sel_bias,
                  const int32_t* forced_idx, int32_t* idx, double* w, double* probs);

int orc_route(int T, int E, int k, int norm, const float* logits, const int32_t* forced_idx,
              int32_t* idx, double* w, double* probs) {
  return orc_route_sel(T, E, k, norm, logits, NULL, forced_idx, idx, w, probs);
}

/* orc_route with a selection-only bias, [LAB17] (DeepSeek-V3's balancing
 * without an auxiliary loss: a per-expert bias moves the routing decision, the
 * model's own scores keep the weights): the k experts are chosen by the fp32
 * key l[t,e] + sel_bias[e] (descending, ties to the lower index), the weights
 * and probs come from the softmax of the unbiased l. sel_bias NULL: no bias. */
int orc_route_sel(int T, int E, int k, int norm, const float* logits, const float* sel_bias,
                  const int32_t* forced_idx, int32_t* idx, double* w, double* probs) {
  if (T < 0 || E < 1 || k < 1 || k > E || !logits || !idx || !w) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    double m = -INFINITY;
    for (int e = 0; e < E; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += exp((double)l[e] - m);
    if (probs)
      for (int e = 0; e < E; ++e) probs[(size_t)t * E + e] = exp((double)l[e] - m) / s;

    int32_t* sel = idx + (size_t)t * k;
    if (forced_idx) {
      for (int j = 0; j < k; ++j) {
        sel[j] = forced_idx[(size_t)t * k + j];
        if (sel[j] >= E) bad = 1;
      }
    } else {
      /* k passes of "largest remaining key, lowest index on ties"; the key is
       * the fp32 logit, plus the selection bias (an fp32 addition) if given */
      for (int j = 0; j < k; ++j) {
        int best = -1;
        float best_key = 0.0f;
        for (int e = 0; e < E; ++e) {
          int taken = 0;
          for (int q = 0; q < j; ++q)
            if (sel[q] == e) taken = 1;
          if (taken) continue;
          const float key = sel_bias ? l[e] + sel_bias[e] : l[e];
          if (best < 0 || key > best_key) { /* strict: earlier index wins ties */
            best = e;
            best_key = key;
          }
        }
        sel[j] = best;
      }
    }
    if (bad) continue;
    double psum = 0.0;
    for (int j = 0; j < k; ++j)
      if (sel[j] >= 0) psum += exp((double)l[sel[j]] - m) / s;
    for (int j = 0; j < k; ++j) {
      if (sel[j] < 0) { /* empty slot (forced routing only) */
        w[(size_t)t * k + j] = 0.0;
        continue;
      }
      double p = exp((double)l[sel[j]] - m) / s;
      w[(size_t)t * k + j] = norm ? p / psum : p;
    }
  }
  return bad ? -1 : 0;
}

/* Entropy-driven number of experts per token, [QWEN3-ROUTE] §二 (dynamic
 * TopK: the token's complexity is the entropy of its router probabilities):
 *   H_t = -sum_e p[t,e] ln(max(p[t,e], 1e-10))
 *   k_t = clamp( floor(k_min + (k_max - k_min) * H_t / ln E), k_min, k_max )
 * then the k_t experts with the largest logits (ties to the lower index) take
 * slots 0..k_t-1 and their weights are renormalised over those k_t (norm) or
 * left as probabilities; slots k_t..k_max-1 are empty (idx -1, w 0).
 * kt [T] receives k_t; xk [T] (nullable) the unfloored k_min + (k_max -
 * k_min) H_t / ln E. */
int orc_route_dynamic(int T, int E, int k_max, int k_min, int norm, const float* logits,
                      int32_t* idx, double* w, int32_t* kt, double* xk) {
  if (T < 0 || E < 2 || k_min < 1 || k_max < k_min || k_max > E || !logits || !idx || !w || !kt)
    return -1;
  double* probs = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * E);
  if (!probs) return -1;
  /* the full top-k_max selection and probabilities first */
  if (orc_route(T, E, k_max, 0, logits, NULL, idx, w, probs)) {
    free(probs);
    return -1;
  }
  for (int t = 0; t < T; ++t) {
    const double* p = probs + (size_t)t * E;
    double H = 0.0;
    for (int e = 0; e < E; ++e) H -= p[e] * log(p[e] > 1e-10 ? p[e] : 1e-10);
    const double x = (double)k_min + (double)(k_max - k_min) * H / log((double)E);
    int k = (int)floor(x);
    if (k < k_min) k = k_min;
    if (k > k_max) k = k_max;
    kt[t] = k;
    if (xk) xk[t] = x;
    double psum = 0.0;
    for (int j = 0; j < k; ++j) psum += w[(size_t)t * k_max + j]; /* unrenormalised p */
    for (int j = 0; j < k_max; ++j) {
      if (j < k) {
        if (norm) w[(size_t)t * k_max + j] /= psum;
      } else {
        idx[(size_t)t * k_max + j] = -1;
        w[(size_t)t * k_max + j] = 0.0;
      }
    }
  }
  free(probs);
  return 0;
}

/* Noisy logits, [MOE-128x8] router pseudocode (noisy_logits = logits + noise *
 * softplus(x @ W_noise)) and [LAB17] noisy top-k gating (standard normal noise
 * times Softplus(W_noise x) added to the gate logits):
 *   out[t,e] = fp32( l[t,e] + noise[t,e] * softplus(nl[t,e]) ),
 *   softplus(z) = ln(1 + e^z)
 * nl = x W_noise^T (orc_logits with the noise matrix); the noise values are an
 * input (drawn by the caller). */
int orc_noisy_logits(int T, int E, const float* logits, const float* nlogits, const float* noise,
                     float* out) {
  if (T < 0 || E < 1 || !logits || !nlogits || !noise || !out) return -1;
  for (size_t i = 0; i < (size_t)T * E; ++i) {
    const double z = (double)nlogits[i];
    const double sp = z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
    out[i] = (float)((double)logits[i] + (double)noise[i] * sp);
  }
  return 0;
}

/* Router z-loss statistic. [MOE-128x8] names a router z-loss for training
 * stability without a formula; the one taken here is the mean over tokens of
 * the squared log-sum-exp of the router logits:
 *   z = (1/T) sum_t ( ln sum_e exp(l[t,e]) )^2
 * PARITY UNPINNED: the page fixes no formula, so the pins (closed forms,
 * scipy logsumexp) check only this chosen definition. */
int orc_z_loss(int T, int E, const float* logits, double* z) {
  if (T < 1 || E < 1 || !logits || !z) return -1;
  double acc = 0.0;
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    double m = -INFINITY;
    for (int e = 0; e < E; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += exp((double)l[e] - m);
    const double lse = m + log(s);
    acc += lse * lse;
  }
  *z = acc / (double)T;
  return 0;
}

/* Dispatch as a counting sort of the pairs by expert ([QWEN3-READ] §三: put the
 * tokens of one expert next to each other, and keep the inverse):
 *   counts[e] = #{p : idx[p] == e};  offsets = exclusive prefix sum;
 *   sorted_pair = pair ids grouped by expert, ascending inside a group;
 *   pair_pos[sorted_pair[i]] = i. An idx of -1 is an empty slot: not a pair,
 *   pair_pos = -1. */
int orc_dispatch(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_pos) {
  if (T < 0 || E < 1 || k < 1 || !idx || !counts || !offsets || !sorted_pair || !pair_pos)
    return -1;
  const long P = (long)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long p = 0; p < P; ++p) {
    if (idx[p] == -1) continue; /* empty slot (a token routed to fewer than k experts) */
    if (idx[p] < 0 || idx[p] >= E) return -1;
    counts[idx[p]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return -1;
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (long p = 0; p < P; ++p) {
    if (idx[p] == -1) {
      pair_pos[p] = -1;
      continue;
    }
    int32_t pos = fill[idx[p]]++;
    sorted_pair[pos] = (int32_t)p;
    pair_pos[p] = pos;
  }
  free(fill);
  return 0;
}

/* Expert capacity, [MOE-128x8] 容量因子设计: capacity = (tokens per batch /
 * experts) x capacity factor. With k slots per token the per-expert load the
 * factor applies to is T*k/E, so C = ceil(T * k * cf / E) (k = 1 is the
 * page's formula). */
int orc_capacity(int T, int E, int k, double cf) {
  if (T < 1 || E < 1 || k < 1 || !(cf > 0.0)) return -1;
  double c = ceil((double)T * (double)k * cf / (double)E);
  if (c < 1.0) c = 1.0;
  if (c > (double)T * k) c = (double)T * k;
  return (int)c;
}

/* Capacity-limited dispatch, [QWEN3-ROUTE] §四 (inference routing with
 * capacity: the tokens are taken in order, and an expert accepts a token while
 * the number it has accepted is below its capacity):
 *   walk the pairs p = t*k + j in increasing order; p is kept iff fewer than
 *   `capacity` earlier pairs went to the same expert;
 *   counts[e] = pairs routed to e (before the limit);
 *   offsets = exclusive prefix sum of the kept counts;
 *   sorted_pair = the kept pair ids grouped by expert, ascending inside a
 *   group; pair_pos[p] = its position, or -1 for a dropped pair;
 *   *dropped = number of dropped pairs. */
int orc_dispatch_capacity(int T, int E, int k, int capacity, const int32_t* idx,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, int32_t* dropped) {
  if (T < 0 || E < 1 || k < 1 || capacity < 1 || !idx || !counts || !offsets || !sorted_pair ||
      !pair_pos || !dropped)
    return -1;
  const long P = (long)T * k;
  int32_t* accepted = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!accepted) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  *dropped = 0;
  for (long p = 0; p < P; ++p) { /* the walk: keep or drop, in pair order */
    const int e = idx[p];
    if (e == -1) { /* empty slot: not a pair */
      pair_pos[p] = -2;
      continue;
    }
    if (e < 0 || e >= E) {
      free(accepted);
      return -1;
    }
    counts[e] += 1;
    if (accepted[e] < capacity) {
      accepted[e] += 1;
      pair_pos[p] = 0; /* kept: position filled in below */
    } else {
      pair_pos[p] = -1;
      *dropped += 1;
    }
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + accepted[e];
  for (int e = 0; e < E; ++e) accepted[e] = offsets[e]; /* next free slot */
  for (long p = 0; p < P; ++p) {
    if (pair_pos[p] < 0) {
      pair_pos[p] = -1; /* dropped or empty */
      continue;
    }
    const int32_t pos = accepted[idx[p]]++;
    sorted_pair[pos] = (int32_t)p;
    pair_pos[p] = pos;
  }
  free(accepted);
  return 0;
}

/* Capacity-limited routing with the least-loaded fallback, [QWEN3-ROUTE] §四
 * (inference routing with expert capacities). The tokens are taken in order.
 * Each of a token's experts, in slot order, accepts it while the number of
 * tokens that expert has accepted is below `capacity`, and its count then
 * grows by one. A token left with fewer than `fallback_min` accepted experts
 * gets the least-loaded experts added: ascending accepted count at that
 * moment (the token's own acceptances included), ties to the lower id, as
 * many as it lacks. Those additions are not counted as acceptances.
 * Slot form of the result (readings: the page keeps token lists per expert
 * and does not weight them): a kept slot keeps its expert and weight; the
 * added experts, in the order taken, go to the token's dropped slots in slot
 * order, each with that slot's weight, and no more are added than the token
 * has dropped slots; dropped slots left over and empty slots (id -1) get id -1
 * and weight 0. *dropped counts the dropped slots left over. fallback_min = 0
 * leaves every dropped slot empty (the plain capacity limit). */
int orc_capacity_fallback(int T, int E, int k, int capacity, int fallback_min,
                          const int32_t* idx, const float* w, int32_t* idx_out, float* w_out,
                          int32_t* dropped) {
  if (T < 0 || E < 1 || k < 1 || capacity < 1 || fallback_min < 0 || fallback_min > k || !idx ||
      !w || !idx_out || !w_out || !dropped)
    return -1;
  int32_t* accepted = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  char* taken = (char*)malloc((size_t)E);
  if (!accepted || !taken) {
    free(accepted);
    free(taken);
    return -1;
  }
  *dropped = 0;
  for (int t = 0; t < T; ++t) {
    const long p0 = (long)t * k;
    int kept = 0, ndrop = 0;
    for (int j = 0; j < k; ++j) { /* the token's experts, in slot order */
      const int e = idx[p0 + j];
      idx_out[p0 + j] = -1;
      w_out[p0 + j] = 0.0f;
      if (e == -1) continue; /* empty slot */
      if (e < 0 || e >= E) {
        free(accepted);
        free(taken);
        return -1;
      }
      if (accepted[e] < capacity) {
        accepted[e] += 1;
        idx_out[p0 + j] = e;
        w_out[p0 + j] = w[p0 + j];
        kept += 1;
      } else {
        ndrop += 1;
      }
    }
    int need = fallback_min - kept;
    if (need > ndrop) need = ndrop;
    if (need < 0) need = 0;
    /* the least-loaded experts, one at a time: the smallest (accepted, id)
     * not taken yet, i.e. the first `need` of the experts sorted by load */
    for (int e = 0; e < E; ++e) taken[e] = 0;
    int slot = 0;
    for (int r = 0; r < need; ++r) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || accepted[e] < accepted[best])) best = e;
      taken[best] = 1;
      /* the next dropped slot of the token */
      while (!(idx[p0 + slot] >= 0 && idx_out[p0 + slot] == -1)) ++slot;
      idx_out[p0 + slot] = best;
      w_out[p0 + slot] = w[p0 + slot];
      ++slot;
    }
    *dropped += ndrop - need;
  }
  free(accepted);
  free(taken);
  return 0;
}

/* One expert MLP per requested row, [MOE-128x8] gate_proj / up_proj / down_proj
 * with the SwiGLU form down(silu(gate x) * up x), no biases:
 *   g_i = sum_h Wg[e,i,h] x[t,h],  u_i = sum_h Wu[e,i,h] x[t,h]
 *   a_i = silu(g_i) * u_i,  silu(z) = z / (1 + exp(-z))
 *   y[r,h] = sum_i Wd[e,h,i] a_i
 * Layouts: x [*,H]; Wg, Wu [E,I,H]; Wd [E,H,I]. Row r uses token tok[r] and
 * expert ex[r]. round_h != 0 rounds each a_i to bf16 first (diagnostic mode
 * mirroring a bf16 intermediate). */
int orc_expert_rows(int H, int I, int dtype, const void* x, const void* wg, const void* wu,
                    const void* wd, int n, const int32_t* tok, const int32_t* ex, int round_h,
                    double* y) {
  if (H < 1 || I < 1 || n < 0 || !x || !wg || !wu || !wd || !tok || !ex || !y) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    if (!a) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
      if (!a) continue;
      const size_t t = (size_t)tok[r], e = (size_t)ex[r];
      for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        const size_t wrow = (e * (size_t)I + (size_t)i) * (size_t)H;
        for (int h = 0; h < H; ++h) {
          const double xv = elem(x, dtype, t * (size_t)H + h);
          g += elem(wg, dtype, wrow + h) * xv;
          u += elem(wu, dtype, wrow + h) * xv;
        }
        a[i] = g / (1.0 + exp(-g)) * u;
        if (round_h) round_bf16_inplace(&a[i]);
      }
      for (int h = 0; h < H; ++h) {
        double s = 0.0;
        const size_t drow = (e * (size_t)H + (size_t)h) * (size_t)I;
        for (int i = 0; i < I; ++i) s += elem(wd, dtype, drow + i) * a[i];
        y[(size_t)r * H + h] = s;
      }
    }
    free(a);
  }
  return bad ? -1 : 0;
}

/* 4-bit group-quantised weights, [MOE-128x8] 参数量化与存储优化 (4-bit codes,
 * group_size 128, an independent scale and bias per group):
 *   w[e,n,k] = scale[e,n,g] * q[e,n,k] + bias[e,n,g],  g = k / 128.
 * Storage (the library's layout, moe.h), rows in blocks of 32 (b = n / 32,
 * r = n % 32):
 *   q: the 1024-byte tile of (e, b, chunk k / 64) holds row r at byte 32 r as
 *      8 32-bit words of 8 consecutive elements, byte j of a word holding
 *      element j in its low nibble and j + 4 in its high nibble;
 *   sb: the (scale, bias) bf16 pair of (e, b, g, r), pairs in that order. */
static double w4_elem(const uint8_t* codes, const uint16_t* sb, int N, int K, size_t e, size_t n,
                      size_t k) {
  const size_t blk = e * (size_t)(N / 32) + n / 32, r = n % 32, j = k % 8;
  const uint8_t byte = codes[(blk * (size_t)(K / 64) + k / 64) * 1024 + r * 32 +
                             4 * ((k % 64) / 8) + j % 4];
  const int q = (j >= 4) ? (byte >> 4) : (byte & 0xF);
  const size_t pair = (blk * (size_t)(K / 128) + k / 128) * 32 + r;
  const double scale = elem(sb, 1, 2 * pair), bias = elem(sb, 1, 2 * pair + 1);
  return scale * (double)q + bias;
}

/* The dequantised matrices [E,N,K] as double. */
int orc_dequant_w4(int E, int N, int K, const uint8_t* codes, const uint16_t* sb, double* w) {
  if (E < 1 || N < 32 || N % 32 || K < 128 || K % 128 || !codes || !sb || !w) return -1;
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k)
        w[((size_t)e * N + n) * K + k] = w4_elem(codes, sb, N, K, e, n, k);
  return 0;
}

/* orc_expert_rows with 4-bit weights, dequantised element by element (the
 * same definition as orc_dequant_w4 followed by orc_expert_rows):
 *   gate/up codes and (scale, bias) of N = I rows by K = H, down of N = H by
 *   K = I, in the tiles of w4_elem; x [*,H] of dtype (0 fp32, 1 bf16). */
int orc_expert_rows_w4(int H, int I, int dtype, const void* x, const uint8_t* cg,
                       const uint16_t* sg, const uint8_t* cu, const uint16_t* su,
                       const uint8_t* cd, const uint16_t* sd, int n, const int32_t* tok,
                       const int32_t* ex, int round_h, double* y) {
  if (H < 128 || I < 128 || H % 128 || I % 128 || n < 0 || !x || !cg || !sg || !cu || !su ||
      H % 32 || I % 32 ||
      !cd || !sd || !tok || !ex || !y)
    return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    if (!a) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
      if (!a) continue;
      const size_t t = (size_t)tok[r], e = (size_t)ex[r];
      for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
          const double xv = elem(x, dtype, t * (size_t)H + h);
          g += w4_elem(cg, sg, I, H, e, i, h) * xv;
          u += w4_elem(cu, su, I, H, e, i, h) * xv;
        }
        a[i] = g / (1.0 + exp(-g)) * u;
        if (round_h) round_bf16_inplace(&a[i]);
      }
      for (int h = 0; h < H; ++h) {
        double s = 0.0;
        for (int i = 0; i < I; ++i) s += w4_elem(cd, sd, H, I, e, h, i) * a[i];
        y[(size_t)r * H + h] = s;
      }
    }
    free(a);
  }
  return bad ? -1 : 0;
}

/* orc_expert_rows for double weight arrays (x of dtype 0 / 1): used to check
 * the 4-bit path against dequantise-first. */
int orc_expert_rows_f64w(int H, int I, int dtype, const void* x, const double* wg,
                         const double* wu, const double* wd, int n, const int32_t* tok,
                         const int32_t* ex, double* y) {
  if (H < 1 || I < 1 || n < 0 || !x || !wg || !wu || !wd || !tok || !ex || !y) return -1;
  for (int r = 0; r < n; ++r) {
    const size_t t = (size_t)tok[r], e = (size_t)ex[r];
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    if (!a) return -1;
    for (int i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      for (int h = 0; h < H; ++h) {
        const double xv = elem(x, dtype, t * (size_t)H + h);
        g += wg[(e * I + i) * (size_t)H + h] * xv;
        u += wu[(e * I + i) * (size_t)H + h] * xv;
      }
      a[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int h = 0; h < H; ++h) {
      double s = 0.0;
      for (int i = 0; i < I; ++i) s += wd[(e * H + h) * (size_t)I + i] * a[i];
      y[(size_t)r * H + h] = s;
    }
    free(a);
  }
  return 0;
}

/* Routing-weighted combine, [QWEN3-READ] forward code (expert output times its
 * routing weight, accumulated into the token's row), over the kept slots:
 *   out[t,:] = sum_{j : keep[t,j]} w[t,j] * y_pair[t*k+j, :]  (slot order, double)
 * keep (nullable: all kept) marks the slots that a capacity limit did not drop;
 * a dropped slot contributes nothing. */
int orc_combine_kept(int T, int H, int k, const double* w, const double* y_pair,
                     const int8_t* keep, double* out) {
  if (T < 0 || H < 1 || k < 1 || !w || !y_pair || !out) return -1;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      double s = 0.0;
      for (int j = 0; j < k; ++j) {
        if (keep && !keep[(size_t)t * k + j]) continue;
        s += w[(size_t)t * k + j] * y_pair[((size_t)t * k + j) * H + h];
      }
      out[(size_t)t * H + h] = s;
    }
  }
  return 0;
}

/* All slots kept:
 *   out[t,:] = sum_{j=0..k-1} w[t,j] * y_pair[t*k+j, :]   (slot order, double) */
int orc_combine(int T, int H, int k, const double* w, const double* y_pair, double* out) {
  return orc_combine_kept(T, H, k, w, y_pair, NULL, out);
}

/* Load-balance statistics, [MOE-128x8] load-balancing section, n = E:
 *   f_e = counts[e] / sum_e' counts[e']   (fraction of routed pairs; = T*k
 *                                         when every token takes k experts)
 *   P_e = (1/T) sum_t probs[t,e]  (mean full-softmax probability)
 *   aux = E * sum_e f_e * P_e */
int orc_aux(int T, int E, int k, const int32_t* counts, const double* probs, double* f,
            double* P, double* aux) {
  if (T < 1 || E < 1 || k < 1 || !counts || !probs || !f || !P || !aux) return -1;
  double acc = 0.0;
  long routed = 0; /* T*k, or fewer when tokens take fewer than k experts */
  for (int e = 0; e < E; ++e) routed += counts[e];
  (void)k;
  for (int e = 0; e < E; ++e) {
    double s = 0.0;
    for (int t = 0; t < T; ++t) s += probs[(size_t)t * E + e];
    f[e] = routed > 0 ? (double)counts[e] / (double)routed : 0.0;
    P[e] = s / (double)T;
    acc += f[e] * P[e];
  }
  *aux = (double)E * acc;
  return 0;
}

/* The block forward for the tokens listed in `tokens` (all T when tokens ==
 * NULL): logits -> route -> experts -> combine, [QWEN3-READ] forward code.
 * n = number of listed tokens. Outputs are per listed token:
 *   logits [n,E] fp32, idx [n,k], w [n,k], out [n,H] double.
 * forced_idx [n,k] (nullable) replaces the selection (negative ids: empty
 * slots, weight 0); keep [n,k] (nullable) marks the slots a capacity limit
 * kept (the others contribute nothing). */
int orc_forward_tokens(int T, int H, int E, int k, int I, int norm, int dtype, const void* x,
                       const void* wr, const float* bias, const void* wg, const void* wu,
                       const void* wd, int n, const int32_t* tokens, const int32_t* forced_idx,
                       const int8_t* keep, int round_h, float* logits, int32_t* idx, double* w,
                       double* out) {
  if (T < 1 || n < 0 || !logits || !idx || !w || !out) return -1;
  const size_t rowb = (size_t)H * (dtype == 0 ? 4 : 2);
  /* gather the listed rows of x so the steps below see a dense [n,H] block */
  char* xs = (char*)malloc(rowb * (size_t)(n > 0 ? n : 1));
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * k);
  int32_t* ex = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * k);
  double* y = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * k * H);
  int rc = -1;
  if (!xs || !tok || !ex || !y) goto done;
  for (int r = 0; r < n; ++r) {
    int t = tokens ? tokens[r] : r;
    if (t < 0 || t >= T) goto done;
    memcpy(xs + rowb * r, (const char*)x + rowb * (size_t)t, rowb);
  }
  if (orc_logits(n, H, E, dtype, xs, wr, bias, logits)) goto done;
  if (orc_route(n, E, k, norm, logits, forced_idx, idx, w, NULL)) goto done;
  for (int r = 0; r < n; ++r)
    for (int j = 0; j < k; ++j) {
      tok[r * k + j] = r;
      /* an empty forced slot has weight 0: any expert's row serves */
      ex[r * k + j] = idx[r * k + j] < 0 ? 0 : idx[r * k + j];
    }
  if (orc_expert_rows(H, I, dtype, xs, wg, wu, wd, n * k, tok, ex, round_h, y)) goto done;
  if (orc_combine_kept(n, H, k, w, y, keep, out)) goto done;
  rc = 0;
done:
  free(xs);
  free(tok);
  free(ex);
  free(y);
  return rc;
}
