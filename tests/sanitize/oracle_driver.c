/*
 * oracle_driver.c — runs every function of oracle/moe_oracle.c on small
 * inputs (both element types, capacity drops, empty slots, 4-bit weights) and
 * on bad arguments, for an AddressSanitizer + UndefinedBehaviorSanitizer
 * build of the oracle (tests/test_sanitize.py). Test infrastructure: exits
 * non-zero when a call returns an unexpected status; the sanitizers abort on
 * any memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_logits(int T, int H, int E, int dtype, const void* x, const void* wr, const float* bias,
               float* logits);
int orc_route(int T, int E, int k, int norm, const float* logits, const int32_t* forced_idx,
              int32_t* idx, double* w, double* probs);
int orc_route_sel(int T, int E, int k, int norm, const float* logits, const float* sel_bias,
                  const int32_t* forced_idx, int32_t* idx, double* w, double* probs);
int orc_route_dynamic(int T, int E, int k_max, int k_min, int norm, const float* logits,
                      int32_t* idx, double* w, int32_t* kt, double* xk);
int orc_noisy_logits(int T, int E, const float* logits, const float* nlogits, const float* noise,
                     float* out);
int orc_z_loss(int T, int E, const float* logits, double* z);
int orc_dispatch(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_pos);
int orc_capacity(int T, int E, int k, double cf);
int orc_dispatch_capacity(int T, int E, int k, int capacity, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* dropped);
int orc_capacity_fallback(int T, int E, int k, int capacity, int fallback_min,
                          const int32_t* idx, const float* w, int32_t* idx_out, float* w_out,
                          int32_t* dropped);
int orc_expert_rows(int H, int I, int dtype, const void* x, const void* wg, const void* wu,
                    const void* wd, int n, const int32_t* tok, const int32_t* ex, int round_h,
                    double* y);
int orc_dequant_w4(int E, int N, int K, const uint8_t* codes, const uint16_t* sb, double* w);
int orc_expert_rows_w4(int H, int I, int dtype, const void* x, const uint8_t* cg,
                       const uint16_t* sg, const uint8_t* cu, const uint16_t* su,
                       const uint8_t* cd, const uint16_t* sd, int n, const int32_t* tok,
                       const int32_t* ex, int round_h, double* y);
int orc_expert_rows_f64w(int H, int I, int dtype, const void* x, const double* wg,
                         const double* wu, const double* wd, int n, const int32_t* tok,
                         const int32_t* ex, double* y);
int orc_combine_kept(int T, int H, int k, const double* w, const double* y_pair,
                     const int8_t* keep, double* out);
int orc_combine(int T, int H, int k, const double* w, const double* y_pair, double* out);
int orc_aux(int T, int E, int k, const int32_t* counts, const double* probs, double* f,
            double* P, double* aux);
int orc_forward_tokens(int T, int H, int E, int k, int I, int norm, int dtype, const void* x,
                       const void* wr, const float* bias, const void* wg, const void* wu,
                       const void* wd, int n, const int32_t* tokens, const int32_t* forced_idx,
                       const int8_t* keep, int round_h, float* logits, int32_t* idx, double* w,
                       double* out);

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

/* xorshift64: the driver's own input bits (no arithmetic of the method) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static float uniform(float lo, float hi) {
  return lo + (hi - lo) * (float)((next_u64() >> 11) * (1.0 / 9007199254740992.0));
}
static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* arrays of n elements of dtype (0 fp32, 1 bf16 bits) with values in [lo, hi] */
static void* make(int dtype, size_t n, float lo, float hi) {
  if (dtype == 0) {
    float* a = malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) a[i] = uniform(lo, hi);
    return a;
  }
  uint16_t* a = malloc(sizeof(uint16_t) * n);
  for (size_t i = 0; i < n; ++i) a[i] = bf16_bits(uniform(lo, hi));
  return a;
}

static void run_block(int dtype, int T, int H, int E, int k, int I) {
  const size_t P = (size_t)T * k;
  void* x = make(dtype, (size_t)T * H, -1.0f, 1.0f);
  void* wr = make(dtype, (size_t)E * H, -0.1f, 0.1f);
  void* wg = make(dtype, (size_t)E * I * H, -0.05f, 0.05f);
  void* wu = make(dtype, (size_t)E * I * H, -0.05f, 0.05f);
  void* wd = make(dtype, (size_t)E * H * I, -0.05f, 0.05f);
  float* bias = malloc(sizeof(float) * E);
  for (int e = 0; e < E; ++e) bias[e] = uniform(-0.5f, 0.5f);
  float* logits = malloc(sizeof(float) * T * E);
  float* nlogits = malloc(sizeof(float) * T * E);
  float* noise = malloc(sizeof(float) * T * E);
  float* noisy = malloc(sizeof(float) * T * E);
  int32_t* idx = malloc(sizeof(int32_t) * P);
  int32_t* forced = malloc(sizeof(int32_t) * P);
  double* w = malloc(sizeof(double) * P);
  double* probs = malloc(sizeof(double) * T * E);
  int32_t* kt = malloc(sizeof(int32_t) * T);
  double* xk = malloc(sizeof(double) * T);
  int32_t* counts = malloc(sizeof(int32_t) * E);
  int32_t* offsets = malloc(sizeof(int32_t) * (E + 1));
  int32_t* sorted_pair = malloc(sizeof(int32_t) * P);
  int32_t* pair_pos = malloc(sizeof(int32_t) * P);
  int32_t* tok = malloc(sizeof(int32_t) * P);
  int32_t* ex = malloc(sizeof(int32_t) * P);
  int8_t* keep = malloc(P);
  double* y = malloc(sizeof(double) * P * H);
  double* out = malloc(sizeof(double) * T * H);
  double* f = malloc(sizeof(double) * E);  /* exact sizes: an overrun is a heap error */
  double* Pe = malloc(sizeof(double) * E);
  double aux, z;
  int32_t dropped = 0;

  expect(orc_logits(T, H, E, dtype, x, wr, bias, logits), 0, "logits");
  expect(orc_logits(T, H, E, dtype, x, wr, NULL, logits), 0, "logits (no bias)");
  expect(orc_route(T, E, k, 1, logits, NULL, idx, w, probs), 0, "route");
  for (int t = 0; t < T; ++t)  /* distinct experts per token for the forced set */
    for (int j = 0; j < k; ++j) forced[(size_t)t * k + j] = (t + j) % E;
  expect(orc_route(T, E, k, 0, logits, forced, idx, w, NULL), 0, "route (forced)");
  expect(orc_route_sel(T, E, k, 1, logits, bias, NULL, idx, w, probs), 0, "route_sel");
  expect(orc_route_dynamic(T, E, k, 1, 1, logits, idx, w, kt, xk), 0, "route_dynamic");
  expect(orc_dispatch(T, E, k, idx, counts, offsets, sorted_pair, pair_pos), 0,
         "dispatch (empty slots)");
  for (int i = 0; i < T * E; ++i) {
    nlogits[i] = uniform(-3.0f, 3.0f);
    noise[i] = uniform(-2.0f, 2.0f);
  }
  expect(orc_noisy_logits(T, E, logits, nlogits, noise, noisy), 0, "noisy_logits");
  expect(orc_z_loss(T, E, logits, &z), 0, "z_loss");
  expect(orc_route(T, E, k, 1, logits, NULL, idx, w, probs), 0, "route");
  expect(orc_dispatch(T, E, k, idx, counts, offsets, sorted_pair, pair_pos), 0, "dispatch");
  expect(orc_aux(T, E, k, counts, probs, f, Pe, &aux), 0, "aux");
  const int cap = orc_capacity(T, E, k, 0.5);
  if (cap < 1) expect(cap, 1, "capacity >= 1");
  expect(orc_dispatch_capacity(T, E, k, cap, idx, counts, offsets, sorted_pair, pair_pos,
                               &dropped),
         0, "dispatch_capacity");
  {
    /* fallback routing, exact-size buffers (with one empty slot) */
    int32_t* fi = malloc(sizeof(int32_t) * P);
    int32_t* fo = malloc(sizeof(int32_t) * P);
    float* fw = malloc(sizeof(float) * P);
    float* fwo = malloc(sizeof(float) * P);
    for (size_t i = 0; i < P; ++i) {
      fi[i] = idx[i];
      fw[i] = (float)w[i];
    }
    fi[P - 1] = -1;
    int32_t fdrop = 0;
    expect(orc_capacity_fallback(T, E, k, cap, k, fi, fw, fo, fwo, &fdrop), 0,
           "capacity_fallback");
    expect(orc_capacity_fallback(T, E, k, cap, k + 1, fi, fw, fo, fwo, &fdrop), -1,
           "capacity_fallback fallback_min > k");
    free(fi);
    free(fo);
    free(fw);
    free(fwo);
  }
  for (size_t i = 0; i < P; ++i) {
    tok[i] = (int32_t)(i / k);
    ex[i] = idx[i];
    keep[i] = (int8_t)(pair_pos[i] >= 0);
  }
  expect(orc_expert_rows(H, I, dtype, x, wg, wu, wd, (int)P, tok, ex, 1, y), 0, "expert_rows");
  expect(orc_combine(T, H, k, w, y, out), 0, "combine");
  expect(orc_combine_kept(T, H, k, w, y, keep, out), 0, "combine_kept");
  {
    double* wgd = malloc(sizeof(double) * E * I * H);
    double* wud = malloc(sizeof(double) * E * I * H);
    double* wdd = malloc(sizeof(double) * E * H * I);
    for (size_t i = 0; i < (size_t)E * I * H; ++i) {
      wgd[i] = uniform(-0.05f, 0.05f);
      wud[i] = uniform(-0.05f, 0.05f);
      wdd[i] = uniform(-0.05f, 0.05f);
    }
    expect(orc_expert_rows_f64w(H, I, dtype, x, wgd, wud, wdd, (int)P, tok, ex, y), 0,
           "expert_rows_f64w");
    free(wgd);
    free(wud);
    free(wdd);
  }
  {
    const int n = T / 2 + 1;
    int32_t* tokens = malloc(sizeof(int32_t) * n);
    for (int i = 0; i < n; ++i) tokens[i] = (i * 5) % T;
    float* lg = malloc(sizeof(float) * n * E);
    int32_t* id = malloc(sizeof(int32_t) * n * k);
    double* ww = malloc(sizeof(double) * n * k);
    double* o = malloc(sizeof(double) * n * H);
    expect(orc_forward_tokens(T, H, E, k, I, 1, dtype, x, wr, bias, wg, wu, wd, n, tokens, NULL,
                              NULL, 1, lg, id, ww, o),
           0, "forward_tokens");
    expect(orc_forward_tokens(T, H, E, k, I, 0, dtype, x, wr, NULL, wg, wu, wd, n, tokens,
                              forced, keep, 0, lg, id, ww, o),
           0, "forward_tokens (forced, keep)");
    free(tokens);
    free(lg);
    free(id);
    free(ww);
    free(o);
  }
  /* bad arguments are rejected, nothing is touched */
  expect(orc_logits(T, 0, E, dtype, x, wr, NULL, logits), -1, "logits H < 1");
  expect(orc_route(T, E, E + 1, 1, logits, NULL, idx, w, probs), -1, "route k > E");
  expect(orc_dispatch(T, E, k, NULL, counts, offsets, sorted_pair, pair_pos), -1,
         "dispatch NULL");
  expect(orc_dispatch_capacity(T, E, k, 0, idx, counts, offsets, sorted_pair, pair_pos,
                               &dropped),
         -1, "dispatch_capacity capacity < 1");
  expect(orc_route_dynamic(T, 1, 1, 1, 1, logits, idx, w, kt, xk), -1, "route_dynamic E < 2");

  free(x); free(wr); free(wg); free(wu); free(wd); free(bias); free(logits); free(nlogits);
  free(noise); free(noisy); free(idx); free(forced); free(w); free(probs); free(kt); free(xk);
  free(counts); free(offsets); free(sorted_pair); free(pair_pos); free(tok); free(ex);
  free(keep); free(y); free(out); free(f); free(Pe);
}

static void run_w4(int T, int H, int E, int k, int I) {
  const size_t P = (size_t)T * k;
  uint16_t* x = make(1, (size_t)T * H, -1.0f, 1.0f);
  const size_t cgate = (size_t)E * I * H / 2, cdown = (size_t)E * H * I / 2;
  uint8_t* cg = malloc(cgate);
  uint8_t* cu = malloc(cgate);
  uint8_t* cd = malloc(cdown);
  for (size_t i = 0; i < cgate; ++i) {
    cg[i] = (uint8_t)next_u64();
    cu[i] = (uint8_t)next_u64();
  }
  for (size_t i = 0; i < cdown; ++i) cd[i] = (uint8_t)next_u64();
  const size_t sgate = (size_t)E * I * (H / 128) * 2, sdown = (size_t)E * H * (I / 128) * 2;
  uint16_t* sg = make(1, sgate, 0.001f, 0.01f);
  uint16_t* su = make(1, sgate, 0.001f, 0.01f);
  uint16_t* sd = make(1, sdown, 0.001f, 0.01f);
  double* wdq = malloc(sizeof(double) * E * I * H);
  int32_t* tok = malloc(sizeof(int32_t) * P);
  int32_t* ex = malloc(sizeof(int32_t) * P);
  double* y = malloc(sizeof(double) * P * H);
  for (size_t i = 0; i < P; ++i) {
    tok[i] = (int32_t)(i / k);
    ex[i] = (int32_t)((i * 3) % E);
  }
  expect(orc_dequant_w4(E, I, H, cg, sg, wdq), 0, "dequant_w4");
  expect(orc_expert_rows_w4(H, I, 1, x, cg, sg, cu, su, cd, sd, (int)P, tok, ex, 1, y), 0,
         "expert_rows_w4");
  expect(orc_dequant_w4(E, I, 100, cg, sg, wdq), -1, "dequant_w4 K % 128");
  free(x); free(cg); free(cu); free(cd); free(sg); free(su); free(sd); free(wdq); free(tok);
  free(ex); free(y);
}

int main(void) {
  run_block(0, 37, 64, 8, 3, 128);
  run_block(1, 37, 64, 8, 3, 128);
  run_block(1, 1, 64, 4, 4, 64);   /* one token, k = E */
  run_block(1, 50, 128, 16, 1, 64);  /* k = 1 */
  run_w4(9, 256, 4, 2, 128);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle driver: all calls ok\n");
  return 0;
}
