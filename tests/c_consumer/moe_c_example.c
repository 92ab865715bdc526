/* moe_c_example.c: the block forward driven from plain C through the library's
 * C ABI (include/moe.h), with no Python and no torch in the process. It uses
 * only the HIP runtime for memory: hipMalloc'd buffers and workspace, the
 * null stream, one hipDeviceSynchronize at the end.
 *
 * Usage: moe_c_example IN OUT
 *   IN : int32 header {T, H, E, k, I, norm_topk_prob, dtype, has_logit_bias},
 *        then x [T,H], w_router [E,H], w_gate [E,I,H], w_up [E,I,H],
 *        w_down [E,H,I] as raw elements of dtype (bf16 bit patterns or fp32),
 *        then logit_bias [E] fp32 when has_logit_bias is 1.
 *   OUT: out [T,H] (dtype), topk_idx [T,k] int32, topk_w [T,k] fp32,
 *        counts [E] int32, f [E] fp32, P [E] fp32, aux [1] fp32.
 * Exits 0 on success; prints the failing call and its status otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      return 2;                                                             \
    }                                                                       \
  } while (0)

/* n bytes from f into a new device buffer */
static void* upload(FILE* f, size_t n) {
  void* h = malloc(n ? n : 1);
  void* d = NULL;
  if (!h) return NULL;
  if (fread(h, 1, n, f) != n || hipMalloc(&d, n ? n : 1) != hipSuccess ||
      hipMemcpy(d, h, n, hipMemcpyHostToDevice) != hipSuccess) {
    free(h);
    if (d) (void)hipFree(d);
    return NULL;
  }
  free(h);
  return d;
}

static int download(FILE* f, const void* d, size_t n) {
  void* h = malloc(n ? n : 1);
  if (!h) return 1;
  if (hipMemcpy(h, d, n, hipMemcpyDeviceToHost) != hipSuccess || fwrite(h, 1, n, f) != n) {
    free(h);
    return 1;
  }
  free(h);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hd[8];
  if (fread(hd, sizeof hd, 1, in) != 1) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  moe_config c;
  c.num_tokens = hd[0];
  c.hidden = hd[1];
  c.num_experts = hd[2];
  c.top_k = hd[3];
  c.intermediate = hd[4];
  c.norm_topk_prob = hd[5];
  c.dtype = (moe_dtype)hd[6];
  const size_t T = (size_t)hd[0], H = (size_t)hd[1], E = (size_t)hd[2], k = (size_t)hd[3],
               I = (size_t)hd[4];
  const size_t es = c.dtype == MOE_DTYPE_BF16 ? 2 : 4;

  void* x = upload(in, T * H * es);
  void* wr = upload(in, E * H * es);
  void* wg = upload(in, E * I * H * es);
  void* wu = upload(in, E * I * H * es);
  void* wd = upload(in, E * H * I * es);
  float* bias = hd[7] ? (float*)upload(in, E * sizeof(float)) : NULL;
  fclose(in);
  if (!x || !wr || !wg || !wu || !wd || (hd[7] && !bias)) {
    fprintf(stderr, "reading or uploading the inputs failed\n");
    return 1;
  }

  void *out, *ws;
  int32_t *idx, *counts;
  float *w, *f, *P, *aux;
  HIP_OK(hipMalloc(&out, T * H * es));
  HIP_OK(hipMalloc((void**)&idx, T * k * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&w, T * k * sizeof(float)));
  HIP_OK(hipMalloc((void**)&counts, E * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&f, E * sizeof(float)));
  HIP_OK(hipMalloc((void**)&P, E * sizeof(float)));
  HIP_OK(hipMalloc((void**)&aux, sizeof(float)));
  const size_t wsb = moe_workspace_size(&c);
  if (wsb == 0) {
    fprintf(stderr, "moe_workspace_size: configuration rejected\n");
    return 1;
  }
  HIP_OK(hipMalloc(&ws, wsb));

  moe_aux_out ao;
  ao.counts = counts;
  ao.f = f;
  ao.P = P;
  ao.aux = aux;
  /* the null stream: the library enqueues on whatever stream it is given */
  const moe_status st = moe_layer_forward(&c, x, wr, bias, wg, wu, wd, out, NULL, idx, w, ao,
                                          ws, wsb, (hipStream_t)0);
  if (st != MOE_OK) {
    fprintf(stderr, "moe_layer_forward: %s\n", moe_status_string(st));
    return 3;
  }
  HIP_OK(hipDeviceSynchronize());

  FILE* o = fopen(argv[2], "wb");
  if (!o) {
    perror(argv[2]);
    return 1;
  }
  if (download(o, out, T * H * es) || download(o, idx, T * k * 4) || download(o, w, T * k * 4) ||
      download(o, counts, E * 4) || download(o, f, E * 4) || download(o, P, E * 4) ||
      download(o, aux, 4)) {
    fprintf(stderr, "writing the outputs failed\n");
    return 1;
  }
  fclose(o);
  void* bufs[] = {x, wr, wg, wu, wd, bias, out, idx, w, counts, f, P, aux, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  printf("moe_c_example: T=%zu H=%zu E=%zu k=%zu I=%zu dtype=%s workspace=%zu bytes: ok\n", T, H,
         E, k, I, c.dtype == MOE_DTYPE_BF16 ? "bf16" : "f32", wsb);
  return 0;
}
