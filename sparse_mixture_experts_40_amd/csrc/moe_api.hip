// moe_api.hip — the C ABI of include/moe.h: argument checks, workspace
// carving and the launch sequence on the caller's stream. No allocation, no
// host synchronisation. The only global state is the per-device address of
// the no-allocation entry point's scratch array (looked up once per device).
#include <string.h>

#include <atomic>
#include <cmath>

#include "aux_small.h"

using namespace moe;

// Scratch of moe_layer_forward_noalloc, for callers that cannot allocate:
// one copy per GPU, in the library's device code object. In host code this
// name is a host-side stand-in, never a device address: the host uses only
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// Per device: the device address of `scratch` (null until the first
// moe_layer_forward_noalloc call on that device looks it up).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

moe_status noalloc_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();  // leave no error behind for the next launch check
      return MOE_ERR_HIP;
    }
    g_scratch_addr[dev].store(p, std::memory_order_release);  // same value from any thread
  }
  *addr = p;
  return MOE_OK;
}

constexpr size_t kAlign = 256;

// Bump carver over the caller's workspace (base == nullptr: size only).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) & ~(kAlign - 1);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

size_t elem_bytes(const moe_config& c) { return c.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

moe_status check_config(const moe_config* cfg) {
  if (!cfg) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = *cfg;
  if (c.num_tokens < 1 || c.hidden < 1 || c.num_experts < 1 || c.top_k < 1 ||
      c.intermediate < 1 || c.top_k > c.num_experts)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c.dtype != MOE_DTYPE_F32 && c.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (c.norm_topk_prob != 0 && c.norm_topk_prob != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c.num_experts > 256 || c.top_k > 16) return MOE_ERR_UNSUPPORTED;
  if (c.hidden % 64 != 0 || c.intermediate % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const long long P = (long long)c.num_tokens * c.top_k;
  const long long wide = c.hidden > c.intermediate ? c.hidden : c.intermediate;
  if (P >= (1LL << 31) || P * wide >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long long)c.num_experts * c.intermediate * c.hidden >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  // one expert's matrix, and the router matrix, are addressed with 32-bit
  // byte offsets
  if ((long long)c.intermediate * c.hidden >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long long)c.num_experts * c.hidden >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Router fields of moe_options against the configuration.
moe_status check_router_options(const moe_config& c, const moe_options& o) {
  if ((o.noise != nullptr) != (o.w_noise != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (o.dynamic_k_min < 0 || o.dynamic_k_min > c.top_k) return MOE_ERR_INVALID_ARGUMENT;
  if (o.dynamic_k_min > 0 && c.num_experts < 2) return MOE_ERR_INVALID_ARGUMENT;
  if (o.dynamic_k_min > 0 && o.select_bias) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Workspace regions. Each entry point carves the prefix it needs, in order.
struct Layout {
  int32_t* hist;
  int32_t* base;
  float* partials;
  double* fp;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* idx;
  float* w;
  float* rpart;   // split-K router partials [splits, T, E]
  float* rlogits; // router logits [T, E] (split-K or noisy routing)
  float* nlogits; // noise logits x W_noise^T [T, E]
  float* zpart;   // per router block z-loss sums
  void* h;
  void* y;
  int32_t* fb_idx;    // routing after the least-loaded fallback [T, k]
  float* fb_w;        // its weights [T, k]
  int32_t* fb_counts; // rows per expert of that routing [E]
  size_t dispatch_end, aux_end, router_end, layer_end;
};

Layout carve(const moe_config& c, void* ws) {
  Carver cv(ws);
  Layout L{};
  const size_t P = (size_t)c.num_tokens * c.top_k, E = c.num_experts;
  L.hist = cv.take<int32_t>((size_t)dispatch_num_chunks(c) * E);
  L.base = cv.take<int32_t>((size_t)dispatch_num_chunks(c) * E);
  L.dispatch_end = cv.off;
  L.partials = cv.take<float>((size_t)router_num_blocks(c, true) * E);  // the larger count
  L.fp = cv.take<double>(E);
  L.counts = cv.take<int32_t>(E);
  L.offsets = cv.take<int32_t>(E + 1);
  L.idx = cv.take<int32_t>(P);
  L.w = cv.take<float>(P);
  L.zpart = cv.take<float>((size_t)router_num_blocks(c, true));  // the larger count
  L.aux_end = cv.off;
  const int ks = router_k_splits(c);
  L.rpart = ks > 1 ? cv.take<float>((size_t)ks * c.num_tokens * E) : nullptr;
  L.rlogits = cv.take<float>((size_t)c.num_tokens * E);
  L.nlogits = cv.take<float>((size_t)c.num_tokens * E);
  L.router_end = cv.off;
  L.sorted_pair = cv.take<int32_t>(P);
  L.pair_pos = cv.take<int32_t>(P);
  L.h = cv.take<char>(P * c.intermediate * elem_bytes(c));
  // y_sorted: fp32 rows, or (bf16 layers) scaled fp16 rows in the first half
  // and their int8 chunk exponents after them
  L.y = cv.take<float>(P * c.hidden);
  L.fb_idx = cv.take<int32_t>(P);
  L.fb_w = cv.take<float>(P);
  L.fb_counts = cv.take<int32_t>(E);
  L.layer_end = cv.off;
  return L;
}

// Logits x w^T (+ bias) into out: split-K for small token counts (part is
// the split-K scratch of the workspace), one pass otherwise.
hipError_t logits_any(const moe_config& c, const void* x, const void* w, const float* bias,
                      float* out, float* part, hipStream_t s) {
  if (router_k_splits(c) > 1) return launch_logits_split(c, x, w, bias, out, part, s);
  return launch_logits(c, x, w, bias, out, s);
}

// gate/up + down alone need only h
size_t swiglu_bytes(const moe_config& c) {
  Carver cv(nullptr);
  cv.take<char>((size_t)c.num_tokens * c.top_k * c.intermediate * elem_bytes(c));
  return cv.off;
}

// 4-bit weight arguments: all six arrays, bf16 activations, H and I
// multiples of 512.
moe_status check_w4(const moe_config& c, const moe_w4_weights* w) {
  if (!w || !w->gate || !w->up || !w->down || !w->gate_sb || !w->up_sb || !w->down_sb)
    return MOE_ERR_INVALID_ARGUMENT;
  return w4_supported(c) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// The block forward with either dtype expert weights (w_gate/w_up/w_down) or
// 4-bit ones (w4 != nullptr). Arguments are checked by the callers.
moe_status layer_forward_impl(const moe_config* cfg, const moe_options* opt, const void* x,
                              const void* w_router, const float* logit_bias, const void* w_gate,
                              const void* w_up, const void* w_down, const moe_w4_weights* w4,
                              void* out, float* router_logits, int32_t* topk_idx, float* topk_w,
                              moe_aux_out aux, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  moe_status st = MOE_OK;
  const moe_options none{};
  const moe_options& o = opt ? *opt : none;
  if (o.capacity < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (o.capacity_fallback_min < 0 || o.capacity_fallback_min > cfg->top_k ||
      (o.capacity_fallback_min > 0 && o.capacity == 0))
    return MOE_ERR_INVALID_ARGUMENT;
  st = check_router_options(*cfg, o);
  if (st != MOE_OK) return st;
  const Layout L = carve(*cfg, workspace);
  if (!workspace || workspace_bytes < L.layer_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_config& c = *cfg;
  int32_t* idx = topk_idx ? topk_idx : L.idx;
  float* w = topk_w ? topk_w : L.w;
  const AuxOut ao{aux.counts, aux.f, aux.P, aux.aux, o.z_loss};
  const bool want_aux = ao.counts || ao.f || ao.P || ao.aux;
  float* partials = want_aux ? L.partials : nullptr;
  RouterExtras ex;
  ex.sel_bias = o.select_bias;
  ex.zpart = ao.z_loss ? L.zpart : nullptr;
  ex.k_min = o.dynamic_k_min;
  ex.kt_out = o.k_per_token;

  int router_blocks;
  if (o.noise) {  // clean logits, noise logits, then the noisy top-k from them
    st = launched(logits_any(c, x, w_router, logit_bias, L.rlogits, L.rpart, stream));
    if (st != MOE_OK) return st;
    st = launched(logits_any(c, x, o.w_noise, nullptr, L.nlogits, L.rpart, stream));
    if (st != MOE_OK) return st;
    ex.noise = o.noise;
    ex.nlogits = L.nlogits;
    ex.logits_final = router_logits;
    st = launched(launch_router(c, nullptr, nullptr, nullptr, L.rlogits, false, idx, w, partials,
                                true, stream, ex));
    router_blocks = router_num_blocks(c, true);
  } else if (router_k_splits(c) > 1) {
    st = launched(launch_router_split(c, x, w_router, logit_bias, router_logits, L.rpart, idx, w,
                                      partials, stream, ex));
    router_blocks = router_num_blocks(c, true);
  } else {
    st = launched(launch_router(c, x, w_router, logit_bias, router_logits,
                                router_logits != nullptr, idx, w, partials, true, stream, ex));
    router_blocks = router_num_blocks(c, false);
  }
  if (st != MOE_OK) return st;
  // with the least-loaded fallback the first dispatch is dropless (it gives
  // the ranks and loads the fallback reads); the routing it makes is then
  // dispatched again
  const bool fallback = o.capacity_fallback_min > 0;
  const int cap1 = fallback ? 0 : o.capacity;
  int32_t* drop1 = o.dropped;  // with the fallback: 0 (no limit), the count starts there
  // with few router blocks and one dispatch chunk (decode batches) the
  // statistics come out of the dispatch block itself
  bool aux_done = false;
  // decode batches of one dispatch chunk: the gate/up kernel sorts the
  // routing itself, with the statistics in its second block, so no dispatch
  // launch sits between the router and it (with the fallback, the first
  // dispatch feeds the fallback kernel and keeps its launch)
  const bool sort_in_gemm = !fallback && !w4 && gate_up_sorts_itself(c);
  AuxSmallArgs sort_aux{};
  const AuxSmallArgs* sort_aux_p = nullptr;
  if (sort_in_gemm) {
    if ((want_aux || ao.z_loss) && aux_small_fits(c, router_blocks)) {
      sort_aux = aux_small_args(c, L.partials, router_blocks, ao, ex.zpart, router_blocks);
      sort_aux_p = &sort_aux;
      aux_done = true;
    }
  } else if ((want_aux || ao.z_loss) && aux_small_fits(c, router_blocks)) {
    st = launched(launch_dispatch_aux(
        c, idx, L.counts, L.offsets, L.sorted_pair, L.pair_pos, L.hist, L.base, cap1, drop1,
        aux_small_args(c, L.partials, router_blocks, ao, ex.zpart, router_blocks), &aux_done,
        stream));
  } else {
    st = launched(launch_dispatch(c, idx, L.counts, L.offsets, L.sorted_pair, L.pair_pos, L.hist,
                                  L.base, true, cap1, drop1, stream));
  }
  if (st != MOE_OK) return st;
  const float* wc = w;  // weights of the combine
  if (fallback) {
    st = launched(launch_capacity_fallback(c, idx, w, o.capacity, o.capacity_fallback_min,
                                           L.offsets, L.sorted_pair, L.pair_pos, L.fb_idx,
                                           L.fb_w, o.dropped, true, stream));
    if (st != MOE_OK) return st;
    st = launched(launch_dispatch(c, L.fb_idx, L.fb_counts, L.offsets, L.sorted_pair, L.pair_pos,
                                  L.hist, L.base, true, 0, nullptr, stream));
    if (st != MOE_OK) return st;
    wc = L.fb_w;
  }
  // bf16 layers keep y_sorted in scaled fp16 where the tiled down kernel
  // writes it (half the bytes between the down GEMM and the combine): the
  // rows in the first half of L.y, their chunk exponents after them
  int8_t* y_exp = nullptr;
  bool y_half = false;
  if (c.dtype == MOE_DTYPE_BF16 && !w4 && combine_half_fits(c))
    y_exp = reinterpret_cast<int8_t*>(L.y) + (size_t)c.num_tokens * c.top_k * c.hidden * 2;
  if (w4) {
    st = launched(launch_gate_up_w4(c, x, L.sorted_pair, L.offsets, *w4, L.h, stream));
    if (st != MOE_OK) return st;
    st = launched(launch_down_w4(c, L.h, L.offsets, *w4, L.y, stream));
  } else {
    if (sort_in_gemm)
      st = launched(launch_gate_up_sorting(c, x, idx, cap1, L.counts, L.offsets, L.sorted_pair,
                                           L.pair_pos, drop1, sort_aux_p, w_gate, w_up, L.h,
                                           stream));
    else
      st = launched(launch_gate_up(c, x, L.sorted_pair, L.offsets, w_gate, w_up, L.h, stream));
    if (st != MOE_OK) return st;
    st = launched(launch_down(c, L.h, L.offsets, w_down, L.y, stream, y_exp, &y_half));
  }
  if (st != MOE_OK) return st;
  st = launched(launch_combine(c, L.y, L.pair_pos, wc, out, stream, y_half ? y_exp : nullptr));
  if (st != MOE_OK) return st;
  if ((want_aux || ao.z_loss) && !aux_done)
    st = launched(launch_aux(c, L.counts, L.partials, router_blocks, L.fp, ao, stream, ex.zpart,
                             router_blocks));
  return st;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return carve(*cfg, nullptr).layer_end;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_router_topk(const moe_config* cfg, const void* x, const void* w_router,
                           const float* logit_bias, float* logits, int32_t* topk_idx,
                           float* topk_w, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (x ? !w_router : !logits) return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_router(*cfg, x, w_router, x ? logit_bias : nullptr, logits,
                                logits != nullptr, topk_idx, topk_w, nullptr, true, stream));
}

moe_status moe_router_topk_ex(const moe_config* cfg, const moe_options* opt, const void* x,
                              const void* w_router, const float* logit_bias, float* logits,
                              int32_t* topk_idx, float* topk_w, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_options none{};
  const moe_options& o = opt ? *opt : none;
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (x ? !w_router : !logits) return MOE_ERR_INVALID_ARGUMENT;
  st = check_router_options(*cfg, o);
  if (st != MOE_OK) return st;
  if (o.noise && !x) return MOE_ERR_INVALID_ARGUMENT;
  RouterExtras ex;
  ex.sel_bias = o.select_bias;
  ex.k_min = o.dynamic_k_min;
  ex.kt_out = o.k_per_token;
  const Layout L = carve(*cfg, workspace);
  const bool have_ws = workspace && workspace_bytes >= L.router_end;
  if (!o.noise) {
    if (x && have_ws && router_k_splits(*cfg) > 1)  // small T: split-K logits
      return launched(launch_router_split(*cfg, x, w_router, logit_bias, logits, L.rpart,
                                          topk_idx, topk_w, nullptr, stream, ex));
    return launched(launch_router(*cfg, x, w_router, x ? logit_bias : nullptr, logits,
                                  logits != nullptr, topk_idx, topk_w, nullptr, true, stream,
                                  ex));
  }
  if (!have_ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
  st = launched(logits_any(*cfg, x, w_router, logit_bias, L.rlogits, L.rpart, stream));
  if (st != MOE_OK) return st;
  st = launched(logits_any(*cfg, x, o.w_noise, nullptr, L.nlogits, L.rpart, stream));
  if (st != MOE_OK) return st;
  ex.noise = o.noise;
  ex.nlogits = L.nlogits;
  ex.logits_final = logits;
  return launched(launch_router(*cfg, nullptr, nullptr, nullptr, L.rlogits, false, topk_idx,
                                topk_w, nullptr, true, stream, ex));
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!topk_idx || !expert_counts || !expert_offsets || !sorted_pair || !pair_pos)
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = carve(*cfg, workspace);
  if (!workspace || workspace_bytes < L.dispatch_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return launched(launch_dispatch(*cfg, topk_idx, expert_counts, expert_offsets, sorted_pair,
                                  pair_pos, L.hist, L.base, true, 0, nullptr, stream));
}

int32_t moe_capacity(const moe_config* cfg, float capacity_factor) {
  if (check_config(cfg) != MOE_OK || !(capacity_factor > 0.0f)) return 0;
  const double pairs = (double)cfg->num_tokens * (double)cfg->top_k;
  double c = ceil(pairs * (double)capacity_factor / (double)cfg->num_experts);
  if (c < 1.0) c = 1.0;
  if (c > pairs) c = pairs;
  return (int32_t)c;
}

moe_status moe_dispatch_capacity(const moe_config* cfg, const int32_t* topk_idx,
                                 int32_t capacity, int32_t* expert_counts,
                                 int32_t* expert_offsets, int32_t* sorted_pair,
                                 int32_t* pair_pos, int32_t* dropped, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!topk_idx || !expert_counts || !expert_offsets || !sorted_pair || !pair_pos ||
      capacity < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = carve(*cfg, workspace);
  if (!workspace || workspace_bytes < L.dispatch_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return launched(launch_dispatch(*cfg, topk_idx, expert_counts, expert_offsets, sorted_pair,
                                  pair_pos, L.hist, L.base, true, capacity, dropped, stream));
}

moe_status moe_capacity_fallback(const moe_config* cfg, const int32_t* topk_idx,
                                 const float* topk_w, int32_t capacity, int32_t fallback_min,
                                 const int32_t* expert_offsets, const int32_t* sorted_pair,
                                 const int32_t* pair_pos, int32_t* topk_idx_out,
                                 float* topk_w_out, int32_t* dropped, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!topk_idx || !topk_w || !expert_offsets || !sorted_pair || !pair_pos || !topk_idx_out ||
      !topk_w_out || capacity < 1 || fallback_min < 0 || fallback_min > cfg->top_k)
    return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_capacity_fallback(*cfg, topk_idx, topk_w, capacity, fallback_min,
                                           expert_offsets, sorted_pair, pair_pos, topk_idx_out,
                                           topk_w_out, dropped, false, stream));
}

moe_status moe_expert_gate_up(const moe_config* cfg, const void* x, const int32_t* sorted_pair,
                              const int32_t* expert_offsets, const void* w_gate,
                              const void* w_up, void* h, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !sorted_pair || !expert_offsets || !w_gate || !w_up || !h)
    return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_gate_up(*cfg, x, sorted_pair, expert_offsets, w_gate, w_up, h, stream));
}

moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                           const void* w_down, void* y_sorted, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !w_down || !y_sorted) return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_down(*cfg, h, expert_offsets, w_down, y_sorted, stream));
}

moe_status moe_expert_swiglu(const moe_config* cfg, const void* x, const int32_t* sorted_pair,
                             const int32_t* expert_offsets, const void* w_gate,
                             const void* w_up, const void* w_down, void* y_sorted,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !sorted_pair || !expert_offsets || !w_gate || !w_up || !w_down || !y_sorted)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < swiglu_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  st = launched(launch_gate_up(*cfg, x, sorted_pair, expert_offsets, w_gate, w_up, workspace,
                               stream));
  if (st != MOE_OK) return st;
  return launched(launch_down(*cfg, workspace, expert_offsets, w_down, y_sorted, stream));
}

moe_status moe_combine(const moe_config* cfg, const void* y_sorted, const int32_t* pair_pos,
                       const float* topk_w, void* out, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!y_sorted || !pair_pos || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_combine(*cfg, y_sorted, pair_pos, topk_w, out, stream));
}

moe_status moe_aux_stats(const moe_config* cfg, const float* logits, const int32_t* topk_idx,
                         moe_aux_out out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = carve(*cfg, workspace);
  if (!workspace || workspace_bytes < L.aux_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!out.counts && !out.f && !out.P && !out.aux) return MOE_OK;
  // per-block softmax sums from the logits (selection skipped)
  st = launched(launch_router(*cfg, nullptr, nullptr, nullptr, const_cast<float*>(logits), false,
                              L.idx, L.w, L.partials, false, stream));
  if (st != MOE_OK) return st;
  // expert counts from the given selection (histogram + scan only)
  st = launched(launch_dispatch(*cfg, topk_idx, L.counts, L.offsets, nullptr, nullptr, L.hist,
                                nullptr, false, 0, nullptr, stream));
  if (st != MOE_OK) return st;
  const int nb = router_num_blocks(*cfg, true);
  const AuxOut ao{out.counts, out.f, out.P, out.aux, nullptr};
  return launched(launch_aux(*cfg, L.counts, L.partials, nb, L.fp, ao, stream));
}

moe_status moe_z_loss(const moe_config* cfg, const float* logits, float* z_loss,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!logits || !z_loss) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = carve(*cfg, workspace);
  if (!workspace || workspace_bytes < L.aux_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  // per-block sums of (ln sum_e exp l)^2 from the logits (selection skipped),
  // then their fixed-order total
  RouterExtras ex;
  ex.zpart = L.zpart;
  st = launched(launch_router(*cfg, nullptr, nullptr, nullptr, const_cast<float*>(logits), false,
                              L.idx, L.w, nullptr, false, stream, ex));
  if (st != MOE_OK) return st;
  const int nb = router_num_blocks(*cfg, true);
  AuxOut ao;
  ao.z_loss = z_loss;
  return launched(launch_aux(*cfg, L.counts, L.partials, nb, L.fp, ao, stream, L.zpart, nb));
}

moe_status moe_layer_forward_ex(const moe_config* cfg, const moe_options* opt, const void* x,
                                const void* w_router, const float* logit_bias,
                                const void* w_gate, const void* w_up, const void* w_down,
                                void* out, float* router_logits, int32_t* topk_idx,
                                float* topk_w, moe_aux_out aux, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return MOE_ERR_INVALID_ARGUMENT;
  return layer_forward_impl(cfg, opt, x, w_router, logit_bias, w_gate, w_up, w_down, nullptr,
                            out, router_logits, topk_idx, topk_w, aux, workspace,
                            workspace_bytes, stream);
}

moe_status moe_layer_forward_w4(const moe_config* cfg, const moe_options* opt, const void* x,
                                const void* w_router, const float* logit_bias,
                                const moe_w4_weights* w, void* out, float* router_logits,
                                int32_t* topk_idx, float* topk_w, moe_aux_out aux,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_w4(*cfg, w);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !out) return MOE_ERR_INVALID_ARGUMENT;
  return layer_forward_impl(cfg, opt, x, w_router, logit_bias, nullptr, nullptr, nullptr, w, out,
                            router_logits, topk_idx, topk_w, aux, workspace, workspace_bytes,
                            stream);
}

moe_status moe_expert_gate_up_w4(const moe_config* cfg, const void* x,
                                 const int32_t* sorted_pair, const int32_t* expert_offsets,
                                 const moe_w4_weights* w, void* h, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_w4(*cfg, w);
  if (st != MOE_OK) return st;
  if (!x || !sorted_pair || !expert_offsets || !h) return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_gate_up_w4(*cfg, x, sorted_pair, expert_offsets, *w, h, stream));
}

moe_status moe_expert_down_w4(const moe_config* cfg, const void* h,
                              const int32_t* expert_offsets, const moe_w4_weights* w,
                              void* y_sorted, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_w4(*cfg, w);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !y_sorted) return MOE_ERR_INVALID_ARGUMENT;
  return launched(launch_down_w4(*cfg, h, expert_offsets, *w, y_sorted, stream));
}

moe_status moe_w4_from_mlx(int E, int N, int K, const uint32_t* mlx_w,
                           const uint16_t* mlx_scales, const uint16_t* mlx_biases,
                           uint8_t* codes, uint16_t* sb) {
  if (!mlx_w || !mlx_scales || !mlx_biases || !codes || !sb || E < 1 || N < 1 || K < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  if (N % 32 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const size_t NB = (size_t)N / 32, KC = (size_t)K / 64, KG = (size_t)K / 128;
  for (size_t e = 0; e < (size_t)E; ++e)
    for (size_t n = 0; n < (size_t)N; ++n) {
      const size_t row = e * N + n, b = e * NB + n / 32, r = n % 32;
      // codes: MLX word w holds elements 8w .. 8w + 7 at nibbles 0..7; the
      // tiled word of those 8 elements holds element j (j < 4) in the low and
      // element j + 4 in the high nibble of byte j
      for (size_t w = 0; w < (size_t)K / 8; ++w) {
        const uint32_t u = mlx_w[row * (K / 8) + w];
        uint8_t* dst = codes + (b * KC + w / 8) * 1024 + r * 32 + 4 * (w % 8);
        for (int j = 0; j < 4; ++j)
          dst[j] = (uint8_t)(((u >> (4 * j)) & 15u) | (((u >> (16 + 4 * j)) & 15u) << 4));
      }
      for (size_t g = 0; g < KG; ++g) {
        uint16_t* d = sb + ((b * KG + g) * 32 + r) * 2;
        d[0] = mlx_scales[row * KG + g];
        d[1] = mlx_biases[row * KG + g];
      }
    }
  return MOE_OK;
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                     const float* logit_bias, const void* w_gate,
                                     const void* w_up, const void* w_down, void* out,
                                     float* router_logits, int32_t* topk_idx, float* topk_w,
                                     moe_aux_out aux, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (carve(*cfg, nullptr).layer_end > MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MOE_OK) return st;
  return layer_forward_impl(cfg, nullptr, x, w_router, logit_bias, w_gate, w_up, w_down, nullptr,
                            out, router_logits, topk_idx, topk_w, aux, ws,
                            MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* logit_bias, const void* w_gate, const void* w_up,
                             const void* w_down, void* out, float* router_logits,
                             int32_t* topk_idx, float* topk_w, moe_aux_out aux,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_layer_forward_ex(cfg, nullptr, x, w_router, logit_bias, w_gate, w_up, w_down, out,
                              router_logits, topk_idx, topk_w, aux, workspace, workspace_bytes,
                              stream);
}

}  // extern "C"
