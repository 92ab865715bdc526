// host_driver.cpp — the library's host code under AddressSanitizer +
// UndefinedBehaviorSanitizer (tests/test_sanitize.py builds the library
// sources with -Xarch_host sanitizers and links this driver against them).
// It runs every path that returns before a launch: configuration and option
// validation, workspace sizing (the carve of every stage's buffers), the
// capacity helper, the null-pointer and small-workspace checks of every entry
// point, the no-allocation entry point's size check, and the host-only 4-bit
// layout converter. No kernel is launched and no GPU is needed. Exits
// non-zero on an unexpected status; the sanitizers abort on memory errors
// and undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe.h"

namespace {

int failures = 0;

void expect(long long got, long long want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: %lld, expected %lld\n", what, got, want);
    ++failures;
  }
}

moe_config cfg(int T, int H, int E, int k, int I, int norm, moe_dtype dt) {
  moe_config c;
  std::memset(&c, 0, sizeof c);
  c.num_tokens = T;
  c.hidden = H;
  c.num_experts = E;
  c.top_k = k;
  c.intermediate = I;
  c.norm_topk_prob = norm;
  c.dtype = dt;
  return c;
}

// Every entry point with a valid configuration but a NULL required pointer,
// a NULL configuration, an invalid configuration, and (where it takes one)
// too small a workspace. Pointers passed are never dereferenced on these
// paths; `d` stands for any device buffer.
void entry_point_checks(const moe_config& c) {
  void* d = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  const auto* di = static_cast<const int32_t*>(d);
  auto* dio = static_cast<int32_t*>(d);
  const auto* df = static_cast<const float*>(d);
  auto* dfo = static_cast<float*>(d);
  const moe_aux_out no_aux{};
  const size_t ws = moe_workspace_size(&c);
  moe_config bad = c;
  bad.top_k = c.num_experts + 1;

  expect(moe_router_topk(nullptr, d, d, nullptr, nullptr, dio, dfo, nullptr), 1, "router NULL cfg");
  expect(moe_router_topk(&bad, d, d, nullptr, nullptr, dio, dfo, nullptr), 1, "router bad cfg");
  expect(moe_router_topk(&c, d, d, nullptr, nullptr, nullptr, dfo, nullptr), 1, "router NULL idx");
  expect(moe_router_topk(&c, d, nullptr, nullptr, nullptr, dio, dfo, nullptr), 1,
         "router NULL w_router");
  expect(moe_router_topk(&c, nullptr, nullptr, nullptr, nullptr, dio, dfo, nullptr), 1,
         "router NULL logits");
  moe_options o;
  std::memset(&o, 0, sizeof o);
  o.noise = df;  // noise without w_noise
  expect(moe_router_topk_ex(&c, &o, d, d, nullptr, nullptr, dio, dfo, d, ws, nullptr), 1,
         "router_ex noise without w_noise");
  std::memset(&o, 0, sizeof o);
  o.dynamic_k_min = c.top_k + 1;
  expect(moe_router_topk_ex(&c, &o, d, d, nullptr, nullptr, dio, dfo, d, ws, nullptr), 1,
         "router_ex k_min > k");
  std::memset(&o, 0, sizeof o);
  if (c.top_k > 1) {
    o.dynamic_k_min = 1;
    o.select_bias = df;
    expect(moe_router_topk_ex(&c, &o, d, d, nullptr, nullptr, dio, dfo, d, ws, nullptr), 2,
           "router_ex dynamic k with select_bias");
  }
  std::memset(&o, 0, sizeof o);
  o.capacity = -1;
  expect(moe_layer_forward_ex(&c, &o, d, d, nullptr, d, d, d, d, nullptr, nullptr, nullptr,
                              no_aux, d, ws, nullptr),
         1, "layer_ex negative capacity");
  std::memset(&o, 0, sizeof o);
  o.capacity_fallback_min = 1;  // fallback without a capacity
  expect(moe_layer_forward_ex(&c, &o, d, d, nullptr, d, d, d, d, nullptr, nullptr, nullptr,
                              no_aux, d, ws, nullptr),
         1, "layer_ex fallback without capacity");
  o.capacity = 4;
  o.capacity_fallback_min = c.top_k + 1;
  expect(moe_layer_forward_ex(&c, &o, d, d, nullptr, d, d, d, d, nullptr, nullptr, nullptr,
                              no_aux, d, ws, nullptr),
         1, "layer_ex fallback_min > k");
  expect(moe_capacity_fallback(&c, di, df, 0, 1, di, di, di, dio, dfo, nullptr, nullptr), 1,
         "capacity_fallback capacity 0");
  expect(moe_capacity_fallback(&c, di, df, 4, c.top_k + 1, di, di, di, dio, dfo, nullptr,
                               nullptr),
         1, "capacity_fallback fallback_min > k");
  expect(moe_capacity_fallback(&c, di, df, 4, 1, di, nullptr, di, dio, dfo, nullptr, nullptr), 1,
         "capacity_fallback NULL sorted_pair");

  expect(moe_dispatch(&c, nullptr, dio, dio, dio, dio, d, ws, nullptr), 1, "dispatch NULL idx");
  expect(moe_dispatch(&c, di, dio, dio, dio, dio, d, 1, nullptr), 3, "dispatch small ws");
  expect(moe_dispatch_capacity(&c, di, 0, dio, dio, dio, dio, dio, d, ws, nullptr), 1,
         "dispatch_capacity capacity 0");
  expect(moe_dispatch_capacity(&c, di, 1, dio, dio, dio, dio, dio, nullptr, ws, nullptr), 3,
         "dispatch_capacity NULL ws");
  expect(moe_expert_gate_up(&c, d, di, di, d, nullptr, d, d, ws, nullptr), 1, "gate_up NULL w_up");
  expect(moe_expert_down(&c, d, di, d, nullptr, d, ws, nullptr), 1, "down NULL y");
  expect(moe_expert_swiglu(&c, d, di, di, d, d, d, d, d, 1, nullptr), 3, "swiglu small ws");
  expect(moe_combine(&c, d, nullptr, df, d, nullptr), 1, "combine NULL pair_pos");
  expect(moe_combine(&bad, d, di, df, d, nullptr), 1, "combine bad cfg");
  expect(moe_aux_stats(&c, df, nullptr, no_aux, d, ws, nullptr), 1, "aux NULL idx");
  expect(moe_aux_stats(&c, df, di, no_aux, d, 8, nullptr), 3, "aux small ws");
  expect(moe_z_loss(&c, df, nullptr, d, ws, nullptr), 1, "z_loss NULL out");
  expect(moe_layer_forward(&c, d, d, nullptr, d, d, nullptr, d, nullptr, nullptr, nullptr,
                           no_aux, d, ws, nullptr),
         1, "layer NULL w_down");
  expect(moe_layer_forward(&c, d, d, nullptr, d, d, d, d, nullptr, nullptr, nullptr, no_aux, d,
                           ws - 1, nullptr),
         3, "layer small ws");
  expect(moe_layer_forward_noalloc(&c, nullptr, d, nullptr, d, d, d, d, nullptr, nullptr,
                                   nullptr, no_aux, nullptr),
         1, "noalloc NULL x");

  moe_w4_weights w4;
  std::memset(&w4, 0, sizeof w4);
  expect(moe_expert_gate_up_w4(&c, d, di, di, &w4, d, nullptr), 1, "gate_up_w4 NULL weights");
  w4.gate = w4.up = w4.down = static_cast<const uint8_t*>(d);
  w4.gate_sb = w4.up_sb = w4.down_sb = d;
  const bool w4_sizes = c.dtype == MOE_DTYPE_BF16 && c.hidden % 512 == 0 &&
                        c.intermediate % 512 == 0;
  if (!w4_sizes)
    expect(moe_expert_down_w4(&c, d, di, &w4, d, nullptr), 2, "down_w4 unsupported sizes");
  else
    expect(moe_expert_down_w4(&c, d, di, &w4, nullptr, nullptr), 1, "down_w4 NULL y");
  expect(moe_layer_forward_w4(&c, nullptr, d, d, nullptr, nullptr, d, nullptr, nullptr, nullptr,
                              no_aux, d, ws, nullptr),
         1, "layer_w4 NULL weights");
}

void workspace_and_capacity() {
  const moe_config shapes[] = {
      cfg(64, 128, 8, 2, 256, 1, MOE_DTYPE_F32),        // fp32 block
      cfg(4096, 4096, 8, 2, 14336, 0, MOE_DTYPE_BF16),  // 8 experts, top-2
      cfg(8192, 2048, 64, 8, 1024, 1, MOE_DTYPE_BF16),  // 64 experts, top-8
      cfg(16384, 4096, 128, 8, 1536, 1, MOE_DTYPE_BF16),
      cfg(64, 4096, 128, 8, 1536, 1, MOE_DTYPE_BF16),   // decode batch (split-K router)
      cfg(1, 64, 1, 1, 64, 1, MOE_DTYPE_BF16),          // smallest
      cfg(300, 128, 256, 16, 64, 1, MOE_DTYPE_BF16),    // E = 256, k = 16
      cfg(41, 192, 40, 3, 320, 0, MOE_DTYPE_BF16),      // odd sizes
  };
  for (const moe_config& c : shapes) {
    const size_t ws = moe_workspace_size(&c);
    if (ws == 0) expect(0, 1, "workspace size of a valid config");
    // h [P, I] and y_sorted [P, H] fp32 at least
    const size_t P = (size_t)c.num_tokens * c.top_k;
    const size_t eb = c.dtype == MOE_DTYPE_BF16 ? 2 : 4;
    if (ws < P * (c.intermediate * eb + c.hidden * 4)) expect(0, 1, "workspace holds h and y");
    for (float cf : {0.25f, 1.0f, 1.25f, 1000.0f}) {
      const int32_t cap = moe_capacity(&c, cf);
      if (cap < 1 || cap > (int32_t)P) expect(cap, 1, "capacity in [1, T*k]");
    }
    entry_point_checks(c);
  }
  // invalid configurations size to 0
  expect((long long)moe_workspace_size(nullptr), 0, "workspace NULL cfg");
  const moe_config bad[] = {
      cfg(0, 64, 8, 2, 64, 1, MOE_DTYPE_BF16), cfg(4, 96, 8, 2, 64, 1, MOE_DTYPE_BF16),
      cfg(4, 64, 300, 2, 64, 1, MOE_DTYPE_BF16), cfg(4, 64, 64, 17, 64, 1, MOE_DTYPE_BF16),
      cfg(1, 1 << 23, 256, 1, 64, 1, MOE_DTYPE_BF16)};
  for (const moe_config& c : bad) expect((long long)moe_workspace_size(&c), 0, "workspace bad");
  // the no-allocation forward rejects what its scratch cannot hold, before any launch
  const moe_config big = cfg(16384, 4096, 128, 8, 1536, 1, MOE_DTYPE_BF16);
  void* d = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  expect(moe_layer_forward_noalloc(&big, d, d, nullptr, d, d, d, d, nullptr, nullptr, nullptr,
                                   moe_aux_out{}, nullptr),
         3, "noalloc too large");
  for (int s = 0; s <= 7; ++s)  // 5..7: inside the enum's value range, unnamed
    if (!moe_status_string(static_cast<moe_status>(s))) expect(0, 1, "status string");
}

void w4_converter() {
  const int E = 2, N = 64, K = 256;
  std::vector<uint32_t> w((size_t)E * N * K / 8);
  std::vector<uint16_t> sc((size_t)E * N * K / 128), bi(sc.size());
  uint32_t s = 12345;
  for (auto& v : w) v = s = s * 1664525u + 1013904223u;
  for (size_t i = 0; i < sc.size(); ++i) {
    sc[i] = (uint16_t)(0x3C00 + (i & 0xFF));
    bi[i] = (uint16_t)(0xBC00 + (i & 0xFF));
  }
  std::vector<uint8_t> codes((size_t)E * N * K / 2);
  std::vector<uint16_t> sb((size_t)E * N * (K / 128) * 2);
  expect(moe_w4_from_mlx(E, N, K, w.data(), sc.data(), bi.data(), codes.data(), sb.data()), 0,
         "w4_from_mlx");
  // spot checks against the documented byte formula
  for (int e = 0; e < E; ++e)
    for (int n = 0; n < N; n += 7)
      for (int k = 0; k < K; k += 13) {
        const uint32_t q = (w[((size_t)e * N + n) * (K / 8) + k / 8] >> (4 * (k % 8))) & 15u;
        const size_t byte = (((size_t)e * (N / 32) + n / 32) * (K / 64) + k / 64) * 1024 +
                            (n % 32) * 32 + 4 * ((k % 64) / 8) + k % 4;
        const uint32_t got = (k % 8 >= 4) ? (codes[byte] >> 4) : (codes[byte] & 15u);
        expect(got, q, "w4 code position");
      }
  expect(moe_w4_from_mlx(E, 48, K, w.data(), sc.data(), bi.data(), codes.data(), sb.data()), 2,
         "w4_from_mlx N % 32");
  expect(moe_w4_from_mlx(E, N, K, nullptr, sc.data(), bi.data(), codes.data(), sb.data()), 1,
         "w4_from_mlx NULL");
}

}  // namespace

int main() {
  workspace_and_capacity();
  w4_converter();
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("host driver: all checks ok\n");
  return 0;
}
