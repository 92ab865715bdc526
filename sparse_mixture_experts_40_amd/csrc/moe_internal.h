// moe_internal.h — shared device helpers and kernel-launcher declarations of
// the gfx950 MoE library. Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 is carried as its 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite by contract).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Scaled fp16 rows of y_sorted (inside the bf16 layer forward): each chunk of
// kYChunk columns of a row holds fp16(v * 2^-e), with one exponent e (int8)
// per row and chunk, chosen from the chunk's largest |v| so that it scales to
// below 2^15: fp16's 11-bit significand (rounding error 2^-11 relative, an
// eighth of bf16's) over fp32's whole exponent range, in bf16's 2 bytes.
// H is a multiple of kYChunk.
constexpr int kYChunk = 64;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// e for a chunk whose largest |v| has bit pattern max_abs_bits (sign clear):
// floor(log2 max) - 14, at least -126 (2^-e stays a normal fp32); inf / NaN
// (biased exponent 255) give 114 and pass through the fp16 conversion as such.
__device__ __forceinline__ int yh_exponent(uint32_t max_abs_bits) {
  return max((int)(max_abs_bits >> 23) - 141, -126);
}

// 2^e as an fp32 for e in [-126, 127]
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// fp32 -> fp16 (round to nearest even), two to a word
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
}

__device__ __forceinline__ float2 unpack_f16x2(uint32_t u) {
  const f16x2_t h = __builtin_bit_cast(f16x2_t, u);
  return make_float2((float)h.x, (float)h.y);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(n) for the counts the pipelines need (n <= 32; a larger
// count waits for 32, which is stricter and so always safe)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    default:
      if (n > 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      break;
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (a __syncthreads() fence
// would drain the whole load pipeline). Each wave waits for its own LDS-DMA
// loads with wait_vmcnt before arriving, so after the barrier every wave's
// stage data is in LDS.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor (raw addressing) whose fields are wave-uniform SGPRs.
__device__ __forceinline__ i32x4_t dec_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// One LDS-DMA instruction: lane l's 16 bytes at rsrc + voff + soff land at LDS
// byte address m0 + 16 l. Written as asm so that the compiler does not tie the
// LDS reads that follow to these writes (it cannot tell the ring buffers
// apart and would drain every load in flight); the ring orders them with
// explicit vmcnt / lgkmcnt waits. The instruction has no register result.
// M0 is named as clobbered; no compiler-generated code in these kernels keeps
// a value in it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The descriptor and the scalar operands are wave-uniform by construction;
// readfirstlane keeps them in SGPRs even where the compiler lost track of that.
__device__ __forceinline__ i32x4_t uniform4(i32x4_t v) {
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(v.x);
  r.y = __builtin_amdgcn_readfirstlane(v.y);
  r.z = __builtin_amdgcn_readfirstlane(v.z);
  r.w = __builtin_amdgcn_readfirstlane(v.w);
  return r;
}

__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(uniform4(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

// dma16 with the non-temporal hint, for data read exactly once (streamed
// expert weights), so it does not displace the rows read again (tokens).
__device__ __forceinline__ void dma16_nt(i32x4_t rsrc, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(uniform4(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
#pragma clang diagnostic pop

// XCD-aware block order. Hardware block ids are dealt round-robin to the 8
// XCDs (id b runs on XCD b % 8, each XCD with its own L2). Map the first
// 8*floor(R/8) ids so that each XCD gets one contiguous range of logical tiles
// (neighbouring tiles share operands in that XCD's L2); the tail is identity.
// A bijection on [0, R).
__device__ __forceinline__ int xcd_remap(int b, int R) {
  const int full = R & ~7;
  return b < full ? (b & 7) * (full >> 3) + (b >> 3) : b;
}

// Row-block tiling of the expert-grouped rows: expert e owns rows
// [offsets[e], offsets[e+1]) and ceil(n_e / BM) row tiles.
// row_tile_scan fills s_scan (2*E+2 ints of LDS): [0,E) inclusive scan of the
// tile counts, [E+1, 2E+2) the offsets; returns the total number of row tiles.
// Must be called by all threads of a block of at least E threads (E <= 256).
template <int BM>
__device__ int row_tile_scan(const int32_t* __restrict__ offsets, int E, int* s_scan) {
  const int e = threadIdx.x;
  for (int i = e; i <= E; i += blockDim.x) s_scan[E + 1 + i] = offsets[i];
  __syncthreads();
  if (e < E) s_scan[e] = (s_scan[E + 2 + e] - s_scan[E + 1 + e] + BM - 1) / BM;
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {  // Hillis-Steele inclusive scan
    const int add = (e < E && e >= d) ? s_scan[e - d] : 0;
    __syncthreads();
    if (e < E) s_scan[e] += add;
    __syncthreads();
  }
  return s_scan[E - 1];
}

// (expert, first row, end row) of row tile `tile_id` < total.
template <int BM>
__device__ void row_tile_find(const int* s_scan, int E, int tile_id, int& expert, int& row0,
                              int& row_end) {
  int lo = 0, hi = E - 1;  // first expert whose inclusive tile count exceeds tile_id
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_scan[mid] > tile_id) hi = mid; else lo = mid + 1;
  }
  expert = lo;
  const int before = (lo == 0) ? 0 : s_scan[lo - 1];
  row0 = s_scan[E + 1 + lo] + (tile_id - before) * BM;
  row_end = s_scan[E + 2 + lo];
}

// ---- launchers (defined in the .hip files; all return hipGetLastError()) ----

// Router: logits (MFMA for bf16, FMA for fp32) + softmax + top-k + weights.
// x == nullptr: logits are read from `logits`. prob_partials (nullable):
// [router_num_blocks(c, x == nullptr), E] per-block sums of the full softmax.
// do_select == 0 skips the top-k (only partials are produced).
// Router variants and extra outputs (all nullable).
struct RouterExtras {
  const float* noise = nullptr;     // [T,E] logits-input mode: l + noise * softplus(nlogits)
  const float* nlogits = nullptr;   // [T,E] x W_noise^T
  const float* sel_bias = nullptr;  // [E] added to the top-k keys only
  float* zpart = nullptr;           // [blocks] per-block sums of (ln sum_e exp l)^2
  float* logits_final = nullptr;    // logits-input mode: the logits the softmax used
  int k_min = 0;                    // > 0: entropy-driven k in [k_min, top_k]
  int32_t* kt_out = nullptr;        // [T] the k of every token (dynamic k)
  const float* part = nullptr;      // logits-input mode: split-K partials [nsplit, T, E],
  int nsplit = 0;                   //   summed in split order (+ bias) as they are read
};
hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const float* bias, float* logits, bool logits_out, int32_t* topk_idx,
                         float* topk_w, float* prob_partials, bool do_select, hipStream_t s,
                         const RouterExtras& ex = {});
// Logits only: out [T,E] = x w^T (+ bias).
hipError_t launch_logits(const moe_config& c, const void* x, const void* w, const float* bias,
                         float* out, hipStream_t s);
int router_num_blocks(const moe_config& c, bool from_logits);
// Split-K router for small token counts (bf16): K splits (1 = not worth it),
// and the launch sequence partial logits -> softmax / top-k, which sums the
// partials in split order (+ bias) as it reads them. part: [splits, T, E]
// fp32; logits_out (optional) receives the summed logits.
int router_k_splits(const moe_config& c);
hipError_t launch_router_split(const moe_config& c, const void* x, const void* w_router,
                               const float* bias, float* logits_out, float* part,
                               int32_t* topk_idx, float* topk_w, float* prob_partials,
                               hipStream_t s, const RouterExtras& ex = {});
// Split-K logits only: out [T,E] = x w^T (+ bias), same summation order.
hipError_t launch_logits_split(const moe_config& c, const void* x, const void* w,
                               const float* bias, float* out, float* part, hipStream_t s);

// Dispatch: histogram per chunk, scan, stable scatter. capacity 0 keeps every
// pair; > 0 keeps the first `capacity` pairs of each expert (pair_pos = -1 for
// the others, their number in *dropped if non-null). counts are before the
// limit, offsets cover the kept pairs.
int dispatch_num_chunks(const moe_config& c);
hipError_t launch_dispatch(const moe_config& c, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* hist, int32_t* rank0, bool scatter, int capacity,
                           int32_t* dropped, hipStream_t s);

// Least-loaded fallback of a capacity limit, from the dropless dispatch
// (offsets, sorted_pair, pair_pos) of topk_idx: the routing in slot form
// (idx_out -1 where no expert) and the dropped slots left over added to
// *dropped, which is zeroed here first unless dropped_zeroed (an earlier
// launch on the stream wrote 0 there).
hipError_t launch_capacity_fallback(const moe_config& c, const int32_t* topk_idx,
                                    const float* topk_w, int capacity, int fallback_min,
                                    const int32_t* offsets, const int32_t* sorted_pair,
                                    const int32_t* pair_pos, int32_t* idx_out, float* w_out,
                                    int32_t* dropped, bool dropped_zeroed, hipStream_t s);

// Expert GEMMs.
hipError_t launch_gate_up(const moe_config& c, const void* x, const int32_t* sorted_pair,
                          const int32_t* offsets, const void* w_gate, const void* w_up, void* h,
                          hipStream_t s);
// y rows are fp32, or, where y_exp is given (bf16 layers) and the tiled
// kernel runs, scaled fp16 with their exponents in y_exp [rows][H / kYChunk];
// *y_half (nullable) says which was written.
hipError_t launch_down(const moe_config& c, const void* h, const int32_t* offsets,
                       const void* w_down, void* y, hipStream_t s, int8_t* y_exp = nullptr,
                       bool* y_half = nullptr);
// 4-bit weights (weight-streaming kernels): bf16 activations, H and I
// multiples of 512.
bool w4_supported(const moe_config& c);
hipError_t launch_gate_up_w4(const moe_config& c, const void* x, const int32_t* sorted_pair,
                             const int32_t* offsets, const moe_w4_weights& w, void* h,
                             hipStream_t s);
hipError_t launch_down_w4(const moe_config& c, const void* h, const int32_t* offsets,
                          const moe_w4_weights& w, void* y, hipStream_t s);

// Statistics outputs inside the library: the public moe_aux_out plus the
// z-loss output of moe_options (each nullable).
struct AuxOut {
  int32_t* counts = nullptr;
  float* f = nullptr;
  float* P = nullptr;
  float* aux = nullptr;
  float* z_loss = nullptr;
};

// Combine and statistics.
// y_exp (nullable): y rows are scaled fp16 with these exponents (bf16 layers,
// combine_half_fits), else fp32; the sum is fp32 either way.
bool combine_half_fits(const moe_config& c);
hipError_t launch_combine(const moe_config& c, const void* y, const int32_t* pair_pos,
                          const float* topk_w, void* out, hipStream_t s,
                          const int8_t* y_exp = nullptr);
// fp_scratch: E doubles of workspace (per-expert f_e * P_e).
// zpart [n_zpart] (nullable): per router block sums of (ln sum_e exp l)^2 for
// out.z_loss.
hipError_t launch_aux(const moe_config& c, const int32_t* counts, const float* prob_partials,
                      int n_partials, double* fp_scratch, const AuxOut& out, hipStream_t s,
                      const float* zpart = nullptr, int n_zpart = 0);

}  // namespace moe
