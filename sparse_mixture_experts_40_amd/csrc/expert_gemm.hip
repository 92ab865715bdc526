// expert_gemm.hip — grouped expert GEMMs of the SwiGLU experts.
//
// [MOE-128x8] "MoE架构深度解析：128专家与8激活的智能路由" (csdn), expert organisation
// (gate_proj / up_proj / down_proj per expert) and the parameter table
// (4096x1536 per projection); [QWEN3-READ] forward code (each expert is an MLP
// of width moe_intermediate_size applied to the tokens routed to it); the
// SwiGLU form down(silu(gate x) * up x).
//
// Rows are the expert-sorted routing pairs: expert e owns rows
// [offsets[e], offsets[e+1]) (built by the dispatch). A block computes one
// BM x BN tile of one expert; the tile is found on the device from `offsets`
// (no host sync, no tile list): the grid is the worst case
// (ceil(P/BM) + E row tiles) x (column tiles), and blocks past the last row
// tile exit at once. Empty experts own no tiles, so their weights are never
// read.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with the WEIGHT rows as the A operand
// and the token rows as B, so D[n][m] puts 4 consecutive output columns of one
// token row in each lane (8-byte stores). Both operands are K-contiguous; K is
// staged 64 at a time through double-buffered, XOR-swizzled LDS (16-byte
// chunk c of row r at chunk c ^ (r & 7): conflict-free ds_read_b128 /
// ds_write_b128).
//   gate/up: the B tile's first BN/2 rows are W_gate rows, the last BN/2 the
//            W_up rows of the same columns, so each lane holds matching g and
//            u; the epilogue writes h = silu(g) * u (fp32 math, one bf16
//            rounding). The A rows are gathered through sorted_pair / k.
//   down:    y_sorted = h W_down^T over contiguous h rows, stored in fp32
//            (the combine adds the k rows of a token in fp32 and rounds once).
// fp32 path (fp32 workloads): plain FMA kernels, one block per sorted row.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_bf16_kernel(
    int E, int K, int N_out, int k_top, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, void* __restrict__ out,
    int n_tiles_n) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;  // token rows per wave
  constexpr int WTN = BN / WAVES_N;  // weight rows per wave
  constexpr int MBW = WTM / 32, NBW = WTN / 32;
  constexpr int ACH = BM * 8 / NT;  // 16-byte chunks per thread per K step
  constexpr int BCH = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile / thread mismatch");
  static_assert(!GATEUP || NBW % 2 == 0, "gate/up needs paired blocks");
  constexpr int NCOL = GATEUP ? BN / 2 : BN;  // output columns per block

  __shared__ __align__(16) uint16_t s_a[2][BM * kBK];
  __shared__ __align__(16) uint16_t s_b[2][BN * kBK];
  __shared__ int s_scan[2 * 256 + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int n_real = row_tile_scan<BM>(offsets, E, s_scan) * n_tiles_n;
  if ((int)blockIdx.x >= n_real) return;  // uniform: beyond the last tile
  const int L = xcd_remap(blockIdx.x, n_real);
  const int m_lin = L / n_tiles_n, n_tile = L - m_lin * n_tiles_n;
  int expert, row0, row_end;
  row_tile_find<BM>(s_scan, E, m_lin, expert, row0, row_end);
  const int n0 = n_tile * NCOL;

  // per-thread source rows (nullptr: zero fill)
  const uint16_t* a_src[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int r = (tid >> 3) + (NT / 8) * i;
    const int gi = row0 + r;
    a_src[i] = nullptr;
    if (gi < row_end) {
      const int arow = GATEUP ? sorted_pair[gi] / k_top : gi;
      a_src[i] = act + (size_t)arow * K + (tid & 7) * 8;
    }
  }
  const uint16_t* b_src[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = (tid >> 3) + (NT / 8) * i;
    int n;
    const uint16_t* w;
    if (GATEUP) {
      n = n0 + (r < BN / 2 ? r : r - BN / 2);
      w = (r < BN / 2) ? w0 : w1;
    } else {
      n = n0 + r;
      w = w0;
    }
    b_src[i] = (n < N_out) ? w + ((size_t)expert * N_out + n) * K + (tid & 7) * 8 : nullptr;
  }

  f32x16_t acc[NBW][MBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = (tid >> 3) + (NT / 8) * i;
      *reinterpret_cast<uint4*>(&s_a[buf][swz(r, tid & 7)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int r = (tid >> 3) + (NT / 8) * i;
      *reinterpret_cast<uint4*>(&s_b[buf][swz(r, tid & 7)]) = rb[i];
    }
  };

  // weight row (within the B tile) of this lane for wave-local block nb
  auto wrow = [&](int nb) {
    if (GATEUP) {
      const int half = nb < NBW / 2 ? 0 : BN / 2;
      const int nbl = nb < NBW / 2 ? nb : nb - NBW / 2;
      return half + wn * (WTN / 2) + nbl * 32 + (lane & 31);
    }
    return wn * WTN + nb * 32 + (lane & 31);
  };

  const int nk = K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t af[NBW], bfr[MBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        af[nb] = *reinterpret_cast<const bf16x8_t*>(&s_b[cur][swz(wrow(nb), ch)]);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        bfr[mb] = *reinterpret_cast<const bf16x8_t*>(
            &s_a[cur][swz(wm * WTM + mb * 32 + (lane & 31), ch)]);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bfr[mb], acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[n][m], m = lane & 31, n = (r/4)*8 + (lane/32)*4 + r%4
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int row = row0 + wm * WTM + mb * 32 + (lane & 31);
    if (row >= row_end) continue;
    if (GATEUP) {
      uint16_t* orow = static_cast<uint16_t*>(out) + (size_t)row * N_out;
#pragma unroll
      for (int nb = 0; nb < NBW / 2; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * (WTN / 2) + nb * 32 + q * 8 + (lane >> 5) * 4;
          if (col < N_out) {
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              hv[j] = silu(acc[nb][mb][q * 4 + j]) * acc[nb + NBW / 2][mb][q * 4 + j];
            *reinterpret_cast<uint2*>(orow + col) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
        }
      }
    } else {
      float* orow = static_cast<float*>(out) + (size_t)row * N_out;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * WTN + nb * 32 + q * 8 + (lane >> 5) * 4;
          if (col < N_out)
            *reinterpret_cast<float4*>(orow + col) =
                make_float4(acc[nb][mb][q * 4 + 0], acc[nb][mb][q * 4 + 1],
                            acc[nb][mb][q * 4 + 2], acc[nb][mb][q * 4 + 3]);
        }
      }
    }
  }
}

// ---- fp32 path ------------------------------------------------------------

__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int i) {
  int lo = 0, hi = E - 1;  // largest e with offsets[e] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(int E, int H, int I, int k_top,
                                                          const float* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ wg,
                                                          const float* __restrict__ wu,
                                                          float* __restrict__ h) {
  extern __shared__ float s_x[];
  const int i = blockIdx.x;
  const int e = expert_of_row(offsets, E, i);
  const int t = sorted_pair[i] / k_top;
  for (int c = threadIdx.x; c < H; c += blockDim.x) s_x[c] = x[(size_t)t * H + c];
  __syncthreads();
  for (int n = threadIdx.x; n < I; n += blockDim.x) {
    const float* g = wg + ((size_t)e * I + n) * H;
    const float* u = wu + ((size_t)e * I + n) * H;
    float sg = 0.0f, su = 0.0f;
    for (int c = 0; c < H; ++c) {
      sg = fmaf(g[c], s_x[c], sg);
      su = fmaf(u[c], s_x[c], su);
    }
    h[(size_t)i * I + n] = sg / (1.0f + expf(-sg)) * su;
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(int E, int H, int I,
                                                       const float* __restrict__ h,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ wd,
                                                       float* __restrict__ y) {
  extern __shared__ float s_h[];
  const int i = blockIdx.x;
  const int e = expert_of_row(offsets, E, i);
  for (int c = threadIdx.x; c < I; c += blockDim.x) s_h[c] = h[(size_t)i * I + c];
  __syncthreads();
  for (int n = threadIdx.x; n < H; n += blockDim.x) {
    const float* d = wd + ((size_t)e * H + n) * I;
    float s = 0.0f;
    for (int c = 0; c < I; ++c) s = fmaf(d[c], s_h[c], s);
    y[(size_t)i * H + n] = s;
  }
}

// bf16 tile shapes
constexpr int GU_BM = 128, GU_BN = 128, GU_WM = 2, GU_WN = 2;
constexpr int DN_BM = 128, DN_BN = 128, DN_WM = 2, DN_WN = 2;

int grid_for(int P, int E, int BM, int n_tiles_n) {
  const long mt = (long)(P + BM - 1) / BM + (E < P ? E : P);
  return (int)(mt * n_tiles_n);
}

}  // namespace

hipError_t launch_gate_up(const moe_config& c, const void* x, const int32_t* sorted_pair,
                          const int32_t* offsets, const void* w_gate, const void* w_up, void* h,
                          hipStream_t s) {
  const int P = c.num_tokens * c.top_k;
  if (c.dtype == MOE_DTYPE_F32) {
    gate_up_f32_kernel<<<P, 256, c.hidden * sizeof(float), s>>>(
        c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const float*>(x),
        sorted_pair, offsets, static_cast<const float*>(w_gate), static_cast<const float*>(w_up),
        static_cast<float*>(h));
    return hipGetLastError();
  }
  const int ntn = (c.intermediate + GU_BN / 2 - 1) / (GU_BN / 2);
  const int grid = grid_for(P, c.num_experts, GU_BM, ntn);
  grouped_gemm_bf16_kernel<GU_BM, GU_BN, GU_WM, GU_WN, true><<<grid, 64 * GU_WM * GU_WN, 0, s>>>(
      c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const uint16_t*>(x),
      sorted_pair, offsets, static_cast<const uint16_t*>(w_gate),
      static_cast<const uint16_t*>(w_up), h, ntn);
  return hipGetLastError();
}

hipError_t launch_down(const moe_config& c, const void* h, const int32_t* offsets,
                       const void* w_down, void* y, hipStream_t s) {
  const int P = c.num_tokens * c.top_k;
  if (c.dtype == MOE_DTYPE_F32) {
    down_f32_kernel<<<P, 256, c.intermediate * sizeof(float), s>>>(
        c.num_experts, c.hidden, c.intermediate, static_cast<const float*>(h), offsets,
        static_cast<const float*>(w_down), static_cast<float*>(y));
    return hipGetLastError();
  }
  const int ntn = (c.hidden + DN_BN - 1) / DN_BN;
  const int grid = grid_for(P, c.num_experts, DN_BM, ntn);
  grouped_gemm_bf16_kernel<DN_BM, DN_BN, DN_WM, DN_WN, false><<<grid, 64 * DN_WM * DN_WN, 0, s>>>(
      c.num_experts, c.intermediate, c.hidden, c.top_k, static_cast<const uint16_t*>(h), nullptr,
      offsets, static_cast<const uint16_t*>(w_down), nullptr, y, ntn);
  return hipGetLastError();
}

}  // namespace moe
