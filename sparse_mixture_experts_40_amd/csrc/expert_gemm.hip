// expert_gemm.hip — grouped expert GEMMs of the SwiGLU experts.
//
// [MOE-128x8] "MoE架构深度解析：128专家与8激活的智能路由" (csdn), expert organisation
// (gate_proj / up_proj / down_proj per expert) and the parameter table
// (4096x1536 per projection); [QWEN3-READ] forward code (each expert is an MLP
// of width moe_intermediate_size applied to the tokens routed to it); the
// SwiGLU form down(silu(gate x) * up x).
//
// Rows are the expert-sorted routing pairs: expert e owns rows
// [offsets[e], offsets[e+1]) (built by the dispatch). The tile of a work item
// is found on the device from `offsets` (no host sync, no tile list). Empty
// experts own no tiles, so their weights are never read.
//
// bf16 path (persistent, one 512-thread block of 8 waves per CU):
//   tile  256 token rows x 256 weight rows; MFMA v_mfma_f32_32x32x16_bf16 with
//         the WEIGHT rows as the A operand and the token rows as B, so D[n][m]
//         puts 4 consecutive output columns of one token row in each lane;
//   gate/up: the weight tile's first 128 rows are W_gate rows, the last 128
//         the W_up rows of the same columns, so each lane holds matching g and
//         u; the epilogue writes h = silu(g) * u (fp32 math, one bf16
//         rounding). The token rows are gathered through sorted_pair / k;
//   down: y_sorted = h W_down^T over contiguous h rows, stored in fp32, or
//         inside the bf16 layer forward as fp16 scaled by 2^-e per row and 64
//         columns (the combine folds 2^e into the routing weight, adds the k
//         rows of a token in fp32 and rounds once).
// Decode-sized batches (few rows per expert) take the weight-streaming
// kernels further down instead.
// fp32 path (fp32 workloads): plain FMA kernels, one block per sorted row.
#include "aux_small.h"
#include "dispatch_chunk.h"
#include "moe_internal.h"

#include <atomic>


namespace moe {

namespace {

// silu(g) = g / (1 + e^-g); the reciprocal is the hardware approximation
// (about 1 ulp of fp32), far below the bf16 rounding of h that follows.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}




// LDS row swizzle: 16-byte chunk c of tile row r is stored at chunk c ^ f(r).
// f makes the fragment reads (16 consecutive rows at one chunk per 256-byte
// LDS cycle, or 8 rows per 128-byte cycle) conflict-free.
template <int BK>
__device__ __forceinline__ int swz_f(int r) {
  if (BK == 64) return (r & 7) ^ ((r >> 3) & 1);               // 8 chunks per row
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);   // 4 chunks per row
}

// LDS-DMA of one K stage: this wave's BK/8 A and BK/8 B load instructions
// (buffer_load_dwordx4 ... lds). Lane l of an instruction lands at M0 + 16 l,
// i.e. the instruction fills 1024 / (2 BK) consecutive tile rows; a_off / b_off
// hold each lane's source row and (swizzled) chunk, the K offset of the stage
// is the scalar offset. Buffer (MUBUF) rather than global (FLAT-encoded) loads:
// an outstanding FLAT load may count against both the vector-memory and the
// LDS counter, which makes the compiler wait for every LDS read in full
// (lgkmcnt(0)) while stage loads are in flight; with buffer loads it waits
// only for the fragments it needs.
// Loads [i0, i1) of the wave's LA + LB (A first, then B); the whole stage by
// default.
template <int BK, int BM, int NW, bool WNT>
__device__ __forceinline__ void dma_stage(uint16_t* __restrict__ dA, uint16_t* __restrict__ dB,
                                          __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t* a_off, const uint32_t* b_off, uint32_t kb,
                                          int wave, int i0 = 0, int i1 = 1 << 30) {
  constexpr int CPR = BK / 8, RPI = 64 / CPR;
  constexpr int LA = BM * BK / (512 * NW), LB = 256 * BK / (512 * NW);  // per wave
#pragma unroll
  for (int i = 0; i < LA; ++i)
    if (i >= i0 && i < i1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(dA + (wave * LA + i) * RPI * BK),
                                               16, a_off[i], kb, 0, 0);
#pragma unroll
  for (int i = 0; i < LB; ++i)
    if (LA + i >= i0 && LA + i < i1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dB + (wave * LB + i) * RPI * BK),
                                               16, b_off[i], kb, 0, WNT ? 2 : 0);
}

// Fragments of k step kk of a stage: NB weight blocks (A operand) and the MBV
// active token blocks (B operand) of this wave, 16 bytes per lane each. Token
// block mb of a wave covers tile rows trow0 + 64 mb (the two row halves of
// the waves interleave in 32-row blocks). A wave with no active block reads
// nothing.
template <int BK, int MB, int NB, int MBV>
__device__ __forceinline__ void stage_frag(const uint16_t* __restrict__ sA,
                                           const uint16_t* __restrict__ sB, int kk,
                                           bf16x8_t (&fa)[NB], bf16x8_t (&fb)[MB],
                                           const int (&wrow)[NB], int trow0, int lane, int sw) {
  if constexpr (MBV > 0) {
    const int pc = ((kk * 2 + (lane >> 5)) ^ sw) * 8;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      fa[nb] = *reinterpret_cast<const bf16x8_t*>(sB + wrow[nb] * BK + pc);
#pragma unroll
    for (int mb = 0; mb < MBV; ++mb)
      fb[mb] = *reinterpret_cast<const bf16x8_t*>(sA + (trow0 + mb * 64) * BK + pc);
  }
}

// One K stage of the pipeline: start the loads of stage (dA, dB) (in two
// halves, see below), multiply stage (cA, cB), wait for stage (nA, nB) and
// read its first fragments.
// Half of the last k step's MFMAs are issued after the stage barrier, so the
// MFMA pipe stays busy while the wave waits at the barrier and while the next
// stage's first fragments arrive from LDS. (On the last stage the "next"
// fragments are stale LDS data that is never used.)
// The distinct __restrict__ pointers give the LDS accesses disjoint alias
// scopes, so the compiler does not drain the in-flight LDS-DMA loads before
// every fragment read; the explicit wait_vmcnt + lds_barrier order them.
template <int BK, int BM, int NW, int MB, int NB, int MBV, bool WNT>
__device__ __forceinline__ void gemm_step(
    uint16_t* __restrict__ dA, uint16_t* __restrict__ dB, bool issue_next,
    __amdgpu_buffer_rsrc_t abase, __amdgpu_buffer_rsrc_t bbase, const uint32_t* a_off,
    const uint32_t* b_off, uint32_t kb,
    const uint16_t* __restrict__ cA, const uint16_t* __restrict__ cB,
    const uint16_t* __restrict__ nA, const uint16_t* __restrict__ nB, int vm_allow,
    f32x16_t (&acc)[NB][MB], bf16x8_t (&fa)[2][NB], bf16x8_t (&fb)[2][MB],
    const int (&wrow)[NB], int trow0, int lane, int sw, int wave) {
  constexpr int KK = BK / 16;
  constexpr int L = (KK - 1) & 1;  // fragment buffer of the last k step
  constexpr int NH = NB / 2;       // last k step: blocks [0, NH) before the barrier
  // The stage loads are issued in two halves (the A rows, then the B rows), at
  // the start of k steps 0 and 1. A wave issues in order, and a burst of all
  // its loads stalled it at issue, MFMAs included, while the memory pipeline
  // took them in (-4% gate/up and down at 128 experts x 16K tokens). Later
  // or finer splits leave the last loads too little time to land (+5%).
  constexpr int NL = BM * BK / (512 * NW) + 256 * BK / (512 * NW);
  constexpr int KD = KK < 2 ? KK : 2;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk < KD && issue_next)
      dma_stage<BK, BM, NW, WNT>(dA, dB, abase, bbase, a_off, b_off, kb, wave, NL * kk / KD,
                            NL * (kk + 1) / KD);
    if (kk + 1 < KK)
      stage_frag<BK, MB, NB, MBV>(cA, cB, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1], wrow,
                                  trow0, lane, sw);
    const int nbe = (kk + 1 < KK) ? NB : NH;
#pragma unroll
    for (int nb = 0; nb < nbe; ++nb)
#pragma unroll
      for (int mb = 0; mb < MBV; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][nb], fb[kk & 1][mb],
                                                              acc[nb][mb], 0, 0, 0);
    // first the fragment reads of the next k step, then this step's MFMAs, so
    // each read has a whole step of MFMAs to land before its use
    if constexpr (MBV > 0) {
      if (kk + 1 < KK) {
        __builtin_amdgcn_sched_group_barrier(0x100, NB + MBV, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NB * MBV, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NH * MBV, 0);
      }
    }
  }
  wait_vmcnt(vm_allow);
  lds_barrier();
  stage_frag<BK, MB, NB, MBV>(nA, nB, 0, fa[0], fb[0], wrow, trow0, lane, sw);
#pragma unroll
  for (int nb = NH; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MBV; ++mb)
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[L][nb], fb[L][mb], acc[nb][mb], 0,
                                                            0, 0);
  if constexpr (MBV > 0) {
#pragma unroll
    for (int i = 0; i < (NB - NH) * MBV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
}

// The K loop of one tile for a wave with MBV active token blocks. The LDS
// stages form a ring that runs on across tiles: global stage g sits in buffer
// g % NST, the tile's K stage kt is global stage g0 + kt, and each step loads
// the stage NST - 1 ahead, which in the tile's last NST - 1 steps is a first
// stage of the next tile (pf), so the pipeline never drains between tiles.
// Waves without active blocks still issue their loads and take every barrier.
// The wait before a step's barrier lets the stages issued after the awaited
// one stay in flight, and for the stages of this tile loaded before the
// previous epilogue (kt < NST - 1 when the tile was prefetched) also st_allow,
// the number of store instructions that epilogue issued: the counter
// completes in order, so the stage has landed once no more than those stores
// remain. The count must never exceed the stores actually issued.
template <int BK, int BM, int NST, int NW, int MB, int NB, int MBV, bool WNT>
__device__ __forceinline__ void tile_k(uint16_t* smem, int nk, int g0, bool pf, int st_allow,
                                       __amdgpu_buffer_rsrc_t abase, __amdgpu_buffer_rsrc_t bbase,
                                       __amdgpu_buffer_rsrc_t bbase_n, const uint32_t* a_off,
                                       const uint32_t* b_off, const uint32_t* a_offn,
                                       const uint32_t* b_offn, f32x16_t (&acc)[NB][MB],
                                       const int (&wrow)[NB], int trow0, int lane, int sw,
                                       int wave) {
  constexpr int LA = BM * BK / (512 * NW), LB = 256 * BK / (512 * NW);
  constexpr int STAGE = (BM + 256) * BK;
  bf16x8_t fa[2][NB], fb[2][MB];
  const uint16_t* c0 = smem + (g0 % NST) * STAGE;
  stage_frag<BK, MB, NB, MBV>(c0, c0 + BM * BK, 0, fa[0], fb[0], wrow, trow0, lane, sw);
  for (int kt = 0; kt < nk; ++kt) {
    const int g = g0 + kt;
    const int is = kt + NST - 1;  // stage loaded by this step, counted from the tile start
    const bool in_cur = is < nk;
    // stages issued after the awaited stage kt + 1 once this step's loads are
    // out. The last step awaits nothing (its post-barrier fragment reads are
    // unused): the next tile's stages stay in flight through the epilogue.
    const int last = (in_cur || pf) ? is : nk - 1;
    const int vm = kt + 1 < nk ? (LA + LB) * (last - (kt + 1)) + (kt + 1 < NST - 1 ? st_allow : 0)
                               : (pf ? (LA + LB) * (NST - 1) : 0);
    uint32_t ao[LA], bo[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) ao[i] = in_cur ? a_off[i] : a_offn[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) bo[i] = in_cur ? b_off[i] : b_offn[i];
    uint16_t* dA = smem + ((g + NST - 1) % NST) * STAGE;
    const uint16_t* cA = smem + (g % NST) * STAGE;
    const uint16_t* nA = smem + ((g + 1) % NST) * STAGE;
    gemm_step<BK, BM, NW, MB, NB, MBV, WNT>(
        dA, dA + BM * BK, in_cur || pf, abase, in_cur ? bbase : bbase_n, ao, bo,
        (uint32_t)((in_cur ? is : is - nk) * BK) * 2u, cA, cA + BM * BK, nA, nA + BM * BK, vm,
        acc, fa, fb, wrow, trow0, lane, sw, wave);
  }
}

// Location and per-lane load offsets of tile L (column tile major inside an
// expert: expert e owns tiles [ntn * S[e-1], ntn * S[e])).
struct GemmTile {
  int row0, row_end, n0, expert;
};

template <bool GATEUP, int BM, int BK, int NW, int NCOL, int LA, int LB>
__device__ __forceinline__ void tile_setup(int L, int n_tiles_n, int E, int K, int N_out,
                                           int k_top, const int* s_scan,
                                           const int32_t* __restrict__ sorted_pair, int wave,
                                           int lane, GemmTile& tl, uint32_t (&a_off)[LA],
                                           uint32_t (&b_off)[LB]) {
  constexpr int CPR = BK / 8, RPI = 64 / CPR;
  int expert, row0, row_end;
  row_tile_find<BM>(s_scan, E, L / n_tiles_n, expert, row0, row_end);
  const int s_prev = expert ? s_scan[expert - 1] : 0;
  const int mt = s_scan[expert] - s_prev;
  const int local = L - n_tiles_n * s_prev;
  const int n_tile = local / mt, m_tile = local - n_tile * mt;
  // the expert's rows split evenly over its mt row tiles, in multiples of 32
  // (q <= BM, and every tile is non-empty since n_e > BM (mt - 1) >= q (mt - 1))
  const int e0 = s_scan[E + 1 + expert];
  const int q = ((row_end - e0 + mt - 1) / mt + 31) & ~31;
  tl.row0 = e0 + m_tile * q;
  tl.row_end = min(tl.row0 + q, row_end);
  tl.n0 = n_tile * NCOL;
  tl.expert = expert;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (wave * LA + i) * RPI + lane / CPR;  // tile row written by this lane
    const int lc = (lane % CPR) ^ swz_f<BK>(r);       // logical chunk for its slot
    int gi = tl.row0 + r;
    gi = gi < tl.row_end ? gi : tl.row_end - 1;
    const int arow = GATEUP ? sorted_pair[gi] / k_top : gi;
    a_off[i] = ((uint32_t)arow * (uint32_t)K + (uint32_t)lc * 8u) * 2u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * RPI + lane / CPR;
    const int lc = (lane % CPR) ^ swz_f<BK>(r);
    int n = tl.n0 + (GATEUP ? (r & 127) : r);
    n = n < N_out ? n : N_out - 1;
    b_off[i] = ((uint32_t)n * (uint32_t)K + (uint32_t)lc * 8u) * 2u;
  }
}

// Buffer descriptor of a byte range (raw addressing, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Persistent grouped GEMM: NW waves per block (2 x NW/2), OCC blocks per CU.
//   tile: BM token rows x 256 weight rows, K staged BK at a time through NST
//         LDS stages (NST - 1 stages of loads in flight under the MFMAs);
//   wave: (BM/2) x (512/NW) = MB x NB blocks of v_mfma_f32_32x32x16_bf16 with
//         fp32 accumulators; with 8 waves, two waves share each SIMD, so one
//         wave's loads, LDS reads and barrier waits overlap the other's MFMAs;
//   fragments of the next 16-wide k step are read while the MFMAs of the
//         current one issue; the first fragments of the next stage are read
//         right after the stage barrier, while deferred MFMAs keep the pipe busy;
//   tiles: each XCD (hardware block b runs on XCD b % 8) walks one contiguous
//         range of tiles; inside an expert the order is column tile major,
//         row tile minor, so concurrent blocks share weight tiles in L2.
// Rows past an expert's end and columns past N are clamped to valid memory on
// load and never stored.
template <bool GATEUP, int BM, int BK, int NST, int NW, int OCC, bool WNT>
__global__ __launch_bounds__(64 * NW, OCC) void grouped_gemm_bf16_kernel(
    int E, int K, int N_out, int k_top, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, void* __restrict__ out,
    int n_tiles_n, int8_t* __restrict__ y_exp) {
  constexpr int BN = 256;
  constexpr int WN = NW / 2;                  // waves along the weight rows
  constexpr int MB = BM / 64;                 // token blocks of 32 rows per wave
  constexpr int NB = BN / (WN * 32);          // weight blocks of 32 rows per wave
  constexpr int NCOL = GATEUP ? BN / 2 : BN;  // output columns per tile
  constexpr int LA = BM * BK / (512 * NW);    // A load instructions per wave per stage
  constexpr int LB = BN * BK / (512 * NW);    // B load instructions per wave per stage
  constexpr int STAGE = (BM + BN) * BK;       // elements per stage
  static_assert(BK / 16 == 1 || (BK / 16) % 2 == 0, "fragment double buffer parity");
  static_assert(NB % 2 == 0 && LA >= 1 && LB >= 1, "tile / wave mismatch");
  __shared__ __align__(1024) uint16_t smem[NST * STAGE];
  __shared__ int s_scan[2 * 256 + 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave & 1, wn = wave >> 1;
  const int R = row_tile_scan<BM>(offsets, E, s_scan) * n_tiles_n;
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3;
  const int chunk = (R + 7) >> 3;
  const int nk = K / BK;

  const int sw = swz_f<BK>(lane & 31);  // swizzle of every fragment row of this lane
  int wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    wrow[nb] = GATEUP ? ((nb / (NB / 2)) * 128 + wn * (NB / 2) * 32 + (nb % (NB / 2)) * 32 +
                         (lane & 31))
                      : (wn * NB * 32 + nb * 32 + (lane & 31));
  const int trow0 = wm * 32 + (lane & 31);  // token block mb: tile rows trow0 + 64 mb

  // A operand: the activation rows (x for gate/up, h for down); offsets stay
  // below 2^32 bytes (checked on the host)
  const __amdgpu_buffer_rsrc_t abase = make_rsrc(act, 0xFFFFFFFFu);
  // B rows [0, 128) of a gate/up tile come from W_gate, [128, 256) from W_up
  const uint16_t* wsel = (GATEUP && wave >= NW / 2) ? w1 : w0;
  const uint32_t wbytes = (uint32_t)N_out * (uint32_t)K * 2u;  // one expert's matrix
  int t = blockIdx.x >> 3;
  bool have = t < chunk && xcd * chunk + t < R;
  GemmTile cur;
  uint32_t a_off[LA], b_off[LB];
  if (have)
    tile_setup<GATEUP, BM, BK, NW, NCOL, LA, LB>(xcd * chunk + t, n_tiles_n, E, K, N_out, k_top,
                                                 s_scan, sorted_pair, wave, lane, cur, a_off,
                                                 b_off);
  bool staged = false;  // first NST - 1 stages of `cur` loaded by the previous tile
  // store instructions this wave issued in the previous tile's epilogue,
  // after those prefetched stages (exact: see the epilogues)
  int st_after = 0;
  int g0 = 0;  // ring position (global stage index) of the tile's first K stage
  while (have) {
    const int tn = t + nper;
    const bool have_n = tn < chunk && xcd * chunk + tn < R;
    GemmTile nxt{};
    uint32_t a_offn[LA], b_offn[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) a_offn[i] = 0u;
#pragma unroll
    for (int i = 0; i < LB; ++i) b_offn[i] = 0u;
    if (have_n)
      tile_setup<GATEUP, BM, BK, NW, NCOL, LA, LB>(xcd * chunk + tn, n_tiles_n, E, K, N_out,
                                                   k_top, s_scan, sorted_pair, wave, lane, nxt,
                                                   a_offn, b_offn);
    // the last NST - 1 steps load the next tile's first stages
    const bool prefetch = have_n && nk >= NST - 1;
    const __amdgpu_buffer_rsrc_t bbase =
        make_rsrc(wsel + (size_t)__builtin_amdgcn_readfirstlane(cur.expert) * N_out * K, wbytes);
    const __amdgpu_buffer_rsrc_t bbase_n =
        make_rsrc(wsel + (size_t)__builtin_amdgcn_readfirstlane(have_n ? nxt.expert : 0) * N_out * K,
                  wbytes);

    f32x16_t acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;
    // prologue: NST - 1 stages in flight (unless prefetched), then wait for
    // the first
    const int npro = nk < NST - 1 ? nk : NST - 1;
    if (!staged) {
      for (int st = 0; st < npro; ++st) {
        uint16_t* d = smem + ((g0 + st) % NST) * STAGE;
        dma_stage<BK, BM, NW, WNT>(d, d + BM * BK, abase, bbase, a_off, b_off,
                              (uint32_t)(st * BK) * 2u, wave);
      }
      wait_vmcnt((LA + LB) * (npro - 1));
    } else {
      wait_vmcnt((LA + LB) * (NST - 2) + st_after);
    }
    lds_barrier();
    const int st_allow = staged ? st_after : 0;

    // token blocks of this wave with at least one row of the expert: the
    // MFMAs (and fragment reads) of the others are skipped, so the last,
    // partly filled tile of an expert costs in proportion to its rows
    const int live = min(BM, cur.row_end - cur.row0) - wm * 32;
    const int mbv = live <= 0 ? 0 : min(MB, (live + 63) / 64);
    if (mbv >= MB)
      tile_k<BK, BM, NST, NW, MB, NB, MB, WNT>(smem, nk, g0, prefetch, st_allow, abase, bbase, bbase_n,
                                          a_off, b_off, a_offn, b_offn, acc, wrow, trow0, lane,
                                          sw, wave);
    else if (mbv == 3)
      tile_k<BK, BM, NST, NW, MB, NB, (MB > 3 ? 3 : MB), WNT>(smem, nk, g0, prefetch, st_allow, abase, bbase,
                                                         bbase_n, a_off, b_off, a_offn, b_offn,
                                                         acc, wrow, trow0, lane, sw, wave);
    else if (mbv == 2)
      tile_k<BK, BM, NST, NW, MB, NB, (MB > 2 ? 2 : MB), WNT>(smem, nk, g0, prefetch, st_allow, abase, bbase,
                                                         bbase_n, a_off, b_off, a_offn, b_offn,
                                                         acc, wrow, trow0, lane, sw, wave);
    else if (mbv == 1)
      tile_k<BK, BM, NST, NW, MB, NB, 1, WNT>(smem, nk, g0, prefetch, st_allow, abase, bbase, bbase_n, a_off, b_off,
                                         a_offn, b_offn, acc, wrow, trow0, lane, sw, wave);
    else
      tile_k<BK, BM, NST, NW, MB, NB, 0, WNT>(smem, nk, g0, prefetch, st_allow, abase, bbase, bbase_n, a_off, b_off,
                                         a_offn, b_offn, acc, wrow, trow0, lane, sw, wave);
    // No barrier here: the only LDS the epilogue touches is the stage computed
    // last (its reads finished before the last stage barrier), and the next
    // tile's first LDS writes are ordered by the barriers of its prologue and
    // first step.
    // At the next tile's start the compiler waits for every outstanding load
    // and store anyway (for the sorted_pair loads of the tile after it, and
    // before the first fragment read, which it cannot tell apart from the
    // prefetched stage's LDS writes), so the epilogue's stores do not stay in
    // flight into the next tile. Both ways of avoiding that (the loads issued
    // from inline asm, and the sorted_pair rows turned into offsets only
    // before the tile's last step) measured 1-2% slower in an A/B in one
    // process: every K step waits for its own stage (vmcnt(0)) in any case.
    // The explicit waits alone are nevertheless correct (exact store counts).
    const int row0 = cur.row0, row_end = cur.row_end, n0 = cur.n0;

    // epilogue: lane holds D[n][m], m = lane & 31, n = (r/4)*8 + (lane/32)*4 + r%4
    if constexpr (GATEUP) {
    // Store instructions this wave issues: one per (token block, column
    // group) in which lane 0 has a row inside the tile and a column inside
    // the matrix. Lane 0 holds the block's first row and the group's first
    // column, so exactly those instructions run with a non-empty exec mask;
    // the others are branched over. The count must never exceed what is
    // issued: the next tile's first wait lets that many operations stay in
    // flight. Columns matter on an expert's last column tile when N_out is
    // not a multiple of 128 (waves whose columns all lie past N_out store
    // nothing there).
    st_after = 0;
    {
      int ncg = 0;  // column groups (nb, q) of this wave with a column inside the matrix
#pragma unroll
      for (int nb = 0; nb < NB / 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ncg += (n0 + wn * (NB / 2) * 32 + nb * 32 + q * 8 < N_out) ? 1 : 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        st_after += (row0 + wm * 32 + mb * 64 < row_end) ? ncg : 0;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = row0 + trow0 + mb * 64;
      if (row >= row_end) continue;
      {
        uint16_t* orow = static_cast<uint16_t*>(out) + (size_t)row * N_out;
#pragma unroll
        for (int nb = 0; nb < NB / 2; ++nb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n0 + wn * (NB / 2) * 32 + nb * 32 + q * 8 + (lane >> 5) * 4;
            if (col < N_out) {
              float hv[4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                hv[j] = silu(acc[nb][mb][q * 4 + j]) * acc[nb + NB / 2][mb][q * 4 + j];
              *reinterpret_cast<uint2*>(orow + col) =
                  make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
            }
          }
        }
      }
    }
    } else {
      constexpr int NG = NB * 32 / kYChunk;  // scaled-fp16 chunks per wave and row
      static_assert(NG * kYChunk == NB * 32 && kYChunk == 64, "whole chunks of two blocks");
      // each kYChunk columns of this wave lie wholly inside N or wholly past it
      const int ycol0 = n0 + wn * NB * 32;
      if (y_exp) {
        // scaled fp16 straight from the accumulators, no LDS: lane l holds 4
        // consecutive columns q*8 + (l/32)*4 .. +3 (q = 0..3) of each 32-column
        // block for token row l & 31. One v_permlane32_swap (lane i <-> lane
        // i + 32) per q pair gives lane l < 32 the block's columns 0..15 and
        // lane l + 32 its columns 16..31, so each lane stores two 16-byte
        // pieces and every row's 128 bytes of this wave are written whole
        // (against a pass through LDS with barriers per 64 rows: the same
        // results, -0.4% layer time at 128 experts x 16K tokens). The chunk
        // exponent comes from the row's largest |v| over the wave's kYChunk
        // columns (fmaxf skips NaN).
        const int h = lane >> 5;
        // store instructions: 2 per block and token block in which lane 0
        // (the block's first row) is inside the tile; the exponent byte
        // stores are not counted (fewer counted than issued only makes the
        // next tile's first wait stricter)
        st_after = 0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int g = 0; g < NG; ++g)
            st_after +=
                (ycol0 + g * kYChunk < N_out && row0 + mb * 64 + wm * 32 < row_end) ? 4 : 0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
          float mx = 0.0f;
#pragma unroll
          for (int nb = 2 * g; nb < 2 * g + 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(acc[nb][mb][r]));
          {
            const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                             __float_as_uint(mx), false, false);
            mx = fmaxf(mx, __uint_as_float(h ? sm[0] : sm[1]));
          }
          const int e = yh_exponent(__float_as_uint(mx));
          const float sc = pow2i(-e);
          const int gcol0 = ycol0 + g * kYChunk;
          const int grow = row0 + mb * 64 + wm * 32 + (lane & 31);
          const bool live = grow < row_end && gcol0 < N_out;
          if (h == 0 && live)
            y_exp[(size_t)grow * (N_out / kYChunk) + gcol0 / kYChunk] = (int8_t)e;
#pragma unroll
          for (int nb = 2 * g; nb < 2 * g + 2; ++nb) {
            uint32_t pk[4][2];  // column group q as 4 fp16 in 2 words
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              pk[q][0] = pack_f16x2(acc[nb][mb][q * 4 + 0] * sc, acc[nb][mb][q * 4 + 1] * sc);
              pk[q][1] = pack_f16x2(acc[nb][mb][q * 4 + 2] * sc, acc[nb][mb][q * 4 + 3] * sc);
            }
            uint32_t r0[2], r1[2];  // received: groups 0 / 1 (lower lanes), 2 / 3 (upper)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const auto s02 = __builtin_amdgcn_permlane32_swap(pk[0][w], pk[2][w], false, false);
              const auto s13 = __builtin_amdgcn_permlane32_swap(pk[1][w], pk[3][w], false, false);
              r0[w] = h ? s02[0] : s02[1];
              r1[w] = h ? s13[0] : s13[1];
            }
            const u32x4_t lo = h ? u32x4_t{r0[0], r0[1], pk[2][0], pk[2][1]}
                                 : u32x4_t{pk[0][0], pk[0][1], r0[0], r0[1]};
            const u32x4_t hi = h ? u32x4_t{r1[0], r1[1], pk[3][0], pk[3][1]}
                                 : u32x4_t{pk[1][0], pk[1][1], r1[0], r1[1]};
            if (live) {
              u32x4_t* dst = reinterpret_cast<u32x4_t*>(
                  static_cast<uint16_t*>(out) + (size_t)grow * N_out + ycol0 + nb * 32 + h * 16);
              // plain stores: L2 merges each row's 128 bytes before writing
              // back (non-temporal 16-byte pieces were 1.7% slower)
              dst[0] = lo;
              dst[1] = hi;
            }
          }
        }
      } else {
      // fp32 rows: the tile goes through the LDS stage computed last (free
      // now: its reads completed before the last stage barrier) in MB passes
      // of 64 rows x 256 columns, so that each store instruction writes one
      // contiguous 1 KB row. 16-byte chunk c of slab row s sits at chunk
      // c ^ (s & 15): conflict-free for the column writes (16 rows, one chunk)
      // and the row reads (one row, 16 chunks).
      static_assert(BN * 64 * 4 <= STAGE * 2, "slab must fit in one stage");
      float* slab = reinterpret_cast<float*>(smem + ((g0 + nk - 1) % NST) * STAGE);
      const int srow_w = wm * 32 + (lane & 31);
      // one store per slab row of this wave inside the tile
      st_after = 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        st_after += min(max(row_end - (row0 + mb * 64 + wave * (64 / NW)), 0), 64 / NW);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = (wn * NB * 32 + nb * 32 + q * 8 + (lane >> 5) * 4) >> 2;
            *reinterpret_cast<float4*>(slab + srow_w * BN + ((chunk ^ (srow_w & 15)) << 2)) =
                make_float4(acc[nb][mb][q * 4 + 0], acc[nb][mb][q * 4 + 1],
                            acc[nb][mb][q * 4 + 2], acc[nb][mb][q * 4 + 3]);
          }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 64 / NW; ++i) {
          const int sr = wave * (64 / NW) + i;  // slab row
          const int row = row0 + mb * 64 + sr;  // slab row sr = 32 wm + m
          const float4 v =
              *reinterpret_cast<const float4*>(slab + sr * BN + ((lane ^ (sr & 15)) << 2));
          const int col = n0 + lane * 4;
          // y_sorted is read once, by the combine: non-temporal stores keep it
          // from displacing the operands in L2 (-2.5% down at 16K tokens)
          if (row < row_end && col < N_out)
            __builtin_nontemporal_store(
                f32x4_t{v.x, v.y, v.z, v.w},
                reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + (size_t)row * N_out + col));
        }
        lds_barrier();
      }
      }
    }

    staged = prefetch;
    g0 += nk;
    cur = nxt;
#pragma unroll
    for (int i = 0; i < LA; ++i) a_off[i] = a_offn[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) b_off[i] = b_offn[i];
    t = tn;
    have = have_n;
  }
}

// tile height, K step, LDS stages (2 x 64 KB), waves per block, blocks per CU.
// The gate/up kernel also runs with BK = 32 and 4 stages (1.5x the bytes in
// flight; the down epilogue needs a 64 KB stage): 8% slower at 128 experts x
// 16K tokens.
constexpr int kGemmBM = 256, kGemmBK = 64, kGemmStages = 2, kGemmWaves = 8, kGemmOcc = 1;

// ---- bf16 decode path (few rows per expert: weight streaming) -------------
//
// Work item = (touched expert e, chunk c of 32 output columns): gate/up reads
// 32 W_gate + 32 W_up rows, down reads 64 W_down rows, each exactly once; the
// expert's token rows (n_e <= 64 per pass, padded to 32-row MFMA blocks) are
// read from L2. K is split over the 4 waves (fixed reduction order through
// LDS, so the result is deterministic). Each wave streams its K quarter in
// groups of 64 elements (128 bytes of every weight and token row) through a
// ring of LDS buffers of its own: LDS-DMA loads (buffer_load_dwordx4 ... lds)
// in which 8 consecutive lanes cover one 128-byte line, so one instruction
// moves 8 whole lines, and the MFMA fragments are then read from LDS. Loading
// the fragments straight from global memory would give each lane of an
// instruction its own cache line (32 weight rows per instruction), and the
// vector L1 serves such an instruction one lane at a time.
// Experts with no rows own no work items and read no weight bytes.
#ifndef MOE_DEC_K
#define MOE_DEC_K 64
#endif
constexpr int kDecWRows = 64;                      // weight rows per work item
constexpr int kDecK = MOE_DEC_K;                   // K elements per group (row bytes / 2)
constexpr int kDecOcc = kDecK == 32 ? 2 : 1;       // blocks per CU
constexpr int kDecRegion = 18432 / kDecOcc;        // LDS ring of one wave, bf16 elements
constexpr int kDecCPR = kDecK / 8;                 // 16-byte chunks per row
constexpr int kDecRPI = 64 / kDecCPR;              // rows per DMA instruction (1 KB)
static_assert(kDecK == 32 || kDecK == 64, "group width");

// Ring geometry for NTB token blocks of 32 rows: a group buffer holds the 64
// weight rows and 32 NTB token rows, kDecK elements each (row r, 16-byte
// chunk c stored at chunk c ^ swz_f<kDecK>(r)); 3 buffers fit for one token
// block, 2 for two.
template <int NTB>
struct DecRing {
  static constexpr int BUF = (kDecWRows + 32 * NTB) * kDecK;
  static constexpr int NBUF = kDecRegion / BUF;
  static constexpr int WI = kDecWRows / kDecRPI;  // weight DMA instructions per group
  static constexpr int TI = 32 / kDecRPI;         // token DMA instructions per token block
  static constexpr int NL = WI + TI * NTB;        // DMA instructions per group
  static_assert(NBUF >= 2 && NBUF <= 3 && NL * (NBUF - 1) <= 32, "ring depth");
};


// LDS-DMA of one group (byte offset kb along this wave's K range) into the
// buffer at LDS byte address dst: WI weight instructions (kDecRPI rows each;
// the first half from rw0, the second from rw1) and TI NTB token instructions.
template <int NTB>
__device__ __forceinline__ void dec_dma(uint32_t dst, i32x4_t rw0, i32x4_t rw1, i32x4_t ract,
                                        const uint32_t (&w_off)[8], const uint32_t (&t_off)[8],
                                        uint32_t kb) {
  constexpr int WI = DecRing<NTB>::WI, TI = DecRing<NTB>::TI;
#pragma unroll
  for (int i = 0; i < WI; ++i)  // weights: read once per pass, non-temporal
    dma16_nt(i < WI / 2 ? rw0 : rw1, dst + i * 1024, w_off[i], kb);
#pragma unroll
  for (int j = 0; j < TI * NTB; ++j)
    dma16(ract, dst + kDecWRows * kDecK * 2 + j * 1024, t_off[j], kb);
}

// The kDecK / 16 k steps of one group from LDS: weight blocks (A operand, rows
// 32 nb + lane & 31) against token blocks (B operand).
template <int NTB>
__device__ __forceinline__ void dec_compute(const uint16_t* src, int rd, int sw, int h,
                                            f32x16_t (&acc)[2][2]) {
  constexpr int KS = kDecK / 16;
  bf16x8_t wf[KS][2], tf[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int pos = ((2 * s + h) ^ sw) * 8;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      wf[s][nb] = *reinterpret_cast<const bf16x8_t*>(src + nb * 32 * kDecK + rd + pos);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      tf[s][tb] = *reinterpret_cast<const bf16x8_t*>(src + (kDecWRows + tb * 32) * kDecK + rd +
                                                     pos);
  }
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s][nb], tf[s][tb], acc[nb][tb],
                                                              0, 0, 0);
  // every fragment read first, so that the reads of later steps land while
  // the MFMAs of the first steps run
  __builtin_amdgcn_sched_group_barrier(0x100, KS * (2 + NTB), 0);
  __builtin_amdgcn_sched_group_barrier(0x008, KS * 2 * NTB, 0);
}

// s_waitcnt vmcnt(NL * r) for r in [0, NBUF - 1), r wave-uniform.
template <int NL, int NBUF>
__device__ __forceinline__ void wait_groups(int r) {
  if constexpr (NBUF <= 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (r >= 1) wait_vmcnt(NL); else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// This wave's ng groups through its ring of NBUF buffers (ring = element
// pointer, ring_lds = its LDS byte address): NBUF - 1 groups in flight while
// one is multiplied. Before a buffer is loaded again, the fragment reads of
// the group it held are complete (lgkmcnt(0); the MFMAs of that group have
// consumed them anyway).
template <int NTB>
__device__ __forceinline__ void dec_kloop(int ng, const uint16_t* ring, uint32_t ring_lds,
                                          i32x4_t rw0, i32x4_t rw1, i32x4_t ract,
                                          const uint32_t (&w_off)[8], const uint32_t (&t_off)[8],
                                          int rd, int sw, int h, f32x16_t (&acc)[2][2]) {
  using R = DecRing<NTB>;
  constexpr int NBUF = R::NBUF, BUF = R::BUF, NL = R::NL;
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < ng)
      dec_dma<NTB>(ring_lds + j * BUF * 2, rw0, rw1, ract, w_off, t_off, j * (kDecK * 2u));
  for (int g0 = 0; g0 < ng; g0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int g = g0 + j, gl = g + NBUF - 1;
      if (g < ng) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (gl < ng) {
          dec_dma<NTB>(ring_lds + ((j + NBUF - 1) % NBUF) * BUF * 2, rw0, rw1, ract, w_off, t_off,
                       (uint32_t)gl * (kDecK * 2u));
          wait_vmcnt(NL * (NBUF - 1));
        } else {
          wait_groups<NL, NBUF>(ng - 1 - g);
        }
        dec_compute<NTB>(ring + j * BUF, rd, sw, h, acc);
      }
    }
  }
}

// The loads of one work item as a wave sees them: weight descriptors and
// per-lane offsets, token offsets of its (single) pass.
// The one-chunk sort of a SORT gate/up launch (idx null otherwise).
struct DecSort {
  const int32_t* idx;  // [P] expert of each routing pair (-1: empty slot)
  int P, cap;          // pairs; capacity (0: none)
  int32_t* counts;     // [E] pairs per expert (nullable)
  int32_t* offsets;    // [E+1] first sorted row of each expert
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* dropped;  // pairs past the capacity (nullable)
  int do_aux;        // block 1 writes the statistics `aux`
  AuxSmallArgs aux;
};

struct DecItem {
  i32x4_t rw0, rw1;
  uint32_t w_off[8], t_off[8];
};

// One token block, one pass (the common decode item): the ring runs on across
// items. pre: the item's groups 0 .. NBUF-2 are already in flight, in buffers
// bq, bq+1, ... (mod NBUF). With nxt, the last NBUF-1 iterations load the
// next item's groups 0 .. NBUF-2 instead of nothing, so its loads overlap this
// item's last groups and its epilogue. Returns the buffer of the last group
// (free when the loop ends; the next item starts at the one after it).
__device__ __forceinline__ int dec_kloop_stream(int ng, const uint16_t* ring, uint32_t ring_lds,
                                                const DecItem& cur, bool pre, int bq,
                                                const DecItem& nxt, bool has_nxt, i32x4_t ract,
                                                int rd, int sw, int h, f32x16_t (&acc)[2][2]) {
  using R = DecRing<1>;
  constexpr int NBUF = R::NBUF, BUF = R::BUF, NL = R::NL;
  if (!pre) {
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
      if (j < ng)
        dec_dma<1>(ring_lds + ((bq + j) % NBUF) * BUF * 2, cur.rw0, cur.rw1, ract, cur.w_off,
                   cur.t_off, j * (kDecK * 2u));
  }
  int bi = bq, bl = (bq + NBUF - 1) % NBUF;
  for (int g = 0; g < ng; ++g) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int gl = g + NBUF - 1;
    if (gl < ng) {
      dec_dma<1>(ring_lds + bl * BUF * 2, cur.rw0, cur.rw1, ract, cur.w_off, cur.t_off,
                 (uint32_t)gl * (kDecK * 2u));
      wait_vmcnt(NL * (NBUF - 1));
    } else if (has_nxt) {
      dec_dma<1>(ring_lds + bl * BUF * 2, nxt.rw0, nxt.rw1, ract, nxt.w_off, nxt.t_off,
                 (uint32_t)(gl - ng) * (kDecK * 2u));
      wait_vmcnt(NL * (NBUF - 1));
    } else {
      wait_groups<NL, NBUF>(ng - 1 - g);
    }
    dec_compute<1>(ring + bi * BUF, rd, sw, h, acc);
    bi = bi + 1 == NBUF ? 0 : bi + 1;
    bl = bl + 1 == NBUF ? 0 : bl + 1;
  }
  return bi == 0 ? NBUF - 1 : bi - 1;
}

// Split-K reduction over the 4 waves in fixed order (waves 0..3), then the
// epilogue of one pass: gate/up blocks (nb 0 = gate, 1 = up) -> h = silu(g) u
// in bf16; down blocks -> y_sorted in fp32. Rows p0.. of the pass, r1 = end
// of the expert's rows; the accumulators hold D[n][m] (n weight row, m token).
// Wave w's partial sums sit at s_part + w * WST, [nb][tb][r][lane].
// Only the partial sums of the first NT token blocks are written (with one
// token block they take 12 KB: one ring buffer). The barriers are LDS-only,
// so loads still in flight (the next item's first groups) are not waited for.
template <bool GATEUP, int NB, int WST, int NT>
__device__ __forceinline__ void dec_epilogue(const f32x16_t (&acc)[NB][2], float* s_part, int p0,
                                             int r1, int ntb, int c, int N_out,
                                             void* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto part = [&](int w, int nb, int tb, int r) -> float& {
    return s_part[w * WST + ((nb * 2 + tb) * 16 + r) * 64 + lane];
  };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) part(wave, nb, tb, r) = acc[nb][tb][r];
  lds_barrier();
  {
    const int tb = (tid >> 6) & 1, half = tid >> 7;  // thread: (tb, lane, half of r)
    const int row = p0 + tb * 32 + (lane & 31);
    if (tb < ntb && row < r1) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = half * 2 + qq;  // group of 4 consecutive columns
        float v[NB][4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = q * 4 + j;
            v[nb][j] = ((part(0, nb, tb, r) + part(1, nb, tb, r)) + part(2, nb, tb, r)) +
                       part(3, nb, tb, r);
          }
        const int n_in = q * 8 + (lane >> 5) * 4;  // column inside a 32-wide block
        if (GATEUP) {
          const int col = c * 32 + n_in;
          if (col < N_out) {
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) hv[j] = silu(v[0][j]) * v[1][j];
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)row * N_out + col) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int col = c * 64 + nb * 32 + n_in;
            if (col < N_out)
              *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)row * N_out + col) =
                  make_float4(v[nb][0], v[nb][1], v[nb][2], v[nb][3]);
          }
        }
      }
    }
  }
}

// act holds act_bytes bytes (token rows x K); every byte offset formed below
// is smaller than that (the launcher checks it fits 32 bits).
// SORT (gate/up of a one-chunk routing): every block sorts the routing pairs
// ds.idx in its own LDS (the dispatch's stable counting sort) and takes its
// rows' tokens from there, so no dispatch launch precedes the kernel. Block 0
// writes the sort's outputs for the kernels that follow (counts, offsets,
// sorted_pair, pair_pos, the dropped count), block 1 the load-balance
// statistics when ds.do_aux; both then run their items like the others.
template <bool GATEUP, bool SORT = false>
__global__ __launch_bounds__(256, kDecOcc) void decode_gemm_bf16_kernel(
    int E, int K, int N_out, int k_top, const uint16_t* __restrict__ act, uint32_t act_bytes,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, void* __restrict__ out,
    int n_chunks, DecSort ds) {
  constexpr int NB = 2;  // weight blocks of 32 rows: gate + up, or 2 down blocks
  static_assert(NB * 2 * 16 * 64 <= kDecRegion / 2, "partial sums fit the wave's ring");
  static_assert(sizeof(DispLds) <= sizeof(uint16_t) * 4 * kDecRegion, "sort LDS fits the ring");
  __shared__ __align__(1024) uint16_t s_ring[4 * kDecRegion];
  __shared__ int s_scan[2 * 256 + 2];
  __shared__ uint16_t s_tok[SORT ? kDispChunk : 1];  // token of each sorted row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // s_scan[e]: inclusive count of experts with rows; offsets in s_scan[E+1..]
  if constexpr (SORT) {
    DispLds& L = *reinterpret_cast<DispLds*>(s_ring);  // the ring is not in use yet
    const int tot = disp_counts(ds.P, E, ds.cap, ds.idx, L);
    if (blockIdx.x == 1 && ds.do_aux) aux_small_body(ds.aux, tot);  // block-uniform
    const bool b0 = blockIdx.x == 0;
    if (b0) {
      if (tid < E) {
        if (ds.counts) ds.counts[tid] = tot;
        ds.offsets[tid] = L.off[tid];
      }
      if (tid == 0) {
        ds.offsets[E] = L.c[255];
        if (ds.dropped) *ds.dropped = L.drop;
      }
    }
    for (int i = tid; i <= E; i += blockDim.x) s_scan[E + 1 + i] = i < E ? L.off[i] : L.c[255];
    scatter_chunk(
        ds.P, E, ds.cap, ds.idx, 0, L.h, L.off, L.wc,
        [&](int p, int pos) {
          s_tok[pos] = (uint16_t)(p / k_top);
          if (b0) {
            ds.sorted_pair[pos] = p;
            ds.pair_pos[p] = pos;
          }
        },
        [&](int p) {
          if (b0) ds.pair_pos[p] = -1;
        });  // ends with a barrier: L is free for the ring
  } else {
    for (int i = tid; i <= E; i += blockDim.x) s_scan[E + 1 + i] = offsets[i];
  }
  __syncthreads();
  if (tid < E) s_scan[tid] = (s_scan[E + 2 + tid] > s_scan[E + 1 + tid]) ? 1 : 0;
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {
    const int add = (tid < E && tid >= d) ? s_scan[tid - d] : 0;
    __syncthreads();
    if (tid < E) s_scan[tid] += add;
    __syncthreads();
  }
  const int items = s_scan[E - 1] * n_chunks;
  const int kw = K / 4;     // this wave's K range [wave*kw, wave*kw + kw)
  const int ng = kw / kDecK;  // groups of kDecK elements
  uint16_t* ring = s_ring + wave * kDecRegion;
  float* s_part = reinterpret_cast<float*>(s_ring);  // wave w at + w * kDecRegion / 2
  const int rd = (lane & 31) * kDecK, sw = swz_f<kDecK>(lane & 31), h = lane >> 5;
  const int lrow = lane / kDecCPR, lch = lane % kDecCPR;  // row / chunk inside a DMA instruction
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void_t*)ring;
  const i32x4_t ract = dec_rsrc(act, act_bytes);

  // item it: its expert (the (rank+1)-th expert with rows), column chunk,
  // rows [r0, r1), and its load descriptors (token offsets for the pass at p0)
  auto locate = [&](int it, int& c, int& e, int& r0, int& r1) {
    const int rank = it / n_chunks;
    c = __builtin_amdgcn_readfirstlane(it - rank * n_chunks);
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_scan[mid] > rank) hi = mid; else lo = mid + 1;
    }
    e = __builtin_amdgcn_readfirstlane(lo);
    r0 = s_scan[E + 1 + e];
    r1 = s_scan[E + 2 + e];
  };
  // weight rows of an item: gate/up rows [32c, 32c + 32) of both matrices,
  // down rows [64c, 64c + 64); rows past N_out are clamped to the last one
  auto weights = [&](int c, int e, DecItem& d) {
    const int nrow0 = GATEUP ? c * 32 : c * 64;
    const int nrows = min(GATEUP ? 32 : 64, N_out - nrow0);
    const uint32_t wbytes = (uint32_t)nrows * (uint32_t)K * 2u;
    d.rw0 = dec_rsrc(w0 + ((size_t)e * N_out + nrow0) * K, wbytes);
    d.rw1 = GATEUP ? dec_rsrc(w1 + ((size_t)e * N_out + nrow0) * K, wbytes) : d.rw0;
#pragma unroll
    for (int i = 0; i < kDecWRows / kDecRPI; ++i) {
      const int r = kDecRPI * i + lrow;  // LDS weight row (32 nb + row inside the block)
      int nl = GATEUP ? (r & 31) : r;
      nl = nl < nrows ? nl : nrows - 1;
      d.w_off[i] = ((uint32_t)nl * (uint32_t)K + (uint32_t)(wave * kw) +
                    (uint32_t)((lch ^ swz_f<kDecK>(r)) * 8)) * 2u;
    }
  };
  auto tokens = [&](int p0, int r1, DecItem& d) {
#pragma unroll
    for (int j = 0; j < 64 / kDecRPI; ++j) {
      const int t = kDecRPI * j + lrow;  // token row of the pass (LDS row 64 + t)
      int gi = p0 + t;
      gi = gi < r1 ? gi : r1 - 1;
      int arow = gi;
      if constexpr (GATEUP) arow = SORT ? (int)s_tok[gi] : sorted_pair[gi] / k_top;
      d.t_off[j] = ((uint32_t)arow * (uint32_t)K + (uint32_t)(wave * kw) +
                    (uint32_t)((lch ^ swz_f<kDecK>(t)) * 8)) * 2u;
    }
  };

  bool pre = false;  // the item's first groups are in flight (loaded by the previous item)
  int bq = 0;        // ring buffer of the item's first group
  DecItem cur, nxt;
  int c, e, r0, r1;
  if (blockIdx.x < items) {
    locate(blockIdx.x, c, e, r0, r1);
    weights(c, e, cur);
  }
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const bool simple = r1 - r0 <= 32;  // one token block, one pass
    // the next item of this block, prefetched when both are simple
    const int itn = it + gridDim.x;
    int cn = 0, en = 0, r0n = 0, r1n = 0;
    if (itn < items) {
      locate(itn, cn, en, r0n, r1n);
      weights(cn, en, nxt);
    }
    const bool has_nxt = simple && itn < items && r1n - r0n <= 32 && ng >= DecRing<1>::NBUF;
    if (simple) {
      if (!pre) tokens(r0, r1, cur);
      if (has_nxt) tokens(r0n, r1n, nxt);
      f32x16_t acc[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb][tb][r] = 0.0f;
      const int bz = dec_kloop_stream(ng, ring, ring_lds, cur, pre, bq, nxt, has_nxt, ract, rd,
                                      sw, h, acc);
      // this wave's reads are done; the buffer of its last group is free
      // (loads still in flight target the other buffers)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dec_epilogue<GATEUP, NB, kDecRegion / 2, 1>(
          acc, reinterpret_cast<float*>(s_ring + bz * DecRing<1>::BUF), r0, r1, 1, c, N_out,
          out);
      lds_barrier();  // the partial sums are read before that buffer is loaded again
      pre = has_nxt;
      bq = bz + 1 == DecRing<1>::NBUF ? 0 : bz + 1;
    } else {
      for (int p0 = r0; p0 < r1; p0 += 64) {  // 64 token rows per pass
        tokens(p0, r1, cur);
        const int ntb = (r1 - p0) > 32 ? 2 : 1;
        f32x16_t acc[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][tb][r] = 0.0f;
        if (ntb > 1)
          dec_kloop<2>(ng, ring, ring_lds, cur.rw0, cur.rw1, ract, cur.w_off, cur.t_off, rd, sw,
                       h, acc);
        else
          dec_kloop<1>(ng, ring, ring_lds, cur.rw0, cur.rw1, ract, cur.w_off, cur.t_off, rd, sw,
                       h, acc);
        // every ring buffer of this wave has landed and been read: the
        // wave's partial sums may overwrite its ring
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        if (ntb > 1)
          dec_epilogue<GATEUP, NB, kDecRegion / 2, 2>(acc, s_part, p0, r1, ntb, c, N_out, out);
        else
          dec_epilogue<GATEUP, NB, kDecRegion / 2, 1>(acc, s_part, p0, r1, ntb, c, N_out, out);
        lds_barrier();  // the partial sums are read before the next pass loads
      }
      pre = false;
      bq = 0;
    }
    cur = nxt;
    // the copy loses the compiler's knowledge that the descriptors are
    // wave-uniform: make them SGPR values once per item
    cur.rw0 = uniform4(cur.rw0);
    cur.rw1 = uniform4(cur.rw1);
    c = cn;
    e = en;
    r0 = r0n;
    r1 = r1n;
  }
}

// ---- 4-bit weights, weight-streaming path --------------------------------
//
// [MOE-128x8] 参数量化与存储优化: 4-bit codes in groups of 128 along K with an
// independent scale and bias per group, w = scale * q + bias. Work items and
// the 4-way split-K are those of decode_gemm_bf16_kernel; the codes and
// (scale, bias) pairs are stored in tiles of 32 rows (moe.h), so one chunk of
// a 32-row block is 1 KB contiguous and its DMA uses whole cache lines.
// No weight is rounded: the MFMA multiplies the exact bf16 values 128 + q
// with the tokens, a second MFMA against ones gives the group's token sums,
// and each group of 128 is folded into the fp32 accumulators as
//   sum_k w x = scale * sum_k (128 + q) x + (bias - 128 scale) * sum_k x.
// The tokens are the A operand and the weights the B operand, so a lane's
// accumulators belong to one weight row (lane & 31) and one (scale, bias)
// per group. K is taken in chunks of 64: lane half h covers elements
// [32h, 32h + 32) of a chunk (16 bytes of codes) in 4 MFMA k steps of 8 and
// reads its token fragments in the same order.
//
// The loop is bound by instruction issue more than by memory, so it is laid
// out to issue few instructions, and two 4-wave blocks share each CU (two
// waves per SIMD: one wave's VALU work overlaps the other's MFMAs and waits):
//  - 16 codes unpack with 13 VALU: two masks and one 64-bit shift give the
//    nibbles as bytes, and each byte permute forms two bf16 values, taking
//    their exponent byte from a constant register;
//  - each wave streams its chunks through a ring of NBUF LDS buffers filled
//    by LDS-DMA: a steady loop keeps D = NBUF - 1 chunks in flight, then the
//    last D chunks run unrolled (entered part-way when the wave has fewer),
//    so every wait count and fragment register set is a compile-time
//    constant;
//  - the (scale, bias) dwords of a group come with its first chunk only, and
//    token rows only in the 8-row groups that exist (TG of them).

// 16 codes -> the bf16 values 128 + q. Byte b of a 32-bit code word holds
// element b of the word's 8 in its low nibble and element b + 4 in its high
// nibble; w holds two words (elements 0..7 low, 8..15 high).
__device__ __forceinline__ void w4_unpack16(uint64_t w, uint32_t c43, bf16x8_t& e0_7,
                                            bf16x8_t& e8_15) {
  constexpr uint64_t m = 0x0F0F0F0F0F0F0F0Full;
  const uint64_t lo = w & m, hi = (w >> 4) & m;
  const uint32_t l0 = (uint32_t)lo, l1 = (uint32_t)(lo >> 32);
  const uint32_t h0 = (uint32_t)hi, h1 = (uint32_t)(hi >> 32);
  // perm(c43, x, s): byte i is x's byte s_i for s_i < 4, else 0x43; so
  // (x_a, 0x43, x_b, 0x43) is the bf16 pair (128 + x_a, 128 + x_b)
  e0_7 = __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_amdgcn_perm(c43, l0, 0x04010400u),
                                                 __builtin_amdgcn_perm(c43, l0, 0x04030402u),
                                                 __builtin_amdgcn_perm(c43, h0, 0x04010400u),
                                                 __builtin_amdgcn_perm(c43, h0, 0x04030402u)));
  e8_15 = __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_amdgcn_perm(c43, l1, 0x04010400u),
                                                  __builtin_amdgcn_perm(c43, l1, 0x04030402u),
                                                  __builtin_amdgcn_perm(c43, h1, 0x04010400u),
                                                  __builtin_amdgcn_perm(c43, h1, 0x04030402u)));
}

// One LDS-DMA instruction of 4 bytes per lane: lane l's dword at
// rsrc + voff + soff lands at LDS byte address m0 + 4 l (no register result).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(i32x4_t rsrc, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Ring geometry for NTB token blocks of 32 rows with TG 8-row token groups
// loaded. One buffer (bytes): the codes of the 64 weight rows (32 bytes
// each, 16-byte piece p of row r at p ^ ((r >> 3) & 1)), the (scale, bias)
// dwords of rows 0..31 and 32..63 (256 bytes each, lane l's slot holding row
// l & 31 of its half), and 8 TG token rows of 128 bytes (chunk c of row t at
// c ^ swz_f<64>(t)).
// LDS per wave of the 4-bit kernel (bytes) and token rows per pass: two
// 4-wave blocks share a CU (two waves per SIMD), so one wave's VALU work
// overlaps the other's MFMAs, loads and waits.
#ifndef MOE_W4_REGION
#define MOE_W4_REGION 19968
#endif
#ifndef MOE_W4_ROWS
#define MOE_W4_ROWS 32
#endif
constexpr int kW4Region = MOE_W4_REGION, kW4Rows = MOE_W4_ROWS;
static_assert(kW4Rows % 8 == 0 && kW4Rows <= 32, "rows per pass");

template <int NTB, int TG>
struct W4Cfg {
  static constexpr int CODE = 0, SB = 2048, TOK = 2560;
  static constexpr int BUF = TOK + TG * 1024;
  static constexpr int NLE = 4 + TG;  // DMA instructions of a group's first chunk
  static constexpr int NLO = 2 + TG;  // and of its second
  static constexpr int FIT = kW4Region / BUF < 9 ? kW4Region / BUF : 9;
  static constexpr int NBUF = FIT % 2 ? FIT : FIT - 1;  // odd, so D is even
  static constexpr int D = NBUF - 1;
  // DMA instructions of n consecutive chunks, the first of them a group's
  // first chunk (even) or second
  static constexpr int run(bool even, int n) {
    int s = 0;
    for (int i = 0; i < n; ++i) s += ((i % 2 == 0) == even) ? NLE : NLO;
    return s;
  }
  static_assert(D >= 2 && run(true, D - 1) <= 32, "ring depth and vmcnt range");
  static_assert(8 * TG >= 32 * (NTB - 1) + 1 && 8 * TG <= 32 * NTB, "token groups");
  static_assert(NBUF * BUF <= kW4Region, "ring fits the wave's region");
};

template <int NTB>
struct W4Frag {
  uint4 cw[2];            // codes of the lane's rows in weight blocks 0, 1
  bf16x8_t tf[4][NTB];    // token fragments of the 4 k steps
};

// One wave's K loop over its nch chunks (an even number, two per group).
template <int NTB, int TG>
struct W4Loop {
  using C = W4Cfg<NTB, TG>;
  const uint8_t* ring;  // the wave's LDS region, for the fragment reads
  uint32_t ring_lds;    // its LDS byte address, for the DMA
  i32x4_t rq0, rq1, rs0, rs1, ract;
  const uint32_t (&q_off)[2];
  const uint32_t (&s_off)[2];
  const uint32_t (&t_off)[4];
  int lane;
  uint32_t c43;

  // LDS-DMA of chunk ch into buffer b; EVEN: ch opens its group and also
  // brings the group's (scale, bias) dwords.
  template <bool EVEN>
  __device__ __forceinline__ void dma(int ch, int b) const {
    const uint32_t dst = ring_lds + (uint32_t)b * C::BUF;
    dma16(rq0, dst + C::CODE, q_off[0], (uint32_t)ch * 1024u);
    dma16(rq1, dst + C::CODE + 1024, q_off[1], (uint32_t)ch * 1024u);
    if constexpr (EVEN) {
      dma4(rs0, dst + C::SB, s_off[0], (uint32_t)(ch >> 1) * 128u);
      dma4(rs1, dst + C::SB + 256, s_off[1], (uint32_t)(ch >> 1) * 128u);
    }
#pragma unroll
    for (int j = 0; j < TG; ++j) dma16(ract, dst + C::TOK + j * 1024, t_off[j], (uint32_t)ch * 128u);
  }

  __device__ __forceinline__ void frag(int b, W4Frag<NTB>& f) const {
    const uint8_t* src = ring + b * C::BUF;
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      f.cw[nb] = *reinterpret_cast<const uint4*>(src + C::CODE + (nb * 32 + n) * 32 +
                                                 ((h ^ ((n >> 3) & 1)) * 16));
    // MFMA rows past the pass's 8 TG token rows read row n % 8 instead: their
    // outputs are never stored, and the reads stay in the buffer
    const int nt = n < 8 * TG ? n : (n & 7);
    const int sw = swz_f<64>(nt);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        f.tf[j][tb] = *reinterpret_cast<const bf16x8_t*>(src + C::TOK + (tb * 32 + nt) * 128 +
                                                         (((4 * h + j) ^ sw) * 16));
  }

  __device__ __forceinline__ void sb(int b, uint32_t (&v)[2]) const {
    const uint8_t* src = ring + b * C::BUF + C::SB + (lane & 31) * 4;
    v[0] = *reinterpret_cast<const uint32_t*>(src);
    v[1] = *reinterpret_cast<const uint32_t*>(src + 256);
  }

  // aq += tokens x (128 + q), ax += tokens x 1 over the 4 k steps of a chunk;
  // FIRST: the chunk opens a group (the first k step starts from zero).
  template <bool FIRST>
  __device__ __forceinline__ void mult(const W4Frag<NTB>& f, f32x16_t (&aq)[2][NTB],
                                       f32x16_t (&ax)[NTB]) const {
    const bf16x8_t ones = __builtin_bit_cast(
        bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    const f32x16_t zero = {};
    bf16x8_t wq[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      w4_unpack16(((uint64_t)f.cw[nb].y << 32) | f.cw[nb].x, c43, wq[nb][0], wq[nb][1]);
      w4_unpack16(((uint64_t)f.cw[nb].w << 32) | f.cw[nb].z, c43, wq[nb][2], wq[nb][3]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          aq[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              f.tf[j][tb], wq[nb][j], (FIRST && j == 0) ? zero : aq[nb][tb], 0, 0, 0);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        ax[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.tf[j][tb], ones,
                                                         (FIRST && j == 0) ? zero : ax[tb], 0, 0,
                                                         0);
    }
  }

  // acc += scale aq + (bias - 128 scale) ax with this lane's rows' (scale,
  // bias) dwords (bf16 scale in the low half, bias in the high half).
  __device__ __forceinline__ void fold(const uint32_t (&sbv)[2], const f32x16_t (&aq)[2][NTB],
                                       const f32x16_t (&ax)[NTB], f32x16_t (&acc)[2][NTB]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float scale = __uint_as_float(sbv[nb] << 16);
      const float bias2 = fmaf(-128.0f, scale, __uint_as_float(sbv[nb] & 0xFFFF0000u));
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[nb][tb][r] = fmaf(scale, aq[nb][tb][r], fmaf(bias2, ax[tb][r], acc[nb][tb][r]));
    }
  }

  // Chunk ch, in buffer b (EVEN: it opens a group): (ISSUE) start the loads
  // of chunk ch + D into the buffer of chunk ch - 1, whose reads have
  // completed; (WAITN >= 0) wait until chunk ch + 1 has landed, WAITN DMA
  // instructions of later chunks still in flight, and read its fragments;
  // multiply chunk ch; when ch closes its group, fold it and read the next
  // group's (scale, bias) (the fold has consumed the previous ones).
  template <bool EVEN, bool ISSUE, int WAITN>
  __device__ __forceinline__ void step(int ch, int b, const W4Frag<NTB>& cur, W4Frag<NTB>& nxt,
                                       uint32_t (&sbv)[2], f32x16_t (&aq)[2][NTB],
                                       f32x16_t (&ax)[NTB], f32x16_t (&acc)[2][NTB]) const {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int bn = b + 1 == C::NBUF ? 0 : b + 1;
    if constexpr (ISSUE) dma<EVEN>(ch + C::D, b == 0 ? C::NBUF - 1 : b - 1);
    if constexpr (WAITN >= 0) {
      wait_vm<WAITN>();
      frag(bn, nxt);
    }
    mult<EVEN>(cur, aq, ax);
    if constexpr (!EVEN) {
      fold(sbv, aq, ax, acc);
      if constexpr (WAITN >= 0) sb(bn, sbv);
    }
  }

  // The last chunks, R of them left at the step (chunk nch - R, whose
  // fragments are in fA when R is even, else in fB); entered at R = r0.
  template <int R>
  __device__ __forceinline__ void drain(int r0, int nch, int& b, W4Frag<NTB>& fA,
                                        W4Frag<NTB>& fB, uint32_t (&sbv)[2],
                                        f32x16_t (&aq)[2][NTB], f32x16_t (&ax)[NTB],
                                        f32x16_t (&acc)[2][NTB]) const {
    if constexpr (R > 0) {
      if (r0 >= R) {
        constexpr bool EVEN = R % 2 == 0;
        if constexpr (EVEN)
          step<true, false, (R > 1 ? C::run(true, R - 2) : -1)>(nch - R, b, fA, fB, sbv, aq, ax,
                                                                 acc);
        else
          step<false, false, (R > 1 ? C::run(false, R - 2) : -1)>(nch - R, b, fB, fA, sbv, aq,
                                                                   ax, acc);
        b = b + 1 == C::NBUF ? 0 : b + 1;
      }
      drain<R - 1>(r0, nch, b, fA, fB, sbv, aq, ax, acc);
    }
  }

  __device__ __forceinline__ void run_k(int nch, f32x16_t (&acc)[2][NTB]) const {
    const int n0 = nch < C::D ? nch : C::D;  // chunks loaded ahead
#pragma unroll
    for (int c = 0; c < C::D; ++c)
      if (c < n0) {
        if (c % 2 == 0)
          dma<true>(c, c);
        else
          dma<false>(c, c);
      }
    // chunk 0 has landed once the loads of chunks 1 .. n0-1 are all that remain
    wait_vmcnt((n0 / 2) * C::NLO + ((n0 - 1) / 2) * C::NLE);
    W4Frag<NTB> fA, fB;
    uint32_t sbv[2];
    frag(0, fA);
    sb(0, sbv);
    f32x16_t aq[2][NTB], ax[NTB];
    int b = 0;
    for (int ch = 0; ch < nch - C::D; ch += 2) {
      step<true, true, C::run(true, C::D - 1)>(ch, b, fA, fB, sbv, aq, ax, acc);
      b = b + 1 == C::NBUF ? 0 : b + 1;
      step<false, true, C::run(false, C::D - 1)>(ch + 1, b, fB, fA, sbv, aq, ax, acc);
      b = b + 1 == C::NBUF ? 0 : b + 1;
    }
    drain<C::D>(n0, nch, b, fA, fB, sbv, aq, ax, acc);
  }
};

// Split-K reduction and stores of one pass of nr <= 8 TG token rows, for
// accumulators in the tokens-x-weights orientation: register r of block nb
// holds token row (r / 4) * 8 + (lane / 32) * 4 + r % 4 and weight row
// lane & 31, so only registers r < 4 TG hold rows of the pass. Each wave
// writes those to its slab s_part + w * WST ([nb][r][lane]); then every
// thread takes whole outputs (gate/up: nr rows x 32 columns of h; down: nr
// rows x 64 columns of y), adding the four waves' partial sums in wave order.
template <bool GATEUP, int TG, int WST>
__device__ __forceinline__ void w4_epilogue(const f32x16_t (&acc)[2][1], float* s_part, int p0,
                                            int nr, int c, int N_out, void* __restrict__ out) {
  constexpr int NR = 4 * TG;  // registers holding rows of the pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < NR; ++r) s_part[wave * WST + (nb * NR + r) * 64 + lane] = acc[nb][0][r];
  __syncthreads();
  constexpr int NC = GATEUP ? 32 : 64;  // output columns of the item
  for (int o = tid; o < nr * NC; o += 256) {
    const int m = o / NC, col = o % NC, nb = GATEUP ? 0 : col >> 5, n = col & 31;
    // token m sits in register (m / 8) * 4 + m % 4 of lane half (m / 4) % 2
    const int at = (nb * NR + (m >> 3) * 4 + (m & 3)) * 64 + ((m >> 2) & 1) * 32 + n;
    auto sum = [&](int off) {
      return ((s_part[at + off] + s_part[WST + at + off]) + s_part[2 * WST + at + off]) +
             s_part[3 * WST + at + off];
    };
    const size_t row = (size_t)(p0 + m);
    if (GATEUP) {
      const float g = sum(0), u = sum(NR * 64);
      static_cast<uint16_t*>(out)[row * N_out + c * 32 + n] = f32_to_bf16(silu(g) * u);
    } else {
      static_cast<float*>(out)[row * N_out + c * 64 + col] = sum(0);
    }
  }
}

// K (= H for gate/up, I for down) is a multiple of 512, so each wave's quarter
// is a whole number of 128-groups. act holds act_bytes bytes; every byte
// offset formed below is smaller (the launcher checks it fits 32 bits).
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void decode_w4_kernel(
    int E, int K, int N_out, int k_top, const uint16_t* __restrict__ act, uint32_t act_bytes,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ offsets,
    const uint8_t* __restrict__ q0, const uint16_t* __restrict__ sb0,
    const uint8_t* __restrict__ q1, const uint16_t* __restrict__ sb1, void* __restrict__ out,
    int n_chunks) {
  constexpr int NB = 2;  // weight blocks of 32 rows: gate + up, or 2 down blocks
  static_assert(NB * (kW4Rows / 2) * 64 * 4 <= kW4Region, "partial sums fit the wave's ring");
  __shared__ __align__(1024) uint8_t s_ring[4 * kW4Region];
  // offsets, and the inclusive count of experts with rows (16 bits: E <= 256),
  // so that two blocks with 3 ring buffers of 32 token rows per wave fit a CU
  __shared__ int s_off[256 + 1];
  __shared__ uint16_t s_cnt[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i <= E; i += blockDim.x) s_off[i] = offsets[i];
  __syncthreads();
  if (tid < E) s_cnt[tid] = (s_off[tid + 1] > s_off[tid]) ? 1 : 0;
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {
    const int add = (tid < E && tid >= d) ? s_cnt[tid - d] : 0;
    __syncthreads();
    if (tid < E) s_cnt[tid] = (uint16_t)(s_cnt[tid] + add);
    __syncthreads();
  }
  const int items = s_cnt[E - 1] * n_chunks;
  const int kw = K / 4;      // this wave's K range [wave*kw, wave*kw + kw)
  const int nch = kw / 64;   // chunks of 64 (an even number)
  const int G = K / 128;     // (scale, bias) groups per row
  uint8_t* ring = s_ring + wave * kW4Region;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void_t*)ring;
  float* s_part = reinterpret_cast<float*>(s_ring);  // wave w at + w * kW4Region / 4
  i32x4_t ract = dec_rsrc(act, act_bytes);
  asm volatile("" : "+s"(ract));
  const uint32_t c43 = 0x43434343u;

  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int rank = it / n_chunks, c = __builtin_amdgcn_readfirstlane(it - rank * n_chunks);
    int lo = 0, hi = E - 1;  // expert = the (rank+1)-th expert with rows
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_cnt[mid] > rank) hi = mid; else lo = mid + 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int r0 = s_off[e], r1 = s_off[e + 1];
    // weight rows of the item: gate/up rows [32c, 32c + 32) of both matrices,
    // down rows [64c, 64c + 64): 32-row blocks rb0 and rb1 of the codes and
    // (scale, bias) tiles (N_out is a multiple of 512)
    const int rb0 = GATEUP ? c : 2 * c, rb1 = GATEUP ? c : 2 * c + 1;
    const size_t blk0 = (size_t)e * (N_out / 32) + rb0, blk1 = (size_t)e * (N_out / 32) + rb1;
    const uint32_t qbytes = (uint32_t)K * 16u, sbytes = (uint32_t)G * 128u;  // per block
    i32x4_t rq0 = dec_rsrc(q0 + blk0 * qbytes, qbytes);
    i32x4_t rq1 = dec_rsrc((GATEUP ? q1 : q0) + blk1 * qbytes, qbytes);
    i32x4_t rs0 = dec_rsrc(reinterpret_cast<const uint8_t*>(sb0) + blk0 * sbytes, sbytes);
    i32x4_t rs1 = dec_rsrc(reinterpret_cast<const uint8_t*>(GATEUP ? sb1 : sb0) + blk1 * sbytes,
                           sbytes);
    // opaque to the compiler from here on: each descriptor stays one aligned
    // SGPR quad instead of being reassembled from shared fields at every load
    asm volatile("" : "+s"(rq0), "+s"(rq1), "+s"(rs0), "+s"(rs1));
    // lane l of a code DMA fills LDS row l / 2 (its slot l % 2 holding piece
    // (l % 2) ^ ((row >> 3) & 1)) from the 1 KB tile of the chunk; the
    // (scale, bias) DMA gives lane l row l % 32 of the group's 128 bytes
    const int qr = lane >> 1;
    const uint32_t q_lane = (uint32_t)(qr * 32 + (((lane & 1) ^ ((qr >> 3) & 1)) * 16)) +
                            (uint32_t)(wave * nch) * 1024u;
    const uint32_t q_off[2] = {q_lane, q_lane};
    const uint32_t s_lane = (uint32_t)((lane & 31) * 4) + (uint32_t)(wave * (nch / 2)) * 128u;
    const uint32_t s_off[2] = {s_lane, s_lane};
    for (int p0 = r0; p0 < r1; p0 += kW4Rows) {  // kW4Rows token rows per pass
      const int rows = min(r1 - p0, kW4Rows);
      uint32_t t_off[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 8 * j + (lane >> 3);  // token row of the pass
        int gi = p0 + t;
        gi = gi < r1 ? gi : r1 - 1;
        const int arow = GATEUP ? sorted_pair[gi] / k_top : gi;
        t_off[j] = ((uint32_t)arow * (uint32_t)K + (uint32_t)(wave * kw) +
                    (uint32_t)(((lane & 7) ^ swz_f<64>(t)) * 8)) * 2u;
      }
      // one pass with TG token groups of 8 rows loaded
      auto pass = [&](auto tg_c) {
        constexpr int NT = 1, TG = decltype(tg_c)::value;
        f32x16_t acc[NB][NT];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int tb = 0; tb < NT; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][tb][r] = 0.0f;
        const W4Loop<NT, TG> lp{ring, ring_lds, rq0, rq1, rs0, rs1, ract,
                                q_off, s_off, t_off, lane, c43};
        lp.run_k(nch, acc);
        // every ring buffer of this wave has landed and been read: its
        // partial sums may overwrite its ring
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        w4_epilogue<GATEUP, TG, kW4Region / 4>(acc, s_part, p0, rows, c, N_out, out);
      };
      if (rows > 24)
        pass(std::integral_constant<int, (kW4Rows > 24 ? 4 : 3)>{});
      else if (rows > 16)
        pass(std::integral_constant<int, 3>{});
      else if (rows > 8)
        pass(std::integral_constant<int, 2>{});
      else
        pass(std::integral_constant<int, 1>{});
      __syncthreads();  // the partial sums are read before the next pass loads
    }
  }
}

// The decode kernels take the block when the average expert has few rows.
// Their token operand is addressed with 32-bit byte offsets.
bool use_decode_path(const moe_config& c) {
  const long P = (long)c.num_tokens * c.top_k;
  return P <= 16L * c.num_experts && c.hidden % 256 == 0 && c.intermediate % 256 == 0 &&
         (long)c.num_tokens * c.hidden * 2 < (1L << 32) && P * c.intermediate * 2 < (1L << 32);
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
  // one block per possible row: rows past offsets[E] (pairs dropped by a
  // capacity limit) have no sorted_pair entry and are skipped
  if (i >= offsets[E]) return;
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
  if (i >= offsets[E]) return;  // no row (see gate_up_f32_kernel)
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

// Number of CUs of the current device, rounded to a multiple of 8 (the
// persistent grid is a multiple of it). Queried once per device and kept: a
// decode step launches four GEMMs in about 0.3 ms, and the attribute query
// costs host time on every launch otherwise. (A value computed twice by two
// threads is the same value.)
int persistent_grid() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int g = cached[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    g = (cus + 7) & ~7;
    cached[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

}  // namespace

// Weight loads of the tiled GEMMs with the non-temporal hint when one
// expert's matrix is large (64 MB or more, e.g. 8 experts x 14336 x 4096): its
// stream would otherwise push the token rows, which every column tile reads
// again, out of the MALL (-3.6% layer time at that shape). With small experts
// the hint costs the L2 reuse of weight tiles across row tiles (+4.8% at 128
// experts of 1536 x 4096), so it is off there.
static bool gemm_weights_streamed(size_t expert_bytes) { return expert_bytes >= ((size_t)64 << 20); }

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
  if (use_decode_path(c)) {
    const int nch = (c.intermediate + 31) / 32;
    decode_gemm_bf16_kernel<true><<<persistent_grid() * kDecOcc, 256, 0, s>>>(
        c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const uint16_t*>(x),
        (uint32_t)((size_t)c.num_tokens * c.hidden * 2), sorted_pair, offsets, static_cast<const uint16_t*>(w_gate),
        static_cast<const uint16_t*>(w_up), h, nch, DecSort{});
    return hipGetLastError();
  }
  const int ntn = (c.intermediate + 127) / 128;
  const size_t wexp = (size_t)2 * c.intermediate * c.hidden * 2;  // gate + up bytes per expert
#define MOE_GATE_UP(WNT)                                                                  \
  grouped_gemm_bf16_kernel<true, kGemmBM, kGemmBK, kGemmStages, kGemmWaves, kGemmOcc, WNT> \
      <<<persistent_grid() * kGemmOcc, 64 * kGemmWaves, 0, s>>>(                          \
          c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const uint16_t*>(x), \
          sorted_pair, offsets, static_cast<const uint16_t*>(w_gate),                    \
          static_cast<const uint16_t*>(w_up), h, ntn, nullptr)
  if (gemm_weights_streamed(wexp))
    MOE_GATE_UP(true);
  else
    MOE_GATE_UP(false);
#undef MOE_GATE_UP
  return hipGetLastError();
}

bool gate_up_sorts_itself(const moe_config& c) {
  const long P = (long)c.num_tokens * c.top_k;
  return c.dtype == MOE_DTYPE_BF16 && use_decode_path(c) && P <= kDispChunk &&
         c.num_experts <= 256 && persistent_grid() >= 2;
}

hipError_t launch_gate_up_sorting(const moe_config& c, const void* x, const int32_t* topk_idx,
                                  int capacity, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_pair, int32_t* pair_pos, int32_t* dropped,
                                  const AuxSmallArgs* aux, const void* w_gate, const void* w_up,
                                  void* h, hipStream_t s) {
  if (!gate_up_sorts_itself(c)) return hipErrorInvalidValue;
  DecSort ds{};
  ds.idx = topk_idx;
  ds.P = c.num_tokens * c.top_k;
  ds.cap = capacity;
  ds.counts = counts;
  ds.offsets = offsets;
  ds.sorted_pair = sorted_pair;
  ds.pair_pos = pair_pos;
  ds.dropped = dropped;
  ds.do_aux = aux ? 1 : 0;
  if (aux) ds.aux = *aux;
  const int nch = (c.intermediate + 31) / 32;
  decode_gemm_bf16_kernel<true, true><<<persistent_grid() * kDecOcc, 256, 0, s>>>(
      c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const uint16_t*>(x),
      (uint32_t)((size_t)c.num_tokens * c.hidden * 2), nullptr, nullptr,
      static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), h, nch, ds);
  return hipGetLastError();
}

hipError_t launch_down(const moe_config& c, const void* h, const int32_t* offsets,
                       const void* w_down, void* y, hipStream_t s, int8_t* y_exp,
                       bool* y_half) {
  if (y_half) *y_half = false;
  const int P = c.num_tokens * c.top_k;
  if (c.dtype == MOE_DTYPE_F32) {
    down_f32_kernel<<<P, 256, c.intermediate * sizeof(float), s>>>(
        c.num_experts, c.hidden, c.intermediate, static_cast<const float*>(h), offsets,
        static_cast<const float*>(w_down), static_cast<float*>(y));
    return hipGetLastError();
  }
  if (use_decode_path(c)) {
    const int nch = (c.hidden + 63) / 64;
    decode_gemm_bf16_kernel<false><<<persistent_grid() * kDecOcc, 256, 0, s>>>(
        c.num_experts, c.intermediate, c.hidden, c.top_k, static_cast<const uint16_t*>(h),
        (uint32_t)((size_t)P * c.intermediate * 2), nullptr, offsets, static_cast<const uint16_t*>(w_down), nullptr, y, nch, DecSort{});
    return hipGetLastError();
  }
  const int ntn = (c.hidden + 255) / 256;
  const size_t wexp = (size_t)c.hidden * c.intermediate * 2;  // down bytes per expert
#define MOE_DOWN(WNT)                                                                      \
  grouped_gemm_bf16_kernel<false, kGemmBM, kGemmBK, kGemmStages, kGemmWaves, kGemmOcc, WNT> \
      <<<persistent_grid() * kGemmOcc, 64 * kGemmWaves, 0, s>>>(                           \
          c.num_experts, c.intermediate, c.hidden, c.top_k, static_cast<const uint16_t*>(h),  \
          nullptr, offsets, static_cast<const uint16_t*>(w_down), nullptr, y, ntn, y_exp)
  if (gemm_weights_streamed(wexp))
    MOE_DOWN(true);
  else
    MOE_DOWN(false);
#undef MOE_DOWN
  if (y_exp && y_half) *y_half = true;
  return hipGetLastError();
}

// The 4-bit kernels address their token operand with 32-bit byte offsets.
bool w4_supported(const moe_config& c) {
  const long P = (long)c.num_tokens * c.top_k;
  return c.dtype == MOE_DTYPE_BF16 && c.hidden % 512 == 0 && c.intermediate % 512 == 0 &&
         (long)c.num_tokens * c.hidden * 2 < (1L << 32) && P * c.intermediate * 2 < (1L << 32);
}

hipError_t launch_gate_up_w4(const moe_config& c, const void* x, const int32_t* sorted_pair,
                             const int32_t* offsets, const moe_w4_weights& w, void* h,
                             hipStream_t s) {
  const int nch = (c.intermediate + 31) / 32;
  decode_w4_kernel<true><<<2 * persistent_grid(), 256, 0, s>>>(
      c.num_experts, c.hidden, c.intermediate, c.top_k, static_cast<const uint16_t*>(x),
      (uint32_t)((size_t)c.num_tokens * c.hidden * 2), sorted_pair, offsets, w.gate, static_cast<const uint16_t*>(w.gate_sb), w.up,
      static_cast<const uint16_t*>(w.up_sb), h, nch);
  return hipGetLastError();
}

hipError_t launch_down_w4(const moe_config& c, const void* h, const int32_t* offsets,
                          const moe_w4_weights& w, void* y, hipStream_t s) {
  const int nch = (c.hidden + 63) / 64;
  decode_w4_kernel<false><<<2 * persistent_grid(), 256, 0, s>>>(
      c.num_experts, c.intermediate, c.hidden, c.top_k, static_cast<const uint16_t*>(h),
      (uint32_t)((size_t)c.num_tokens * c.top_k * c.intermediate * 2), nullptr, offsets, w.down, static_cast<const uint16_t*>(w.down_sb), nullptr, nullptr, y,
      nch);
  return hipGetLastError();
}

}  // namespace moe
