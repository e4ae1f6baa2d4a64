// Grouped GEMM over the per-expert layout on gfx950 (MFMA), and its device-side tile
// metadata.
//
// "Add Triton grouped-GEMM for MoE experts on Ampere/Ada" (DeepSpeed PR 8180), "What
// this PR does": one kernel multiplies the 2D row block by a 3D weight stack using the
// per-group offsets, the tile -> group map is computed on the device from the offsets
// (no device -> host sync), and the weights stay in their native [E, N, K] layout.
// Here the groups are the experts of moe_dispatch_layout: rows [expert_offset[e],
// expert_offset[e] + expert_count[e]) of the slot-indexed expert inputs, and
//     y[r, n] = bf16( sum_k x[r, k] * w[e, n, k] ),   fp32 accumulation.
//
// gemm_tiles_kernel: one 1024-thread workgroup turns counts into row tiles (experts
// in ascending id, tile_m rows each, the last shorter); unused entries of the tile
// arrays get expert -1 so a GEMM grid sized by the host-side bound simply exits there.
//
// grouped_gemm_kernel / grouped_gemm_direct_kernel: one workgroup per (tile of up to 256
// rows, column block of 256, or of 128 when Nout is not a multiple of 256 or the grid
// would not fill the chip), details at the kernels.  The direct kernel (operands copied
// global -> LDS with no register staging) runs when K % 128 == 0 and the grid fills the
// chip; the register-staged one otherwise.  Both operands are K-contiguous ([rows, K] and [Nout, K]), which
// is what an MFMA lane needs: 8 consecutive k of one row or one column.  Accumulator lane
// layout of
// v_mfma_f32_32x32x16_bf16 (verified on the GPU): value v of lane l is
// C[8*(v/4) + 4*(l/32) + v%4][l%32]; operand lane l holds A[l%32][8*(l/32) + i] and
// B[8*(l/32) + i][l%32].
#include <type_traits>

#include "moe_internal.h"

namespace moedl {
namespace {

constexpr int kMaxBM = 256;  // rows per tile of moe_grouped_gemm_tiles (tile_m)
constexpr int kBK = 64;    // k per pipeline step
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource: no format, no swizzle
constexpr int kPadK = kBK + 8;  // LDS row pitch in bf16: 16-byte fragment reads of
                                // consecutive rows land in distinct bank groups

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(1024) void gemm_tiles_kernel(
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ expert_count,
    int32_t G, int32_t tile_m, int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_row0,
    int32_t* __restrict__ tile_rows, int32_t max_tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int32_t wave_sums[16];
  __shared__ int32_t total_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int e = tid;  // G <= 1024: one expert per thread
  const int cnt = e < G ? expert_count[e] : 0;
  const int nt = cnt > 0 ? (cnt + tile_m - 1) / tile_m : 0;
  // exclusive scan of the per-expert tile counts, ascending expert id
  int incl = nt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int q = 0; q < 16; ++q) {
      const int s = wave_sums[q];
      wave_sums[q] = run;
      run += s;
    }
    total_s = run;
    num_tiles[0] = min(run, max_tiles);
  }
  __syncthreads();
  const int first = wave_sums[w] + incl - nt;
  if (e < G) {
    const int off = expert_offset[e];
    for (int i = 0; i < nt && first + i < max_tiles; ++i) {
      tile_expert[first + i] = e;
      tile_row0[first + i] = off + i * tile_m;
      tile_rows[first + i] = min(tile_m, cnt - i * tile_m);
    }
  }
  for (int t = total_s + tid; t < max_tiles; t += 1024) tile_expert[t] = -1;
}

// Workgroup -> (row tile, column block): row tile major, column blocks fastest, so the
// workgroups of one row tile are dispatched together and share its x rows while
// consecutive tiles of an expert reuse its weight columns.  Measured on the Zipf layout
// (131072 rows, K = 7168, Nout = 2048), this plain order beats XCD-aware remaps that
// give each XCD a contiguous range, with or without grouping 4 to 32 tiles per
// column-block sweep (992 vs 714..947 TFLOP/s in the same run).
__device__ __forceinline__ void gemm_block_order(int bid, int nblk, int* tile, int* jblk) {
  *tile = bid / nblk;
  *jblk = bid - *tile * nblk;
}

// One tile body = BM rows (128 or 256) x BN columns, 2 * BN / 64 waves: wave (wm, wn)
// owns the BM/2 x 64 output block at rows wm*BM/2, columns wn*64, i.e. BM/64 x 2
// accumulator blocks of 32 x 32.  With BN = 256 that is 8 waves, two per SIMD.
// What bounds it (measured on the Zipf layout with 128-row tiles, random bf16): the
// kernel runs at ~0.87 PFLOP/s; with the global loads replaced by register constants
// (LDS writes kept) at 1.38, with every load redirected to one tile so that all hit in
// L2 at 1.11, and with the LDS writes dropped at 0.98.  So the global loads set the
// rate, about half through the bytes each CU moves per flop and half through L2 misses
// to the fabric.  Hence the 256-row body for full tiles: a third fewer bytes per flop.
// With it (same process, outputs bit-identical): uniform layout 948 -> 1019 TFLOP/s,
// Zipf 884 -> 904 (most Zipf experts have under 256 rows).
// Short tiles (an expert's last rows): x is read through a buffer resource whose size
// ends at the tile's last row, so rows past the end come back as zeros with no memory
// traffic and every load stays unconditional.  (Skipping the MFMAs of 32-row blocks
// past the end was measured slower: the branch splits the MFMA / load interleave.)
// Per 64-wide k step s: the MFMAs read LDS buffer s%2 (rows padded to 72 bf16: the
// 16-byte fragment reads of consecutive rows hit distinct bank groups; fragments are
// double-buffered in registers across the four 16-wide k slices) while the tile of step
// s+1, loaded into registers during step s-2, is written to buffer (s+1)%2 and the tile
// of step s+3 is loaded into the registers it leaves: two register sets give the loads
// two steps to arrive (2-3% faster than one step ahead, bit-identical output; the
// 256-row body keeps one set, loading step s+2, for lack of registers).  A wave
// issues in order, so those LDS writes and global loads are placed between the MFMA
// groups of the k slices (sched_barrier fences keep them there): the address unit then
// works while the matrix cores do.  Issued after all of a step's MFMAs instead, they
// form one burst per step that the matrix cores wait through.  The loop body has no
// branches (steps run in pairs so each register set is static; the last steps are
// peeled), which keeps the compiler's memory wait counts exact.  One barrier per step
// orders the two LDS buffers.
template <int BM, int BN, int NSETS>
__device__ __forceinline__ void gemm_tile(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wb, int32_t K, int32_t Nout,
    int r0, int nrows, int n0, uint16_t (&As)[2][kMaxBM * kPadK],
    uint16_t (&Bs)[2][BN * kPadK], uint16_t* __restrict__ y) {
  constexpr int NT = 2 * BN;                // threads
  constexpr int RS = NT / 8;                // rows staged per pass (8 threads per row)
  constexpr int AP = BM / RS;               // x rows per thread per step
  constexpr int BP = BN / RS;               // w rows per thread per step
  constexpr int WR = BM / 2;                // rows per wave
  constexpr int I = WR / 32, J = 2;         // 32 x 32 blocks per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int wm = w & 1, wn = w >> 1;

  // x through a buffer resource ending at the tile's last row: loads past it read 0
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)r0 * K), (short)0, nrows * K * 2, kBufferWord3);

  // global -> register staging: thread t moves the 16-byte chunk (t % 8) of rows
  // t / 8 + RS p; eight consecutive threads cover one row's 128 bytes.  With two
  // register sets the tile of step s+1 is in set (s+1)%2 and that of step s+2 in set
  // s%2; with one, the set holds the tile of step s+1 until it is written to LDS.
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;
  u32x4 ra[NSETS][AP], rb[NSETS][BP];
  auto load_a = [&](int set, int k0) {
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const int row = lrow + p * RS;
      ra[set][p] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (row * K + k0 + lcol) * 2, 0, 0));
    }
  };
  auto load_b = [&](int set, int k0, int p0, int p1) {
#pragma unroll
    for (int p = 0; p < BP; ++p)
      if (p >= p0 && p < p1)
        rb[set][p] = *(const u32x4*)(wb + (int64_t)(lrow + p * RS) * K + k0 + lcol);
  };
  auto store_a = [&](int set, int buf) {
#pragma unroll
    for (int p = 0; p < AP; ++p) *(u32x4*)(&As[buf][(lrow + p * RS) * kPadK + lcol]) = ra[set][p];
  };
  auto store_b = [&](int set, int buf) {
#pragma unroll
    for (int p = 0; p < BP; ++p) *(u32x4*)(&Bs[buf][(lrow + p * RS) * kPadK + lcol]) = rb[set][p];
  };

  f32x16_t acc[I][J];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[i][j] = (f32x16_t){};

  const int steps = K / kBK;
  if constexpr (NSETS == 2) {
    load_a(0, 0);
    load_b(0, 0, 0, BP);
    if (steps > 1) {
      load_a(1, kBK);
      load_b(1, kBK, 0, BP);
    }
    store_a(0, 0);
    store_b(0, 0);
    if (steps > 2) {
      load_a(0, 2 * kBK);
      load_b(0, 2 * kBK, 0, BP);
    }
  } else {
    load_a(0, 0);
    load_b(0, 0, 0, BP);
    store_a(0, 0);
    store_b(0, 0);
    if (steps > 1) {
      load_a(0, kBK);
      load_b(0, kBK, 0, BP);
    }
  }
  __syncthreads();
  // One k step on LDS buffer s%2.  NEXT: the tile of step s+1 (in register set SET) is
  // written to the other buffer; LOAD: the tile of step s + NSETS + 1 is then loaded
  // into that set.  The loops below run with both set and no branches in their bodies,
  // so the compiler's wait counts stay exact; the last steps are peeled.
  auto step = [&](int s, auto set_c, auto next_c, auto load_c) {
    constexpr int SET = decltype(set_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool LOAD = decltype(load_c)::value;
    const int buf = s & 1;
    const int kl = (s + NSETS + 1) * kBK;
    const uint16_t* Ab = As[buf] + (wm * WR + (lane & 31)) * kPadK + (lane >> 5) * 8;
    const uint16_t* Bb = Bs[buf] + (wn * 64 + (lane & 31)) * kPadK + (lane >> 5) * 8;
    bf16x8_t af[2][I], bfr[2][J];
    auto load_frags = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < I; ++i) af[slot][i] = *(const bf16x8_t*)(Ab + i * 32 * kPadK + kk * 16);
#pragma unroll
      for (int j = 0; j < J; ++j) bfr[slot][j] = *(const bf16x8_t*)(Bb + j * 32 * kPadK + kk * 16);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < I; ++i)
#pragma unroll
        for (int j = 0; j < J; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j],
                                                              0, 0, 0);
    };
    load_frags(0, 0);
    // k slice 0: write the x part of step s+1, then load the x part of a later step
    load_frags(1, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) store_a(SET, buf ^ 1);
    if constexpr (LOAD) load_a(SET, kl);
    __builtin_amdgcn_sched_barrier(0);
    // k slice 1: write the w part of step s+1, load half of the later step's w part
    load_frags(2, 0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) store_b(SET, buf ^ 1);
    if constexpr (LOAD) load_b(SET, kl, 0, BP / 2);
    __builtin_amdgcn_sched_barrier(0);
    // k slice 2: the other half of the w loads
    load_frags(3, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LOAD) load_b(SET, kl, BP / 2, BP);
    __builtin_amdgcn_sched_barrier(0);
    // k slice 3
    mfmas(1);
    __syncthreads();
  };
  using yes = std::true_type;
  using no = std::false_type;
  using set0 = std::integral_constant<int, 0>;
  using set1 = std::integral_constant<int, 1>;
  if constexpr (NSETS == 2) {
    // pairs of steps (s even, then s + 1), so the register set of each is static
    int s = 0;
    for (; s + 4 < steps; s += 2) {
      step(s, set1{}, yes{}, yes{});
      step(s + 1, set0{}, yes{}, yes{});
    }
    switch (steps - s) {  // 1 to 4 steps left, s even
      case 4:
        step(s, set1{}, yes{}, yes{});
        step(s + 1, set0{}, yes{}, no{});
        step(s + 2, set1{}, yes{}, no{});
        step(s + 3, set0{}, no{}, no{});
        break;
      case 3:
        step(s, set1{}, yes{}, no{});
        step(s + 1, set0{}, yes{}, no{});
        step(s + 2, set1{}, no{}, no{});
        break;
      case 2:
        step(s, set1{}, yes{}, no{});
        step(s + 1, set0{}, no{}, no{});
        break;
      default:
        step(s, set1{}, no{}, no{});
        break;
    }
  } else {
    int s = 0;
    for (; s + 2 < steps; ++s) step(s, set0{}, yes{}, yes{});
    if (s + 1 < steps) step(s++, set0{}, yes{}, no{});
    step(s, set0{}, no{}, no{});
  }

  // epilogue: fp32 -> bf16 (round to nearest even), rows past the tile end skipped
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WR + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < nrows)
          y[(int64_t)(r0 + row) * Nout + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
      }
}

// Workgroup -> (tile, column block) -> one of two tile bodies.  Tiles hold up to 256 rows
// (moe_grouped_gemm_tiles with tile_m = 256): a tile of more than 128 rows runs the
// 256-row body, which moves a third fewer bytes per flop, with one register set (two
// would not fit beside its accumulators); a tile of at most 128 rows runs the 128-row
// body with two register sets.  An expert's rows are thus padded to a multiple of 128,
// as with 128-row tiles, while its full 256-row blocks take the cheaper body.  The
// branch is uniform over the workgroup and taken once.  SPLIT (grids too small to fill
// the chip): two workgroups per tile, each running the 128-row body on one half.
template <int BN, bool SPLIT>
__global__ __launch_bounds__(2 * BN) void grouped_gemm_kernel(
    const uint16_t* __restrict__ x, int64_t rows, const uint16_t* __restrict__ wgt, int32_t G,
    int32_t K, int32_t Nout, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ tile_rows,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kMaxBM * kPadK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kPadK];
  int tile, jblk, half = 0;
  if constexpr (SPLIT) {
    int unit;
    gemm_block_order(blockIdx.x, Nout / BN, &unit, &jblk);
    tile = unit >> 1;
    half = unit & 1;
  } else {
    gemm_block_order(blockIdx.x, Nout / BN, &tile, &jblk);
  }
  // Uniform exits: past the last tile (expert -1), or metadata that names no expert or
  // no row of x.  Rows are clipped to [0, rows), so whatever the tile arrays hold,
  // every access stays inside x, w and y.
  const int e = tile_expert[tile];
  if (e < 0 || e >= G) return;
  int r0 = tile_row0[tile];
  if (r0 < 0 || r0 >= rows) return;
  int nrows = (int)min((int64_t)min(tile_rows[tile], kMaxBM), rows - r0);
  const int n0 = jblk * BN;
  const uint16_t* wb = wgt + ((int64_t)e * Nout + n0) * K;
  if constexpr (SPLIT) {
    r0 += half * (kMaxBM / 2);
    nrows = min(nrows - half * (kMaxBM / 2), kMaxBM / 2);
    if (nrows < 1) return;
    gemm_tile<kMaxBM / 2, BN, 2>(x, wb, K, Nout, r0, nrows, n0, As, Bs, y);
  } else {
    if (nrows < 1) return;
    if (nrows > kMaxBM / 2)
      gemm_tile<kMaxBM, BN, 1>(x, wb, K, Nout, r0, nrows, n0, As, Bs, y);
    else
      gemm_tile<kMaxBM / 2, BN, 2>(x, wb, K, Nout, r0, nrows, n0, As, Bs, y);
  }
}

// ------------------------------------------------- direct-to-LDS body (K % 128 == 0)
// The same tile (BM rows x BN columns, 2 * BN / 64 waves, wave (wm, wn) owning BM/2 x 64)
// and the same MFMA sequence per output element as gemm_tile, so the outputs are
// identical bit for bit; only the way the operands reach LDS differs.  Each 64-wide k
// step of x and w is copied global -> LDS by buffer_load ... lds (16 bytes per lane, no
// registers, no LDS write instructions): one wave instruction fills 1 KiB of LDS, lane L
// at byte 16 L, which is 8 rows of 128 bytes.  The rows are not padded; instead lane L
// fetches the global chunk (L % 8) ^ ((row >> 1) & 7) of its row, an XOR swizzle under
// which the 16 lanes of each fragment read group hit 16 distinct 16-byte bank slots.
// Two LDS stages, each its own array so the compiler can tell a fragment read of one
// stage from the loads in flight into the other: step s waits for its own loads (issued
// during step s - 1), passes the barrier, issues step s + 1 into the other stage and runs
// its MFMAs.  Measured (Zipf layout, 131072 rows, K 7168 -> 2048; the register-staged
// body, same run): loads kept but fragment reads dropped 1.07 PFLOP/s, fragment reads
// kept but loads dropped 1.68, MFMAs alone 2.02, so the global loads still set the rate;
// four stages of k = 32 (loads three steps ahead) ran slower than two stages of 64.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kChunkBf16 = 8;  // bf16 per 16-byte chunk

template <int BM, int BN>
__device__ __forceinline__ void gemm_tile_direct(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wb, int32_t K, int32_t Nout,
    int r0, int nrows, int n0, uint16_t (&A0)[kMaxBM * kBK], uint16_t (&A1)[kMaxBM * kBK],
    uint16_t (&B0)[BN * kBK], uint16_t (&B1)[BN * kBK], uint16_t* __restrict__ y) {
  constexpr int NWV = 2 * BN / 64;         // waves
  constexpr int QA = BM / 8, QB = BN / 8;  // 8-row (1 KiB) load instructions per stage
  static_assert(QA % NWV == 0 && QB % NWV == 0, "whole load instructions per wave");
  constexpr int PA = QA / NWV, PB = QB / NWV;
  constexpr int WR = BM / 2;
  constexpr int I = WR / 32, J = 2;
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int wm = w & 1, wn = w >> 1;

  // x through a buffer resource ending at the tile's last row (loads past it read 0),
  // w through one covering the BN x K block
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)r0 * K), (short)0, nrows * K * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wb, (short)0, BN * K * 2, kBufferWord3);
  (void)xr;  // the loads that use them exist in the device pass only
  (void)wr;
  // wave w issues instructions q = w, w + NWV, ...; lane L of instruction q loads row
  // 8 q + L / 8, global chunk (L % 8) ^ swizzle: byte offsets at k = 0
  const int lr = lane >> 3, pos = lane & 7;
  int va[PA], vb[PB];
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const int row = (p * NWV + w) * 8 + lr;
    va[p] = (row * K + (pos ^ ((row >> 1) & 7)) * kChunkBf16) * 2;
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int row = (p * NWV + w) * 8 + lr;
    vb[p] = (row * K + (pos ^ ((row >> 1) & 7)) * kChunkBf16) * 2;
  }
  auto issue = [&](auto stage_c, int k0) {
#if defined(__HIP_DEVICE_COMPILE__)  // LDS address-space pointers exist in the device pass only
    constexpr int ST = decltype(stage_c)::value;
    uint16_t* Ad = ST == 0 ? A0 : A1;
    uint16_t* Bd = ST == 0 ? B0 : B1;
#pragma unroll
    for (int p = 0; p < PA; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(Ad + (p * NWV + w) * 8 * kBK), 16,
                                               va[p] + k0 * 2, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < PB; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)(Bd + (p * NWV + w) * 8 * kBK), 16,
                                               vb[p] + k0 * 2, 0, 0, 0);
#endif
  };

  f32x16_t acc[I][J];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[i][j] = (f32x16_t){};

  // fragment reads: row R = (multiple of 32) + lane % 32, so the swizzle of every row a
  // lane reads is (lane >> 1) & 7; k slice kk holds chunks 2 kk (lanes 0-31), 2 kk + 1
  const int sw = (lane >> 1) & 7, hi = lane >> 5;
  auto step = [&](int s, auto stage_c, auto next_c) {
    constexpr int ST = decltype(stage_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const uint16_t* As = ST == 0 ? A0 : A1;
    const uint16_t* Bs = ST == 0 ? B0 : B1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this step's loads are in LDS
    __syncthreads();                                   // everyone's are; stage ST^1 is free
    if constexpr (NEXT) issue(std::integral_constant<int, ST ^ 1>{}, (s + 1) * kBK);
    const uint16_t* Ab = As + (wm * WR + (lane & 31)) * kBK;
    const uint16_t* Bb = Bs + (wn * 64 + (lane & 31)) * kBK;
    bf16x8_t af[2][I], bfr[2][J];
    auto load_frags = [&](int kk, int slot) {
      const int off = ((kk * 2 + hi) ^ sw) * kChunkBf16;
#pragma unroll
      for (int i = 0; i < I; ++i) af[slot][i] = *(const bf16x8_t*)(Ab + i * 32 * kBK + off);
#pragma unroll
      for (int j = 0; j < J; ++j) bfr[slot][j] = *(const bf16x8_t*)(Bb + j * 32 * kBK + off);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < I; ++i)
#pragma unroll
        for (int j = 0; j < J; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j],
                                                              0, 0, 0);
    };
    // fragments double-buffered across the four 16-wide k slices; the fences keep the
    // compiler from hoisting all of a step's reads (and their registers) to its start
    load_frags(0, 0);
    load_frags(1, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(2, 0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(3, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
  };
  using yes = std::true_type;
  using no = std::false_type;
  using st0 = std::integral_constant<int, 0>;
  using st1 = std::integral_constant<int, 1>;
  // steps run in pairs so each stage is static, and the last pair is peeled, so there
  // is no branch between loop and epilogue (an odd tail merged there made the compiler
  // shuffle the accumulators through scratch): hence K % 128 == 0
  const int steps = K / kBK;
  issue(st0{}, 0);
  int s = 0;
  for (; s + 2 < steps; s += 2) {
    step(s, st0{}, yes{});
    step(s + 1, st1{}, yes{});
  }
  step(s, st0{}, yes{});
  step(s + 1, st1{}, no{});

#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WR + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < nrows)
          y[(int64_t)(r0 + row) * Nout + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
      }
}

// Workgroup -> (tile, column block) for the direct body: the column blocks of one tile
// run on one XCD and consecutive tiles on consecutive XCDs (workgroups are handed to the
// 8 XCDs round-robin), so a tile's x rows are fetched into one L2 and shared by its
// column blocks.  The grid covers the tile count rounded up to 8; workgroups past
// max_tiles exit.  Measured against the row-tile-major order of the register-staged
// body (same run): Zipf 925 -> 952 TFLOP/s, uniform 904 -> 952, 64 experts x 1024 rows
// (K 2048 -> 1024) 833 -> 899, 8 x 4096 rows (K 4096 -> 1024) 878 -> 865.  Contiguous
// tile ranges per XCD did no better, and ranges cut from the host's max_tiles bound
// (which exceeds the real count) left the last XCDs idle: 833 on Zipf.
template <int BN>
__global__ __launch_bounds__(2 * BN) void grouped_gemm_direct_kernel(
    const uint16_t* __restrict__ x, int64_t rows, const uint16_t* __restrict__ wgt, int32_t G,
    int32_t K, int32_t Nout, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ tile_rows,
    int32_t max_tiles, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t A0[kMaxBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t A1[kMaxBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t B0[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t B1[BN * kBK];
  const int nblk = Nout / BN;
  const int xcd = blockIdx.x & 7;
  const int l = blockIdx.x >> 3;
  const int tile = (l / nblk) * 8 + xcd;
  const int jblk = l - (l / nblk) * nblk;
  if (tile >= max_tiles) return;
  // the same uniform exits and clipping as grouped_gemm_kernel
  const int e = tile_expert[tile];
  if (e < 0 || e >= G) return;
  const int r0 = tile_row0[tile];
  if (r0 < 0 || r0 >= rows) return;
  const int nrows = (int)min((int64_t)min(tile_rows[tile], kMaxBM), rows - r0);
  if (nrows < 1) return;
  const int n0 = jblk * BN;
  const uint16_t* wb = wgt + ((int64_t)e * Nout + n0) * K;
  if (nrows > kMaxBM / 2)
    gemm_tile_direct<kMaxBM, BN>(x, wb, K, Nout, r0, nrows, n0, A0, A1, B0, B1, y);
  else
    gemm_tile_direct<kMaxBM / 2, BN>(x, wb, K, Nout, r0, nrows, n0, A0, A1, B0, B1, y);
}

}  // namespace

hipError_t launch_gemm_tiles(const int32_t* expert_offset, const int32_t* expert_count, int32_t G,
                             int32_t tile_m, int32_t* tile_expert, int32_t* tile_row0,
                             int32_t* tile_rows, int32_t max_tiles, int32_t* num_tiles,
                             hipStream_t stream) {
  hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, stream, expert_offset,
                     expert_count, G, tile_m, tile_expert, tile_row0, tile_rows, max_tiles,
                     num_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint16_t* x, int64_t rows, const uint16_t* w, int32_t G,
                               int32_t K, int32_t Nout, const int32_t* tile_expert,
                               const int32_t* tile_row0, const int32_t* tile_rows,
                               int32_t max_tiles, uint16_t* y, hipStream_t stream) {
  if (max_tiles == 0) return hipSuccess;
  // Three launch shapes, by how far the grid fills the chip's 256 CUs (the host knows
  // only the bound max_tiles):
  //  - 256-column blocks move the fewest bytes per flop: used when that grid has at
  //    least one workgroup per CU;
  //  - else 128-column blocks, which double the grid;
  //  - else 128-column blocks with each tile split over two workgroups (128 rows each),
  //    four times the 256-column grid.
  // Measured on MI355X, same outputs bit for bit: 16 experts x 760 rows, K 2048 -> 768:
  // 25.0 us with 256-column blocks vs 19.8 with 128-column ones; 8 x 4096 rows, 4096 ->
  // 1024: 60 vs 54 us; but 64 x 8192 rows, 2048 -> 1024 (256 workgroups): 70 vs 81 us,
  // hence the switch at the CU count.
  // With K % 128 == 0 the first two shapes run the direct-to-LDS body (identical
  // outputs); the split shape always runs the register-staged one, which was faster
  // there (16 x 760 rows: 21.7 vs 25.7 us).
  constexpr int64_t kCUs = 256;
  const int64_t grid256 = Nout % 256 == 0 ? (int64_t)max_tiles * (Nout / 256) : 0;
  const int64_t grid128 = (int64_t)max_tiles * (Nout / 128);
  const int64_t tiles8 = ((int64_t)max_tiles + 7) / 8 * 8;
  if (K % (2 * kBK) == 0 && grid256 >= kCUs) {
    hipLaunchKernelGGL((grouped_gemm_direct_kernel<256>), dim3((unsigned)(tiles8 * (Nout / 256))),
                       dim3(512), 0, stream, x, rows, w, G, K, Nout, tile_expert, tile_row0,
                       tile_rows, max_tiles, y);
  } else if (K % (2 * kBK) == 0 && grid128 >= kCUs) {
    hipLaunchKernelGGL((grouped_gemm_direct_kernel<128>), dim3((unsigned)(tiles8 * (Nout / 128))),
                       dim3(256), 0, stream, x, rows, w, G, K, Nout, tile_expert, tile_row0,
                       tile_rows, max_tiles, y);
  } else if (grid256 >= kCUs) {
    hipLaunchKernelGGL((grouped_gemm_kernel<256, false>), dim3((unsigned)grid256), dim3(512), 0,
                       stream, x, rows, w, G, K, Nout, tile_expert, tile_row0, tile_rows, y);
  } else if (grid128 >= kCUs) {
    hipLaunchKernelGGL((grouped_gemm_kernel<128, false>), dim3((unsigned)grid128), dim3(256), 0,
                       stream, x, rows, w, G, K, Nout, tile_expert, tile_row0, tile_rows, y);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<128, true>), dim3((unsigned)(2 * grid128)), dim3(256),
                       0, stream, x, rows, w, G, K, Nout, tile_expert, tile_row0, tile_rows, y);
  }
  return hipGetLastError();
}

}  // namespace moedl
