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
// grouped_gemm_kernel: one 256-thread workgroup per (row tile, 128-column block).
//  - Grid: one linear index, column blocks fastest (max_tiles * Nout / 128 groups).
//  - Both operands are K-contiguous ([rows, K] and [Nout, K]), which is what an MFMA
//    lane needs: 8 consecutive k of one row / one column.
//  - Per 64-wide k step the workgroup stages a 128 x 64 tile of x and of w in LDS
//    (rows padded to 72 bf16 so the 16-byte fragment reads of 8 consecutive rows hit
//    distinct bank groups), while the next step's tiles are already loading into
//    registers.
//  - The four waves form a 2 x 2 grid of 64 x 64 output blocks; each wave runs
//    2 x 2 v_mfma_f32_32x32x16_bf16 per 16-wide k slice (64 fp32 accumulators per
//    lane).  Accumulator lane layout (verified on the GPU): value v of lane l is
//    C[8*(v/4) + 4*(l/32) + v%4][l%32]; operand lane l holds A[l%32][8*(l/32) + i] and
//    B[8*(l/32) + i][l%32].
//  - Rows past the tile's end read as zero and are not stored.
#include "moe_internal.h"

namespace moedl {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kPadK = kBK + 8;  // LDS row pitch in bf16

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

__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgt, int32_t K, int32_t Nout,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ tile_rows, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kPadK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kPadK];
  // one linear grid, column blocks fastest: the workgroups of one row tile are
  // dispatched back to back and share its x rows in cache
  const int nblk = Nout / kBN;
  const int tile = blockIdx.x / nblk;
  const int e = tile_expert[tile];
  if (e < 0) return;  // uniform: past the last tile
  const int r0 = tile_row0[tile];
  const int nrows = min(tile_rows[tile], kBM);
  const int n0 = (blockIdx.x - tile * nblk) * kBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int wm = w >> 1, wn = w & 1;

  const uint16_t* xa = x + (int64_t)r0 * K;
  const uint16_t* wb = wgt + ((int64_t)e * Nout + n0) * K;

  // global -> register staging: 4 rows x 16 bytes of A and of B per thread per step
  const int lrow = tid >> 3;        // 0..31
  const int lcol = (tid & 7) * 8;   // bf16 column of the 16-byte chunk
  u32x4 ra[4], rb[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = lrow + p * 32;
      const int rc = row < nrows ? row : nrows - 1;  // clamped: the load is unconditional
      ra[p] = *(const u32x4*)(xa + (int64_t)rc * K + k0 + lcol);
      rb[p] = *(const u32x4*)(wb + (int64_t)row * K + k0 + lcol);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = lrow + p * 32;
      *(u32x4*)(As + row * kPadK + lcol) = row < nrows ? ra[p] : (u32x4){0u, 0u, 0u, 0u};
      *(u32x4*)(Bs + row * kPadK + lcol) = rb[p];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};

  load_tiles(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();  // previous step's fragments are consumed
    store_tiles();
    __syncthreads();
    if (k0 + kBK < K) load_tiles(k0 + kBK);  // in flight during the MFMAs below
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kc = kk * 16 + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        af[i] = *(const bf16x8_t*)(As + row * kPadK + kc);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8_t*)(Bs + col * kPadK + kc);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: fp32 -> bf16 (round to nearest even), rows past the tile end skipped
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < nrows)
          y[(int64_t)(r0 + row) * Nout + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
      }
}

}  // namespace

int32_t gemm_tile_rows() { return kBM; }

hipError_t launch_gemm_tiles(const int32_t* expert_offset, const int32_t* expert_count, int32_t G,
                             int32_t tile_m, int32_t* tile_expert, int32_t* tile_row0,
                             int32_t* tile_rows, int32_t max_tiles, int32_t* num_tiles,
                             hipStream_t stream) {
  hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, stream, expert_offset,
                     expert_count, G, tile_m, tile_expert, tile_row0, tile_rows, max_tiles,
                     num_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint16_t* x, const uint16_t* w, int32_t K, int32_t Nout,
                               const int32_t* tile_expert, const int32_t* tile_row0,
                               const int32_t* tile_rows, int32_t max_tiles, uint16_t* y,
                               hipStream_t stream) {
  if (max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)(max_tiles * (Nout / kBN))), dim3(256), 0,
                     stream, x, w,
                     K, Nout, tile_expert, tile_row0, tile_rows, y);
  return hipGetLastError();
}

}  // namespace moedl
