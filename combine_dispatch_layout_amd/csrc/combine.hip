// Combine on gfx950: y[t] = bf16( sum_j w[t,j] * expert_out[slot[t,j]] ).
//
// Determinism follows "Purlin: Separating Orchestration from the Datapath of
// Collectives", section 3.3 (SCORE): exactly one lane owns each output element and
// accumulates its k sources in source order (j ascending), each step one rounded
// fp32 multiply and one rounded fp32 add (this file is built without FP
// contraction), starting from +0.0, then one round-to-nearest-even to bf16
// (v_cvt_pk_bf16_f32).  The result is bitwise reproducible and independent of the
// launch geometry.  As in that section's pipelined reduction, the sources are
// fetched concurrently and consumed in source order.
//
// Mapping (LDS-staged).  A row is cut into 1 KiB pieces (64 lanes x 16 bytes = 512
// bf16).  One workgroup owns one (token, piece) and has NW = k/2 wave64s: wave w fetches
// the piece of source rows j = w, w + NW, ... into LDS (one 16-byte non-temporal
// load per lane per row), then wave 0 reads the k staged vectors back in j order,
// accumulates in fp32 and stores the 16-byte bf16 result (non-temporal).
//
// Why this shape: measured on MI355X at 16384 tokens x 14 KiB x 8 sources, one wave
// that loads all k sources of a piece and stores the result sustains ~6.0 TB/s; the
// same with k/2 waves of two loads each, joined through LDS, ~6.2 TB/s (1, 2 or 8
// loading waves do no better).  A read-only pass over the same scattered rows runs
// at ~6.9 TB/s: the mix of scattered reads with the output write stream is what
// limits HBM efficiency here; the arithmetic is hidden behind the loads.
#include "moe_internal.h"

#pragma clang fp contract(off)

namespace moedl {
namespace {

constexpr int kPieceVecs = 64;

template <int K, int NW>
__global__ __launch_bounds__(64 * NW) void combine_piece_kernel(
    const u32x4* __restrict__ eo, int64_t expert_rows, const float* __restrict__ wts,
    const int32_t* __restrict__ slot, int64_t M, int32_t row_vecs, int32_t pieces,
    u32x4* __restrict__ y) {
  __shared__ u32x4 stage[K][64];
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;  // uniform over the workgroup
  const int c = piece * kPieceVecs + lane;
  const int32_t* srow = slot + t * K;

  // Branch-free loads, so all H loads of a lane are in flight together: a lane past
  // the row end, or a source outside [0, expert_rows), reads an in-bounds address
  // (its own output position) and the value is replaced by zero.
  constexpr int H = (K + NW - 1) / NW;  // source rows per wave
  const int cc = c < row_vecs ? c : row_vecs - 1;
  const u32x4* fallback = (const u32x4*)y + t * row_vecs + cc;
  u32x4 d[H];
  bool ok[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int j = w + h * NW;
    const int s = j < K ? srow[j] : -1;
    ok[h] = s >= 0 && s < expert_rows && c < row_vecs;
    const u32x4* src = (s >= 0 && s < expert_rows) ? eo + (int64_t)s * row_vecs + cc : fallback;
    d[h] = __builtin_nontemporal_load(src);
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int j = w + h * NW;
    if (j < K) stage[j][lane] = ok[h] ? d[h] : (u32x4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (w != 0 || c >= row_vecs) return;

  // Source order, unfused.  A skipped source contributes w = 0 times a zero vector:
  // +0, and the accumulator is never -0 (it starts at +0 and IEEE sums that cancel
  // round to +0), so adding +0 leaves it unchanged -- the same result as skipping.
  const float* wrow = wts + t * K;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int s = srow[j];
    const float wj = (s >= 0 && s < expert_rows) ? wrow[j] : 0.0f;
    const u32x4 v = stage[j][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t u = v[q];
      const float lo = __builtin_bit_cast(float, u << 16);
      const float hi = __builtin_bit_cast(float, u & 0xFFFF0000u);
      const float plo = wj * lo;
      const float phi = wj * hi;
      acc[2 * q] = acc[2 * q] + plo;
      acc[2 * q + 1] = acc[2 * q + 1] + phi;
    }
  }
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  __builtin_nontemporal_store(o, y + t * row_vecs + c);
}

template <int K>
hipError_t launch_k(const uint16_t* expert_out, int64_t expert_rows, const float* weights,
                    const int32_t* slot, int64_t M, int32_t row_vecs, uint16_t* y,
                    hipStream_t stream) {
  constexpr int NW = K >= 2 ? K / 2 : 1;  // two source rows per wave
  const int32_t pieces = (row_vecs + kPieceVecs - 1) / kPieceVecs;
  const int64_t blocks = M * pieces;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_piece_kernel<K, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                     stream, (const u32x4*)expert_out, expert_rows, weights, slot, M,
                     row_vecs, pieces, (u32x4*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* expert_out, int64_t expert_rows, const float* weights,
                          const int32_t* slot, int64_t M, int32_t k, int32_t N, uint16_t* y,
                          hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = N / 8;
#define MOEDL_CASE(K) \
  case K:             \
    return launch_k<K>(expert_out, expert_rows, weights, slot, M, row_vecs, y, stream);
  switch (k) {
    MOEDL_CASE(1) MOEDL_CASE(2) MOEDL_CASE(3) MOEDL_CASE(4) MOEDL_CASE(5) MOEDL_CASE(6)
    MOEDL_CASE(7) MOEDL_CASE(8) MOEDL_CASE(9) MOEDL_CASE(10) MOEDL_CASE(11) MOEDL_CASE(12)
    MOEDL_CASE(13) MOEDL_CASE(14) MOEDL_CASE(15) MOEDL_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOEDL_CASE
}

}  // namespace moedl
