// Receiver-side expansion of dedup rows and the per-(token, bucket) pre-reduced
// combine, on gfx950.
//
// In dedup mode a (token, destination bucket) pair travels as one row ("Zyphra says
// routing-pattern expert placement ...", the copy-reduction item).  Around the path:
//  - moe_expand (receiver): expert_in[slot[t,j]] = recv[send_row[t,j]], so each
//    expert gets its own expert-major input rows again;
//  - moe_combine_partial (receiver, return direction): one row per (t, b), the sum of
//    the token's experts in bucket b, partial[r] = bf16(sum_j w*o over the j with
//    send_row[t,j] = r, j ascending, fp32 from +0, unfused);
//  - moe_combine_reduce (sender): y[t] = bf16(sum of the token's distinct partial
//    rows in ascending row order, i.e. ascending bucket, fp32 from +0, unfused).
// The accumulation order follows the one-owner, source-order rule of "Purlin:
// Separating Orchestration from the Datapath of Collectives", section 3.3 (SCORE).
//
// Mapping: as dispatch and combine, one workgroup per (token, 1 KiB row piece).
//  - expand: k/2 waves, each copying two entries' 16-byte vectors per lane
//    (non-temporal loads and stores).
//  - combine_partial: k/2 waves stage the source pieces in LDS with branch-free loads;
//    wave w then sums the token's distinct rows d = w, w + NW, ... (numbered by first
//    occurrence).
//  - combine_reduce: one wave loads the token's distinct partial rows, stages them in
//    LDS in ascending row order and adds them.
//  The distinct-row bookkeeping (first occurrence, rank among the token's rows) is
//  wave-uniform and runs on the scalar unit.
#include "moe_internal.h"

#pragma clang fp contract(off)

namespace moedl {
namespace {

constexpr int kPieceVecs = 64;

__device__ __forceinline__ void accumulate(float (&acc)[8], const u32x4 v, const float wj) {
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

__device__ __forceinline__ u32x4 to_bf16x8(const float (&acc)[8]) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  return o;
}

// ------------------------------------------------------------------ expand
// NW = k/2 waves, wave w copies entries j = w, w + NW (two 16-byte loads in flight,
// then two stores).  Measured on MI355X (Zipf M=16384 dedup): ~5.7 TB/s, against
// ~4.5 for k single-entry waves.  The loads are non-temporal: with plain loads the
// received rows stay in the caches, and the next dispatch into the same send buffer
// (the next layer or batch) ran 227 instead of 188 us; the dedup round trip as a whole
// (layout, dispatch, expand, pre-reduced combine, reduce) took 1533 instead of 1509 us.
// Scales travel only in the SCALES instantiation (a run-time test costs the rows-only
// dispatch 3%; the same split is kept here).
template <int K, int NW, bool SCALES>
__global__ __launch_bounds__(64 * NW) void expand_kernel(
    const u32x4* __restrict__ recv, int64_t recv_rows, int32_t row_vecs, int32_t pieces,
    const float* __restrict__ recv_scale, int32_t scale_cols,
    const int32_t* __restrict__ send_row, const int32_t* __restrict__ slot, int64_t M,
    u32x4* __restrict__ ein, float* __restrict__ ein_scale, int64_t expert_rows) {
  constexpr int H = (K + NW - 1) / NW;
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  __builtin_assume(w >= 0 && w < NW);
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;
  const int c = piece * kPieceVecs + lane;
  const int cc = c < row_vecs ? c : row_vecs - 1;
  u32x4 v[H];
  bool ok[H];
  int dst[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {  // loads first, unconditional (row 0 stands in)
    const int j = w + h * NW;
    const int r = j < K ? send_row[t * K + j] : -1;
    const int s = j < K ? slot[t * K + j] : -1;
    ok[h] = r >= 0 && r < recv_rows && s >= 0 && s < expert_rows;
    dst[h] = s;
    v[h] = __builtin_nontemporal_load(recv + (int64_t)(ok[h] ? r : 0) * row_vecs + cc);
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    if (!ok[h]) continue;
    if (c < row_vecs)
      __builtin_nontemporal_store(v[h], ein + (int64_t)dst[h] * row_vecs + c);
    if (SCALES && piece == 0) {
      const int r = send_row[t * K + w + h * NW];
      for (int sc = lane; sc < scale_cols; sc += 64)
        ein_scale[(int64_t)dst[h] * scale_cols + sc] = recv_scale[(int64_t)r * scale_cols + sc];
    }
  }
}

// ------------------------------------------------------------------ combine_partial
template <int K, int NW>
__global__ __launch_bounds__(64 * NW) void combine_partial_kernel(
    const u32x4* __restrict__ eo, int64_t expert_rows, const float* __restrict__ wts,
    const int32_t* __restrict__ slot, const int32_t* __restrict__ send_row, int64_t M,
    int32_t row_vecs, int32_t pieces, u32x4* __restrict__ partial, int64_t partial_rows) {
  __shared__ u32x4 stage[K][64];
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;  // uniform over the workgroup
  const int c = piece * kPieceVecs + lane;
  const int cc = c < row_vecs ? c : row_vecs - 1;
  // The token's slot, send-row and weight rows, read first (wave-uniform scalar loads,
  // all in flight together while the data loads travel; read after the barrier they
  // would cost a dependent round trip each).  The empty asm keeps the compiler from
  // sinking the loads of values only used after the barrier.
  int srow[K], rrow[K];
  float wrow[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    srow[j] = slot[t * K + j];
    rrow[j] = send_row[t * K + j];
    wrow[j] = wts[t * K + j];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) asm volatile("" : "+s"(rrow[j]), "+s"(wrow[j]));
  asm volatile("" : "+s"(partial), "+s"(partial_rows));

  // stage the k source pieces.  Loads are unconditional, so all of a lane's loads are
  // in flight together: an invalid slot reads row 0 (in bounds whenever any row
  // exists) and the value is replaced by zero.
  constexpr int H = (K + NW - 1) / NW;
  __builtin_assume(w >= 0 && w < NW);
  u32x4 d[H];
  bool ok[H];
  if (expert_rows > 0) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int j = w + h * NW;
      const int s = j < K ? srow[j] : -1;
      const bool valid = s >= 0 && s < expert_rows;
      ok[h] = valid && c < row_vecs;
      d[h] = __builtin_nontemporal_load(eo + (valid ? (int64_t)s * row_vecs : 0) + cc);
    }
  } else {
#pragma unroll
    for (int h = 0; h < H; ++h) ok[h] = false;
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int j = w + h * NW;
    if (j < K) stage[j][lane] = ok[h] ? d[h] : (u32x4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (c >= row_vecs) return;

  // distinct send rows of the token, numbered by first occurrence (scalar bookkeeping)
  int dcount = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = rrow[j];
    bool first = r >= 0 && r < partial_rows;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) first = first && rrow[jj] != r;
    if (!first) continue;
    const int di = dcount++;
    if (di % NW != w) continue;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < K; ++jj) {
      if (jj < j || rrow[jj] != r) continue;
      const int s = srow[jj];
      accumulate(acc, stage[jj][lane], (s >= 0 && s < expert_rows) ? wrow[jj] : 0.0f);
    }
    __builtin_nontemporal_store(to_bf16x8(acc), partial + (int64_t)r * row_vecs + c);
  }
}

// ------------------------------------------------------------------ combine_reduce
template <int K, int NW>
__global__ __launch_bounds__(64 * NW) void combine_reduce_kernel(
    const u32x4* __restrict__ partial, int64_t partial_rows, const int32_t* __restrict__ send_row,
    int64_t M, int32_t row_vecs, int32_t pieces, u32x4* __restrict__ y) {
  __shared__ u32x4 stage[K][64];
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;
  const int c = piece * kPieceVecs + lane;
  const int cc = c < row_vecs ? c : row_vecs - 1;
  const int32_t* rrow = send_row + t * K;

  // first occurrences of the token's distinct rows as a bitmask, and each distinct
  // row's rank among them in ascending order (wave-uniform, scalar unit; static
  // indices only, so nothing spills)
  int rv_[K];
#pragma unroll
  for (int j = 0; j < K; ++j) rv_[j] = rrow[j];
  uint32_t firstmask = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    bool f = rv_[j] >= 0 && rv_[j] < partial_rows;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) f = f && rv_[jj] != rv_[j];
    firstmask |= f ? (1u << j) : 0u;
  }
  const int nd = __builtin_popcount(firstmask);

  // unconditional loads (a skipped row reads the token's own output position, in
  // bounds, and is not staged)
  constexpr int H = (K + NW - 1) / NW;
  __builtin_assume(w >= 0 && w < NW);
  const u32x4* fallback = (const u32x4*)y + t * row_vecs + cc;
  u32x4 d[H];
  int slot_of[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int j = w + h * NW;
    const bool load = j < K && ((firstmask >> j) & 1u);
    const int r = load ? rrow[j] : 0;
    int rank = 0;
#pragma unroll
    for (int jj = 0; jj < K; ++jj) rank += (((firstmask >> jj) & 1u) && rv_[jj] < r) ? 1 : 0;
    slot_of[h] = load ? rank : -1;
    d[h] = __builtin_nontemporal_load(load ? partial + (int64_t)r * row_vecs + cc : fallback);
  }
#pragma unroll
  for (int h = 0; h < H; ++h)
    if (slot_of[h] >= 0) stage[slot_of[h]][lane] = d[h];
  if (NW > 1) __syncthreads();
  if (w != 0 || c >= row_vecs) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  for (int i = 0; i < nd; ++i) {
    const u32x4 v = stage[i][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t u = v[q];
      acc[2 * q] = acc[2 * q] + __builtin_bit_cast(float, u << 16);
      acc[2 * q + 1] = acc[2 * q + 1] + __builtin_bit_cast(float, u & 0xFFFF0000u);
    }
  }
  __builtin_nontemporal_store(to_bf16x8(acc), y + t * row_vecs + c);
}

template <int K>
hipError_t launch_partial_k(const uint16_t* eo, int64_t expert_rows, const float* w,
                            const int32_t* slot, const int32_t* send_row, int64_t M,
                            int32_t row_vecs, uint16_t* partial, int64_t partial_rows,
                            hipStream_t stream) {
  constexpr int NW = K >= 2 ? K / 2 : 1;
  const int32_t pieces = (row_vecs + kPieceVecs - 1) / kPieceVecs;
  const int64_t blocks = M * pieces;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_partial_kernel<K, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                     stream, (const u32x4*)eo, expert_rows, w, slot, send_row, M, row_vecs,
                     pieces, (u32x4*)partial, partial_rows);
  return hipGetLastError();
}

template <int K>
hipError_t launch_reduce_k(const uint16_t* partial, int64_t partial_rows, const int32_t* send_row,
                           int64_t M, int32_t row_vecs, uint16_t* y, hipStream_t stream) {
  constexpr int NW = 1;  // one wave per (token, piece): ~5.5 TB/s, against ~3.3 for k/2
  const int32_t pieces = (row_vecs + kPieceVecs - 1) / kPieceVecs;
  const int64_t blocks = M * pieces;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_reduce_kernel<K, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                     stream, (const u32x4*)partial, partial_rows, send_row, M, row_vecs, pieces,
                     (u32x4*)y);
  return hipGetLastError();
}

template <int K>
hipError_t launch_expand_k(const void* recv, int64_t recv_rows, int32_t row_vecs, int32_t pieces,
                           const float* recv_scale, int32_t scale_cols, const int32_t* send_row,
                           const int32_t* slot, int64_t M, void* expert_in, float* expert_scale,
                           int64_t expert_rows, hipStream_t stream) {
  constexpr int NW = K >= 2 ? K / 2 : 1;
  if (recv_scale != nullptr)
    hipLaunchKernelGGL((expand_kernel<K, NW, true>), dim3((unsigned)(M * pieces)), dim3(64 * NW),
                       0, stream, (const u32x4*)recv, recv_rows, row_vecs, pieces, recv_scale,
                       scale_cols, send_row, slot, M, (u32x4*)expert_in, expert_scale,
                       expert_rows);
  else
    hipLaunchKernelGGL((expand_kernel<K, NW, false>), dim3((unsigned)(M * pieces)), dim3(64 * NW),
                       0, stream, (const u32x4*)recv, recv_rows, row_vecs, pieces, recv_scale,
                       scale_cols, send_row, slot, M, (u32x4*)expert_in, expert_scale,
                       expert_rows);
  return hipGetLastError();
}

}  // namespace

#define MOEDL_K_SWITCH(CALL)                                                                \
  switch (k) {                                                                              \
    case 1: return CALL(1); case 2: return CALL(2); case 3: return CALL(3);                 \
    case 4: return CALL(4); case 5: return CALL(5); case 6: return CALL(6);                 \
    case 7: return CALL(7); case 8: return CALL(8); case 9: return CALL(9);                 \
    case 10: return CALL(10); case 11: return CALL(11); case 12: return CALL(12);           \
    case 13: return CALL(13); case 14: return CALL(14); case 15: return CALL(15);           \
    case 16: return CALL(16);                                                               \
    default: return hipErrorInvalidValue;                                                   \
  }

hipError_t launch_expand(const void* recv, int64_t recv_rows, int64_t row_bytes,
                         const float* recv_scale, int32_t scale_cols, const int32_t* send_row,
                         const int32_t* slot, int64_t M, int32_t k, void* expert_in,
                         float* expert_scale, int64_t expert_rows, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = (int32_t)(row_bytes / 16);
  const int32_t pieces = (row_vecs + kPieceVecs - 1) / kPieceVecs;
  if (M * pieces > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (recv_rows == 0) return hipSuccess;  // nothing to copy from
#define MOEDL_CALL(K)                                                                      \
  launch_expand_k<K>(recv, recv_rows, row_vecs, pieces, recv_scale, scale_cols, send_row, \
                     slot, M, expert_in, expert_scale, expert_rows, stream)
  MOEDL_K_SWITCH(MOEDL_CALL)
#undef MOEDL_CALL
}


hipError_t launch_combine_partial(const uint16_t* expert_out, int64_t expert_rows,
                                  const float* weights, const int32_t* slot,
                                  const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                                  uint16_t* partial, int64_t partial_rows, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = N / 8;
#define MOEDL_CALL(K) \
  launch_partial_k<K>(expert_out, expert_rows, weights, slot, send_row, M, row_vecs, partial, \
                      partial_rows, stream)
  MOEDL_K_SWITCH(MOEDL_CALL)
#undef MOEDL_CALL
}

hipError_t launch_combine_reduce(const uint16_t* partial, int64_t partial_rows,
                                 const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                                 uint16_t* y, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = N / 8;
#define MOEDL_CALL(K) launch_reduce_k<K>(partial, partial_rows, send_row, M, row_vecs, y, stream)
  MOEDL_K_SWITCH(MOEDL_CALL)
#undef MOEDL_CALL
}

#undef MOEDL_K_SWITCH

}  // namespace moedl
