// Dispatch row scatter on gfx950.
//
// The gather of token rows into the destination-grouped send buffer that precedes
// the exchange ("All2all performance comparison between Triton-distributed and
// DeepEP": the note under "Results" and the send buffer / scale buffer arguments of
// "Test Code Snippet").  Push form: each token's row is read from HBM once and
// written once to every distinct send row of that token.
//
// Mapping.  A row is cut into 1 KiB pieces (64 lanes x 16 bytes).  One workgroup
// owns one (token, piece) and has k wave64s; wave j copies the piece to the send row
// of the token's j-th choice, unless an earlier choice already names that row
// (dedup mode) or the row is outside the buffer.  So every wave issues exactly one
// 16-byte load and one 16-byte non-temporal store per lane and retires.
//
// Why this shape: the destinations of a token are k rows scattered over the send
// buffer.  Measured on MI355X at 16384 tokens x 14 KiB x 8 destinations, a wave that
// holds a whole row and stores it k times sustains ~4.8 TB/s; one wave per
// (token, piece) storing k times ~5.5 TB/s; one store per wave ~6.8 TB/s.  Many
// short waves, each with a single store in flight, keep HBM write efficiency high
// under the scattered row pattern.  The k waves of a workgroup read the same x
// piece; the loads are cached (plain, not non-temporal) so the repeats hit L2 and
// HBM sees x once (rocprofv3 FETCH_SIZE confirms); the stores are non-temporal,
// since nothing rereads the send buffer soon.
//
// Scales (fp8 rows): the workgroup of piece 0 copies each destination's
// N/128-float scale row beside the data.  Whether scales travel is a template
// argument, not a run-time test: with the scale code compiled out, the rows-only
// kernel runs the Zipf workload above in 313 instead of 323 us (6.74 TB/s, the
// plain-copy ceiling) and correlated pairs (4 KiB rows) in 94 instead of 97 us.
//
// With a dedup layout (the caller says so), or rows x larger than the Infinity Cache
// (k > 1), a second shape is used, below.  Both shapes write the same bytes.
#include "moe_internal.h"

namespace moedl {
namespace {

constexpr int kPieceVecs = 64;  // 16-byte vectors per row piece (one per lane)

template <bool SCALES>
__global__ __launch_bounds__(64 * MOE_MAX_TOPK) void dispatch_piece_kernel(
    const u32x4* __restrict__ x, int64_t M, int32_t row_vecs, int32_t pieces,
    const float* __restrict__ x_scale, int32_t scale_cols,
    const int32_t* __restrict__ send_row, int32_t k, u32x4* __restrict__ out,
    float* __restrict__ out_scale, int64_t out_rows) {
  const int lane = threadIdx.x & 63;
  const int j = wave_index();
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;
  const int32_t* rows = send_row + t * k;
  const int r = rows[j];
  bool skip = r < 0 || r >= out_rows;
  for (int jj = 0; jj < j; ++jj) skip |= rows[jj] == r;
  if (skip) return;

  const int c = piece * kPieceVecs + lane;
  // the first 64 scales of the row are loaded together with the data, so the wave
  // waits for one round trip, not two
  const bool scales = SCALES && piece == 0;
  float s0 = 0.0f;
  if (scales && lane < scale_cols) s0 = x_scale[t * scale_cols + lane];
  if (c < row_vecs) {
    const u32x4 v = x[t * row_vecs + c];
    __builtin_nontemporal_store(v, out + (int64_t)r * row_vecs + c);
  }
  if (scales) {
    if (lane < scale_cols) __builtin_nontemporal_store(s0, out_scale + (int64_t)r * scale_cols + lane);
    for (int sc = lane + 64; sc < scale_cols; sc += 64)
      __builtin_nontemporal_store(x_scale[t * scale_cols + sc], out_scale + (int64_t)r * scale_cols + sc);
  }
}

// Dedup layouts: a token has fewer distinct send rows than k (4.6 of 8 on average at
// 8 buckets of 32 experts), so k single-store waves would leave ~40% of them idle.
// Here NW waves share the token's distinct rows (wave w stores the distinct rows
// d = w, w + NW, ..., numbered by first occurrence).  Measured on MI355X (Zipf
// M=16384, 76k send rows): NW = 2 sustains ~7 TB/s where the k-wave shape gets ~4.8.
template <int K, int NW, bool SCALES>
__global__ __launch_bounds__(64 * NW) void dispatch_dedup_kernel(
    const u32x4* __restrict__ x, int64_t M, int32_t row_vecs, int32_t pieces,
    const float* __restrict__ x_scale, int32_t scale_cols,
    const int32_t* __restrict__ send_row, u32x4* __restrict__ out,
    float* __restrict__ out_scale, int64_t out_rows) {
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int64_t t = blockIdx.x / pieces;
  const int piece = (int)(blockIdx.x - t * pieces);
  if (t >= M) return;
  const int32_t* rows = send_row + t * K;
  const int c = piece * kPieceVecs + lane;
  const bool in_row = c < row_vecs;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (in_row) v = x[t * row_vecs + c];
  int d = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = rows[j];
    bool first = r >= 0 && r < out_rows;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) first = first && rows[jj] != r;
    if (!first) continue;
    if (d % NW == w) {
      if (in_row) __builtin_nontemporal_store(v, out + (int64_t)r * row_vecs + c);
      if (SCALES && piece == 0) {
        for (int sc = lane; sc < scale_cols; sc += 64)
          out_scale[(int64_t)r * scale_cols + sc] = x_scale[t * scale_cols + sc];
      }
    }
    ++d;
  }
}

template <int K>
hipError_t launch_dedup_k(const void* x, int64_t M, int32_t row_vecs, int32_t pieces,
                          const float* x_scale, int32_t scale_cols, const int32_t* send_row,
                          void* out, float* out_scale, int64_t out_rows, hipStream_t stream) {
  constexpr int NW = K >= 2 ? 2 : 1;
  if (x_scale != nullptr)
    hipLaunchKernelGGL((dispatch_dedup_kernel<K, NW, true>), dim3((unsigned)(M * pieces)),
                       dim3(64 * NW), 0, stream, (const u32x4*)x, M, row_vecs, pieces, x_scale,
                       scale_cols, send_row, (u32x4*)out, out_scale, out_rows);
  else
    hipLaunchKernelGGL((dispatch_dedup_kernel<K, NW, false>), dim3((unsigned)(M * pieces)),
                       dim3(64 * NW), 0, stream, (const u32x4*)x, M, row_vecs, pieces, x_scale,
                       scale_cols, send_row, (u32x4*)out, out_scale, out_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const void* x, int64_t M, int64_t row_bytes, const float* x_scale,
                           int32_t scale_cols, const int32_t* send_row, int32_t k, int32_t dedup,
                           void* out, float* out_scale, int64_t out_rows, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = (int32_t)(row_bytes / 16);
  const int32_t pieces = (row_vecs + kPieceVecs - 1) / kPieceVecs;
  const int64_t blocks = M * pieces;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  // The k single-store waves shape is the faster one while x fits the 256 MB Infinity
  // Cache: 6.1-6.7 TB/s against 5.8 for two waves at x = 235 MB.  Once x outgrows it,
  // the dispatch's own plain x loads leave lines in the caches, and with such lines
  // present (left by any earlier kernel's plain loads or stores too) the k-wave shape
  // falls to ~3.5-3.8 TB/s, while the shape of two waves sharing a token's rows (about
  // four stores per load) holds 4.8-5.5: at a fixed 1.88 GB send buffer, x = 470 MB
  // (k = 4) runs at 4.1 vs 5.3 TB/s, x = 940 MB (k = 2) at 5.0 vs 5.6; at k = 1 the
  // shapes are within 4% (5.65 vs 5.44).  The send-buffer size itself does not matter
  // (1.88 GB written inside a 4 GiB allocation, or a 2.35 GB buffer with x below the
  // cache, behave like their x).  Nor does the latency the storing waves see: with x
  // prefetched into L2 ahead of them (their loads return in ~275 instead of ~1,600
  // cycles) the k-wave shape is no faster.  Measured on MI355X with rocprofv3
  // read-latency counters; the threshold sits between x = 235 MB (k-wave faster) and
  // 264 MB (two-wave faster).  A caller whose earlier kernels leave plainly accessed
  // lines behind can ask for the two-wave shape with the dedup flag, which selects the
  // shape only.
  constexpr int64_t kCacheResidentXBytes = (int64_t)240 << 20;
  if (dedup || (k >= 2 && M * row_bytes > kCacheResidentXBytes)) {
#define MOEDL_CASE(K)                                                                          \
  case K:                                                                                      \
    return launch_dedup_k<K>(x, M, row_vecs, pieces, x_scale, scale_cols, send_row, out,     \
                             out_scale, out_rows, stream);
    switch (k) {
      MOEDL_CASE(1) MOEDL_CASE(2) MOEDL_CASE(3) MOEDL_CASE(4) MOEDL_CASE(5) MOEDL_CASE(6)
      MOEDL_CASE(7) MOEDL_CASE(8) MOEDL_CASE(9) MOEDL_CASE(10) MOEDL_CASE(11) MOEDL_CASE(12)
      MOEDL_CASE(13) MOEDL_CASE(14) MOEDL_CASE(15) MOEDL_CASE(16)
      default:
        return hipErrorInvalidValue;
    }
#undef MOEDL_CASE
  }
  if (x_scale != nullptr)
    hipLaunchKernelGGL(dispatch_piece_kernel<true>, dim3((unsigned)blocks), dim3(64 * k), 0,
                       stream, (const u32x4*)x, M, row_vecs, pieces, x_scale, scale_cols,
                       send_row, k, (u32x4*)out, out_scale, out_rows);
  else
    hipLaunchKernelGGL(dispatch_piece_kernel<false>, dim3((unsigned)blocks), dim3(64 * k), 0,
                       stream, (const u32x4*)x, M, row_vecs, pieces, x_scale, scale_cols,
                       send_row, k, (u32x4*)out, out_scale, out_rows);
  return hipGetLastError();
}

}  // namespace moedl
