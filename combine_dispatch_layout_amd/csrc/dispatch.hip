// Dispatch row scatter on gfx950.
//
// The gather of token rows into the destination-grouped send buffer that precedes
// the exchange ("All2all performance comparison between Triton-distributed and
// DeepEP": the note under "Results" and the send buffer / scale buffer arguments of
// "Test Code Snippet").  Push form: each token's row is read from HBM once and
// written to every distinct send row of that token, so the bytes moved are exactly
// one row read per token plus one row write per send row.
//
// Mapping: one wave64 per token, four tokens per 256-thread workgroup.  Each lane
// holds up to VPL 16-byte vectors of the row in registers (lane-interleaved, so one
// wave instruction moves 1 KiB of contiguous bytes), then stores them to each
// destination.  The send rows of a token are wave-uniform scalar loads, and the
// duplicate check (dedup mode: several experts of one token in one bucket share a
// row) runs on the scalar unit.  Loads and stores are non-temporal: every byte is
// touched once, so nothing is worth keeping in L2 or the Infinity Cache.
#include "moe_internal.h"

namespace moedl {
namespace {

constexpr int kTokensPerBlock = 4;

template <int VPL>
__global__ __launch_bounds__(256) void dispatch_rows_kernel(
    const u32x4* __restrict__ x, int64_t M, int32_t row_vecs,
    const float* __restrict__ x_scale, int32_t scale_cols,
    const int32_t* __restrict__ send_row, int32_t k, u32x4* __restrict__ out,
    float* __restrict__ out_scale, int64_t out_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + wave_index();
  if (t >= M) return;
  const int32_t* rows = send_row + t * k;

  for (int base = 0; base < row_vecs; base += 64 * VPL) {
    u32x4 v[VPL];
    const u32x4* src = x + t * row_vecs + base + lane;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (base + lane + 64 * i < row_vecs) v[i] = __builtin_nontemporal_load(src + 64 * i);
    }
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      bool skip = r < 0 || r >= out_rows;
      for (int jj = 0; jj < j; ++jj) skip |= rows[jj] == r;
      if (skip) continue;
      u32x4* dst = out + (int64_t)r * row_vecs + base + lane;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        if (base + lane + 64 * i < row_vecs) __builtin_nontemporal_store(v[i], dst + 64 * i);
      }
    }
  }

  if (x_scale != nullptr) {
    for (int c = lane; c < scale_cols; c += 64) {
      const float s = x_scale[t * scale_cols + c];
      for (int j = 0; j < k; ++j) {
        const int r = rows[j];
        bool skip = r < 0 || r >= out_rows;
        for (int jj = 0; jj < j; ++jj) skip |= rows[jj] == r;
        if (!skip) out_scale[(int64_t)r * scale_cols + c] = s;
      }
    }
  }
}

template <int VPL>
hipError_t launch_vpl(const void* x, int64_t M, int32_t row_vecs, const float* x_scale,
                      int32_t scale_cols, const int32_t* send_row, int32_t k, void* out,
                      float* out_scale, int64_t out_rows, hipStream_t stream) {
  const int64_t blocks = (M + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(dispatch_rows_kernel<VPL>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4*)x, M, row_vecs, x_scale, scale_cols, send_row, k,
                     (u32x4*)out, out_scale, out_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const void* x, int64_t M, int64_t row_bytes, const float* x_scale,
                           int32_t scale_cols, const int32_t* send_row, int32_t k, void* out,
                           float* out_scale, int64_t out_rows, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = (int32_t)(row_bytes / 16);
  const int vpl = (row_vecs + 63) / 64;
#define MOEDL_CASE(V)                                                                   \
  case V:                                                                               \
    return launch_vpl<V>(x, M, row_vecs, x_scale, scale_cols, send_row, k, out, out_scale, \
                         out_rows, stream);
  switch (vpl) {
    MOEDL_CASE(1) MOEDL_CASE(2) MOEDL_CASE(3) MOEDL_CASE(4) MOEDL_CASE(5) MOEDL_CASE(6)
    MOEDL_CASE(7) MOEDL_CASE(8) MOEDL_CASE(9) MOEDL_CASE(10) MOEDL_CASE(11) MOEDL_CASE(12)
    MOEDL_CASE(13) MOEDL_CASE(14) MOEDL_CASE(15)
    default:  // rows above 15 KiB: loop over the row in 16 KiB pieces
      return launch_vpl<16>(x, M, row_vecs, x_scale, scale_cols, send_row, k, out, out_scale,
                            out_rows, stream);
  }
#undef MOEDL_CASE
}

}  // namespace moedl
