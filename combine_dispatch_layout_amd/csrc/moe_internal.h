// Internal declarations shared by the libmoedl translation units: kernel
// launchers (one per .hip file) and the small wave-level helpers every kernel uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moedl {

// ---------------------------------------------------------------- layout tiling
// One layout tile = 256 tokens = one 256-thread workgroup (4 wave64s, 64 tokens
// each).  Per-tile partial counts live in the caller's workspace.
constexpr int kTileTokens = 256;
constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / 64;
constexpr int kScanThreads = 1024;
constexpr int kNoError = 0x7FFFFFFF;

// Up to kOnePassMaxTiles tiles the layout is one launch: every tile publishes its
// counts, waits (bounded) until all tiles have, and reduces the columns itself.
constexpr int kOnePassMaxTiles = 64;

struct LayoutWorkspace {
  // one-launch layout (2..kOnePassMaxTiles tiles): a header of four words
  //   [0] tiles that have left the current call   [1] region the next call publishes in
  //   [2] tiles and [3] row pitch of the call that published last (its rows are
  //       cleared by the next one-launch call)
  // and two publication regions at fixed offsets, used by alternate calls.  Each
  // region holds kOnePassMaxTiles rows of up to MOE_MAX_EXPERTS + MOE_MAX_BUCKETS
  // counts, then one error word per tile, all stored as value + 1 so that zero means
  // "not yet published".  Zero everywhere between calls, except the region of the
  // last call.
  uint32_t* header;
  int32_t* region[2];
  // three-launch layout (more tiles)
  int32_t* tile_hist;   // [T][G]: per-tile expert counts, then their column prefix
  int32_t* tile_bhist;  // [T][B]: per-tile distinct (token, bucket) counts, then prefix
  int32_t* tile_err;    // [T]:    first bad flat index in the tile, or kNoError
};

constexpr int kRegionCols = MOE_MAX_EXPERTS + MOE_MAX_BUCKETS;  // widest row, in ints
constexpr int kRegionErrOffset = kOnePassMaxTiles * kRegionCols;  // error words, in ints
constexpr size_t kRegionBytes = ((size_t)(kRegionErrOffset + kOnePassMaxTiles) * 4 + 255) & ~(size_t)255;

inline int64_t layout_tiles(int64_t M) { return (M + kTileTokens - 1) / kTileTokens; }

size_t layout_workspace_bytes(int64_t M, int32_t G, int32_t B);
LayoutWorkspace carve_layout_workspace(void* base, int64_t M, int32_t G, int32_t B);

hipError_t launch_layout(const int32_t* topk_idx, int64_t M, int32_t k,
                         const int32_t* expert_bucket, int32_t G, int32_t B, int32_t dedup,
                         int32_t* expert_count, int32_t* expert_offset,
                         int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                         int32_t* send_row, int32_t* send_token, int32_t* status,
                         const LayoutWorkspace& ws, hipStream_t stream);

constexpr int kFusedMaxTokens = MOE_FUSED_MAX_TOKENS;  // layout + dispatch in one launch
hipError_t launch_layout_dispatch(const int32_t* topk_idx, int64_t M, int32_t k,
                                  const int32_t* expert_bucket, int32_t G, int32_t B,
                                  int32_t dedup, int32_t* expert_count, int32_t* expert_offset,
                                  int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                                  int32_t* send_row, int32_t* send_token, int32_t* status,
                                  const void* x, int64_t row_bytes, const float* x_scale,
                                  int32_t scale_cols, void* out, float* out_scale,
                                  int64_t out_rows, hipStream_t stream);

hipError_t launch_dispatch(const void* x, int64_t M, int64_t row_bytes,
                           const float* x_scale, int32_t scale_cols,
                           const int32_t* send_row, int32_t k, int32_t dedup, void* out,
                           float* out_scale, int64_t out_rows, hipStream_t stream);

hipError_t launch_combine(const uint16_t* expert_out, int64_t expert_rows,
                          const float* weights, const int32_t* slot, int64_t M,
                          int32_t k, int32_t N, uint16_t* y, hipStream_t stream);

hipError_t launch_expand(const void* recv, int64_t recv_rows, int64_t row_bytes,
                         const float* recv_scale, int32_t scale_cols, const int32_t* send_row,
                         const int32_t* slot, int64_t M, int32_t k, void* expert_in,
                         float* expert_scale, int64_t expert_rows, hipStream_t stream);

hipError_t launch_combine_partial(const uint16_t* expert_out, int64_t expert_rows,
                                  const float* weights, const int32_t* slot,
                                  const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                                  uint16_t* partial, int64_t partial_rows, hipStream_t stream);

hipError_t launch_combine_reduce(const uint16_t* partial, int64_t partial_rows,
                                 const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                                 uint16_t* y, hipStream_t stream);

hipError_t launch_pair_counts(const int32_t* topk_idx, int64_t M, int32_t k, int32_t G,
                              int32_t* counts, hipStream_t stream);

void place_experts_greedy(const int32_t* pair_counts, int32_t G, int32_t B, int32_t* bucket);

hipError_t launch_gemm_tiles(const int32_t* expert_offset, const int32_t* expert_count, int32_t G,
                             int32_t tile_m, int32_t* tile_expert, int32_t* tile_row0,
                             int32_t* tile_rows, int32_t max_tiles, int32_t* num_tiles,
                             hipStream_t stream);
hipError_t launch_grouped_gemm(const uint16_t* x, int64_t rows, const uint16_t* w, int32_t G,
                               int32_t K, int32_t Nout, const int32_t* tile_expert,
                               const int32_t* tile_row0, const int32_t* tile_rows,
                               int32_t max_tiles, uint16_t* y, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}
// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values to a packed pair of bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
#endif

}  // namespace moedl
