// C ABI of libmoedl: argument validation, workspace carving and kernel launches on
// the caller's stream.  Every check here runs on the host before any HIP call, so a
// rejected call touches neither the device nor the stream.
#include <stdint.h>

#include "moe_internal.h"

namespace {

constexpr int32_t kAbiVersion = 3;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

moe_status check_layout_sizes(int64_t M, int32_t k, int32_t G, int32_t B) {
  if (M < 0 || k < 1 || G < 1 || B < 1 || k > G) return MOE_ERR_INVALID_ARGUMENT;
  if (G > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || B > MOE_MAX_BUCKETS) return MOE_ERR_UNSUPPORTED;
  if (M * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or format";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

size_t moe_dispatch_layout_workspace_bytes(int64_t M, int32_t k, int32_t G, int32_t B) {
  if (check_layout_sizes(M, k, G, B) != MOE_OK) return 0;
  return moedl::layout_workspace_bytes(M, G, B);
}

moe_status moe_dispatch_layout(const int32_t* topk_idx, int64_t M, int32_t k,
                               const int32_t* expert_bucket, int32_t G, int32_t B,
                               int32_t dedup, int32_t* expert_count, int32_t* expert_offset,
                               int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                               int32_t* send_row, int32_t* send_token, int32_t* status,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const moe_status s = check_layout_sizes(M, k, G, B);
  if (s != MOE_OK) return s;
  if (!expert_bucket || !expert_count || !expert_offset || !bucket_count || !bucket_offset ||
      !status || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && (!topk_idx || !slot || !send_row || !send_token)) return MOE_ERR_INVALID_ARGUMENT;
  if (dedup != 0 && dedup != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moedl::layout_workspace_bytes(M, G, B)) return MOE_ERR_WORKSPACE;
  const moedl::LayoutWorkspace ws = moedl::carve_layout_workspace(workspace, M, G, B);
  return from_hip(moedl::launch_layout(topk_idx, M, k, expert_bucket, G, B, dedup, expert_count,
                                       expert_offset, bucket_count, bucket_offset, slot,
                                       send_row, send_token, status, ws, stream));
}

moe_status moe_dispatch(const void* x, moe_dtype dtype, int64_t M, int32_t N,
                        const float* x_scale, const int32_t* send_row, int32_t k, int32_t dedup,
                        void* out, float* out_scale, int64_t out_rows, hipStream_t stream) {
  if (M < 0 || N < 1 || k < 1 || out_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dedup != 0 && dedup != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  if (k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((x_scale == nullptr) != (out_scale == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (x_scale && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t row_bytes = (int64_t)N * (dtype == MOE_BF16 ? 2 : 1);
  if (row_bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (x_scale && N % MOE_SCALE_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && (!x || !send_row)) return MOE_ERR_INVALID_ARGUMENT;
  if (out_rows > 0 && !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((x && !aligned16(x)) || (out && !aligned16(out))) return MOE_ERR_INVALID_ARGUMENT;
  if (x_scale && (((uintptr_t)x_scale & 3u) || ((uintptr_t)out_scale & 3u)))
    return MOE_ERR_INVALID_ARGUMENT;
  const int32_t scale_cols = x_scale ? N / MOE_SCALE_BLOCK : 0;
  return from_hip(moedl::launch_dispatch(x, M, row_bytes, x_scale, scale_cols, send_row, k,
                                         dedup, out, out_scale, out_rows, stream));
}

moe_status moe_layout_dispatch(const int32_t* topk_idx, int64_t M, int32_t k,
                               const int32_t* expert_bucket, int32_t G, int32_t B, int32_t dedup,
                               const void* x, moe_dtype dtype, int32_t N, const float* x_scale,
                               int32_t* expert_count, int32_t* expert_offset,
                               int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                               int32_t* send_row, int32_t* send_token, int32_t* status,
                               void* out, float* out_scale, int64_t out_rows,
                               hipStream_t stream) {
  const moe_status s = check_layout_sizes(M, k, G, B);
  if (s != MOE_OK) return s;
  if (N < 1 || out_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dedup != 0 && dedup != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  if (M > MOE_FUSED_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (!expert_bucket || !expert_count || !expert_offset || !bucket_count || !bucket_offset ||
      !status)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && (!topk_idx || !slot || !send_row || !send_token || !x))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((x_scale == nullptr) != (out_scale == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (x_scale && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t row_bytes = (int64_t)N * (dtype == MOE_BF16 ? 2 : 1);
  if (row_bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (x_scale && N % MOE_SCALE_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
  if (out_rows > 0 && !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((x && !aligned16(x)) || (out && !aligned16(out))) return MOE_ERR_INVALID_ARGUMENT;
  if (x_scale && (((uintptr_t)x_scale & 3u) || ((uintptr_t)out_scale & 3u)))
    return MOE_ERR_INVALID_ARGUMENT;
  const int32_t scale_cols = x_scale ? N / MOE_SCALE_BLOCK : 0;
  return from_hip(moedl::launch_layout_dispatch(
      topk_idx, M, k, expert_bucket, G, B, dedup, expert_count, expert_offset, bucket_count,
      bucket_offset, slot, send_row, send_token, status, x, row_bytes, x_scale, scale_cols, out,
      out_scale, out_rows, stream));
}

moe_status moe_combine(const uint16_t* expert_out, int64_t expert_rows, const float* weights,
                       const int32_t* slot, int64_t M, int32_t k, int32_t N, uint16_t* y,
                       hipStream_t stream) {
  if (M < 0 || N < 1 || k < 1 || expert_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (k > MOE_MAX_TOPK || N % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && (!weights || !slot || !y)) return MOE_ERR_INVALID_ARGUMENT;
  if (expert_rows > 0 && !expert_out) return MOE_ERR_INVALID_ARGUMENT;
  if ((expert_out && !aligned16(expert_out)) || (y && !aligned16(y)))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(
      moedl::launch_combine(expert_out, expert_rows, weights, slot, M, k, N, y, stream));
}

moe_status moe_expand(const void* recv, moe_dtype dtype, int64_t recv_rows, int32_t N,
                      const float* recv_scale, const int32_t* send_row, const int32_t* slot,
                      int64_t M, int32_t k, void* expert_in, float* expert_scale,
                      int64_t expert_rows, hipStream_t stream) {
  if (M < 0 || N < 1 || k < 1 || recv_rows < 0 || expert_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  if (k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((recv_scale == nullptr) != (expert_scale == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (recv_scale && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t row_bytes = (int64_t)N * (dtype == MOE_BF16 ? 2 : 1);
  if (row_bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (recv_scale && N % MOE_SCALE_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && (!send_row || !slot)) return MOE_ERR_INVALID_ARGUMENT;
  if ((recv_rows > 0 && !recv) || (expert_rows > 0 && !expert_in)) return MOE_ERR_INVALID_ARGUMENT;
  if ((recv && !aligned16(recv)) || (expert_in && !aligned16(expert_in)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (recv_scale && (((uintptr_t)recv_scale & 3u) || ((uintptr_t)expert_scale & 3u)))
    return MOE_ERR_INVALID_ARGUMENT;
  const int32_t scale_cols = recv_scale ? N / MOE_SCALE_BLOCK : 0;
  return from_hip(moedl::launch_expand(recv, recv_rows, row_bytes, recv_scale, scale_cols,
                                       send_row, slot, M, k, expert_in, expert_scale,
                                       expert_rows, stream));
}

moe_status moe_combine_partial(const uint16_t* expert_out, int64_t expert_rows,
                               const float* weights, const int32_t* slot,
                               const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                               uint16_t* partial, int64_t partial_rows, hipStream_t stream) {
  if (M < 0 || N < 1 || k < 1 || expert_rows < 0 || partial_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (k > MOE_MAX_TOPK || N % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && (!weights || !slot || !send_row)) return MOE_ERR_INVALID_ARGUMENT;
  if ((expert_rows > 0 && !expert_out) || (partial_rows > 0 && !partial))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((expert_out && !aligned16(expert_out)) || (partial && !aligned16(partial)))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(moedl::launch_combine_partial(expert_out, expert_rows, weights, slot, send_row,
                                                M, k, N, partial, partial_rows, stream));
}

moe_status moe_combine_reduce(const uint16_t* partial, int64_t partial_rows,
                              const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                              uint16_t* y, hipStream_t stream) {
  if (M < 0 || N < 1 || k < 1 || partial_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (k > MOE_MAX_TOPK || N % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && (!send_row || !y)) return MOE_ERR_INVALID_ARGUMENT;
  if (partial_rows > 0 && !partial) return MOE_ERR_INVALID_ARGUMENT;
  if ((partial && !aligned16(partial)) || (y && !aligned16(y))) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(
      moedl::launch_combine_reduce(partial, partial_rows, send_row, M, k, N, y, stream));
}

moe_status moe_expert_pair_counts(const int32_t* topk_idx, int64_t M, int32_t k, int32_t G,
                                  int32_t* pair_counts, hipStream_t stream) {
  if (M < 0 || k < 1 || G < 1 || !pair_counts) return MOE_ERR_INVALID_ARGUMENT;
  if (G > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (M * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (M > 0 && !topk_idx) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(moedl::launch_pair_counts(topk_idx, M, k, G, pair_counts, stream));
}

moe_status moe_place_experts(const int32_t* pair_counts, int32_t G, int32_t B,
                             int32_t* expert_bucket) {
  if (!pair_counts || !expert_bucket || G < 1 || B < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (G > MOE_MAX_EXPERTS || B > MOE_MAX_BUCKETS) return MOE_ERR_UNSUPPORTED;
  if (G % B != 0) return MOE_ERR_INVALID_ARGUMENT;
  moedl::place_experts_greedy(pair_counts, G, B, expert_bucket);
  return MOE_OK;
}

int32_t moe_grouped_gemm_max_tiles(int64_t rows, int32_t G, int32_t tile_m) {
  if (rows < 0 || G < 1 || tile_m < 1) return 0;
  const int64_t t = (rows + tile_m - 1) / tile_m + G;
  return t > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)t;
}

moe_status moe_grouped_gemm_tiles(const int32_t* expert_offset, const int32_t* expert_count,
                                  int32_t G, int32_t tile_m, int32_t* tile_expert,
                                  int32_t* tile_row0, int32_t* tile_rows, int32_t max_tiles,
                                  int32_t* num_tiles, hipStream_t stream) {
  if (!expert_offset || !expert_count || !num_tiles || G < 1 || tile_m < 1 || max_tiles < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (max_tiles > 0 && (!tile_expert || !tile_row0 || !tile_rows)) return MOE_ERR_INVALID_ARGUMENT;
  if (G > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  return from_hip(moedl::launch_gemm_tiles(expert_offset, expert_count, G, tile_m, tile_expert,
                                           tile_row0, tile_rows, max_tiles, num_tiles, stream));
}

moe_status moe_grouped_gemm(const uint16_t* x, int64_t rows, int32_t K, const uint16_t* w,
                            int32_t G, int32_t Nout, const int32_t* tile_expert,
                            const int32_t* tile_row0, const int32_t* tile_rows,
                            int32_t max_tiles, uint16_t* y, hipStream_t stream) {
  if (rows < 0 || K < 1 || G < 1 || Nout < 1 || max_tiles < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 64 != 0 || Nout % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)MOE_GEMM_TILE_M * K * 2 > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;  // 32-bit offsets
  if ((int64_t)max_tiles * (Nout / 128) > (int64_t)1 << 23) return MOE_ERR_UNSUPPORTED;  // grid
  if (!w || (max_tiles > 0 && (!tile_expert || !tile_row0 || !tile_rows))) return MOE_ERR_INVALID_ARGUMENT;
  if (rows > 0 && (!x || !y)) return MOE_ERR_INVALID_ARGUMENT;
  if ((x && !aligned16(x)) || !aligned16(w)) return MOE_ERR_INVALID_ARGUMENT;
  if (rows == 0) return MOE_OK;
  return from_hip(moedl::launch_grouped_gemm(x, rows, w, G, K, Nout, tile_expert, tile_row0,
                                             tile_rows, max_tiles, y, stream));
}

}  // extern "C"
