/*
 * moe_harness.h -- C ABI of libmoedl_harness: test and measurement helpers that sit
 * BESIDE the dispatch/combine path, not on it.
 *
 *  - moe_harness_expert_outputs: fixed elementwise "experts" that turn dispatched
 *    rows into the slot-indexed expert outputs combine reads, so that the combine
 *    result is known in closed form.  No trained experts exist here.
 *  - moe_harness_copy: a plain 16-byte streaming copy of known size, the reference
 *    that HBM traffic counters and the achievable-bandwidth ceiling are calibrated
 *    against.
 *
 * All pointers are device pointers; calls are asynchronous on `stream`; the return
 * value is 0 on success, 1 for an invalid argument and 4 for a launch failure.
 */
#ifndef MOE_HARNESS_H_
#define MOE_HARNESS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Expert stand-ins. */
#define MOE_STANDIN_IDENTITY 0 /* o = row (bf16 rows only)                          */
#define MOE_STANDIN_SCALE 1    /* o = bf16_rne(f32(row) * (1 + e/256)) (bf16 rows)    */
#define MOE_STANDIN_DEQUANT 2  /* o = bf16_rne(f32(q) * scale of q's 128-block) (fp8) */

/*
 * For every entry f = t*k + j with 0 <= send_row[f] < sent_rows and
 * 0 <= slot[f] < expert_rows: expert_out[slot[f]] = standin(sent[send_row[f]],
 * e = topk_idx[f]).  sent is bf16 [sent_rows, N] (kinds 0, 1) or fp8 e4m3
 * [sent_rows, N] with float sent_scale [sent_rows, N/128] (kind 2); expert_out is
 * bf16 [expert_rows, N].  This is the receiver-side expansion of dedup rows into
 * per-expert rows, fused with the stand-in expert.
 */
int moe_harness_expert_outputs(int32_t kind, const void* sent, const float* sent_scale,
                               int64_t sent_rows, int32_t N, const int32_t* send_row,
                               const int32_t* slot, const int32_t* topk_idx, int64_t M,
                               int32_t k, uint16_t* expert_out, int64_t expert_rows,
                               hipStream_t stream);

/* dst[0, bytes) = src[0, bytes); bytes % 16 == 0, both 16-byte aligned. */
int moe_harness_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HARNESS_H_ */
