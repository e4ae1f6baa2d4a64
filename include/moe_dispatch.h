/*
 * moe_dispatch.h -- C ABI of libmoedl: MoE token dispatch layout, dispatch and
 * combine on one AMD Instinct MI355X (gfx950).
 *
 * The three calls are one GPU's share of expert-parallel all-to-all dispatch and
 * combine, as the problem is stated in "All2all performance comparison between
 * Triton-distributed and DeepEP" (sections "Test Code Snippet" and "Benchmark
 * Configuration"): M tokens of hidden size N (HIDDEN), G experts in total
 * (NUM_TOT_EXPERTS), top-k routing, experts grouped into destinations
 * (EXPERTS_PER_RANK, WORLD_SIZE; here "buckets" with an arbitrary expert -> bucket
 * map), an element size of 2 (bf16) or 1 (fp8) bytes with optional per-block
 * scales (WITH_SCALE, SCALE_ELEMENT_SIZE), and per-destination splits with their
 * cumulative sums.
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer (hipMalloc'd or torch memory),
 *    except where a comment says otherwise.  The caller owns and allocates every
 *    buffer, including the layout workspace; the library allocates nothing, keeps
 *    no global state and has no handle.
 *  - Calls are asynchronous on `stream` (0 = the legacy default stream) and never
 *    synchronise the host.  Outputs are valid once the stream reaches them.
 *  - Host-checkable argument errors are returned synchronously, before any
 *    launch, as a moe_status; nothing is written in that case.
 *  - Data-dependent errors (an expert id or bucket id out of range) are reported
 *    in the device status word written by moe_dispatch_layout; the layout outputs
 *    are then unspecified but every kernel stays in bounds.
 *  - All row buffers are row-major with a row pitch equal to the row size; row
 *    bases must be 16-byte aligned and row sizes a multiple of 16 bytes.
 *  - Calls are reentrant across streams as long as their output buffers and
 *    workspaces differ.
 */
#ifndef MOE_DISPATCH_H_
#define MOE_DISPATCH_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, k > G, misaligned */
  MOE_ERR_UNSUPPORTED = 2,      /* beyond the limits below */
  MOE_ERR_WORKSPACE = 3,        /* workspace smaller than the query returns */
  MOE_ERR_LAUNCH = 4            /* the HIP runtime refused a kernel launch */
} moe_status;

typedef enum moe_dtype {
  MOE_BF16 = 0,     /* bfloat16, 2 bytes per element */
  MOE_FP8_E4M3 = 1  /* OCP fp8 e4m3 ("fn": no infinities, max 448), 1 byte */
} moe_dtype;

#define MOE_MAX_EXPERTS 1024 /* G */
#define MOE_MAX_TOPK 16      /* k */
#define MOE_MAX_BUCKETS 64   /* B */
#define MOE_SCALE_BLOCK 128  /* elements per fp32 scale */

/* Status word of moe_dispatch_layout when the one-launch layout (2 to 64 tiles of
 * 256 tokens, or of 1024 tokens up to M = 65536 at k <= 8) gave up waiting for its
 * workgroups to be resident together (about a second); the other outputs are then
 * unspecified but in bounds. */
#define MOE_LAYOUT_STATUS_WAIT_EXPIRED (-2147483647 - 1)

/* Version of this ABI (bumped on any signature change). */
int32_t moe_abi_version(void);

/* Static, NUL-terminated description of a status (host pointer). */
const char* moe_status_string(moe_status status);

/*
 * Bytes of device workspace moe_dispatch_layout needs for these sizes (a pure
 * host computation; 0 if the sizes are invalid).  The workspace holds a 256-byte
 * header and the two publication regions of the one-launch layout at fixed offsets,
 * then, for sizes that take the three-launch layout, per-tile partial counts.  It
 * must be zero-filled once, before its first use (e.g. hipMemset after allocation);
 * every call leaves it ready for the next one (the header and the region the next
 * call publishes in are cleared), so it may then be reused by any later call on the
 * same stream, for any sizes it is large enough for.
 */
size_t moe_dispatch_layout_workspace_bytes(int64_t M, int32_t k, int32_t G, int32_t B);

/*
 * moe_dispatch_layout -- counts, cumulative offsets, the stable slot map and the
 * send-row map of one routing batch.
 *
 * Passages: the send buffer grouped by destination, its splits and cumulative sums
 * ("All2all performance comparison ...", "Test Code Snippet"); per-expert row
 * offsets that stay on the device for a grouped GEMM ("Add Triton grouped-GEMM for
 * MoE experts on Ampere/Ada", "What this PR does"); one copy per (token,
 * destination) pair even when several of the token's experts share that destination
 * ("Zyphra says routing-pattern expert placement ...", the 58% copy-reduction item).
 *
 * Inputs:
 *   topk_idx      int32 [M*k], row-major [M][k]: expert id of token t's j-th choice,
 *                 in [0, G).  A token may repeat an expert; each repeat is its own
 *                 entry.
 *   expert_bucket int32 [G]: destination bucket of each expert, in [0, B).
 *   dedup         0: one send row per (t, j).  1: one send row per distinct
 *                 (t, bucket).
 * Outputs (all written by this call; M may be 0):
 *   expert_count  int32 [G]: entries routed to each expert (sum = M*k).
 *   expert_offset int32 [G]: first slot of each expert's run.  Runs are laid out
 *                 in (bucket, expert id) order, so expert_offset/expert_count are
 *                 the grouped-GEMM `offs` of the per-expert buffers.
 *   bucket_count  int32 [B]: send rows of each bucket (the splits).
 *   bucket_offset int32 [B+1]: exclusive cumulative sum of bucket_count;
 *                 bucket_offset[B] = R, the number of send rows.
 *   slot          int32 [M*k]: position of entry (t, j) in slot space: its expert's
 *                 offset plus the number of earlier entries (ascending t, then j)
 *                 routed to the same expert.  A bijection onto [0, M*k).
 *   send_row      int32 [M*k]: send-buffer row of entry (t, j).  dedup=0: equals
 *                 slot.  dedup=1: bucket_offset[b] + number of tokens t' < t that
 *                 also send to b, where b = expert_bucket[topk_idx[t,j]].
 *   send_token    int32 [capacity]: token of each send row, rows [0, R) written.
 *                 Capacity M*k (dedup=0) or M*min(k, B) (dedup=1).
 *   status        int32 [1]: 0 when all ids are valid; t*k + j + 1 for the first
 *                 entry whose expert id is outside [0, G); -(e + 1) for the first
 *                 expert e whose bucket is outside [0, B) (checked first);
 *                 MOE_LAYOUT_STATUS_WAIT_EXPIRED (see above; checked before both).
 *   workspace     device scratch of at least
 *                 moe_dispatch_layout_workspace_bytes(M, k, G, B) bytes, 16-byte
 *                 aligned, zero-filled before its first use; calls that overlap
 *                 in time must not share it.
 * Errors: MOE_ERR_INVALID_ARGUMENT (M < 0, k < 1, k > G, G < 1, B < 1, a null
 * pointer for a non-empty array), MOE_ERR_UNSUPPORTED (G > 1024, k > 16, B > 64,
 * M*k >= 2^31), MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 */
moe_status moe_dispatch_layout(const int32_t* topk_idx, int64_t M, int32_t k,
                               const int32_t* expert_bucket, int32_t G, int32_t B,
                               int32_t dedup, int32_t* expert_count,
                               int32_t* expert_offset, int32_t* bucket_count,
                               int32_t* bucket_offset, int32_t* slot, int32_t* send_row,
                               int32_t* send_token, int32_t* status, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_layout_noalloc -- moe_dispatch_layout with no workspace argument and
 * no allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it.
 *
 * Inputs, outputs, status word and errors are those of moe_dispatch_layout, and the
 * results are identical.  The workspace is a static device array of
 * MOE_LAYOUT_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends; sizes whose workspace query exceeds it are refused with
 * MOE_ERR_WORKSPACE (every G, k and B up to 65,536 tokens fit; at G = 256, B = 8,
 * about 850,000 tokens).  The call runs on the current device (`stream` must belong
 * to it).  Every call on one GPU shares that GPU's array: calls that overlap in time
 * race, calls ordered on a stream do not.  Nothing is allocated and no memset is
 * issued: the array starts zero-filled, the state a new workspace must be in, and
 * every call leaves it ready for the next one, as moe_dispatch_layout does with
 * its workspace (the header and the region the next call publishes in are
 * cleared by the kernels).
 */
#define MOE_LAYOUT_SCRATCH_BYTES (4u << 20)

moe_status moe_dispatch_layout_noalloc(const int32_t* topk_idx, int64_t M, int32_t k,
                                       const int32_t* expert_bucket, int32_t G, int32_t B,
                                       int32_t dedup, int32_t* expert_count,
                                       int32_t* expert_offset, int32_t* bucket_count,
                                       int32_t* bucket_offset, int32_t* slot,
                                       int32_t* send_row, int32_t* send_token,
                                       int32_t* status, hipStream_t stream);

/*
 * moe_dispatch -- copy each token's row (and its scales) into its send rows.
 *
 * Passage: the gather of token rows into the destination-grouped send buffer, with
 * scales travelling beside fp8 data ("All2all performance comparison ...", "Test
 * Code Snippet" and the note under "Results").  Each x row is read once and written
 * once to every distinct row among send_row[t, 0..k).
 *
 * Inputs:
 *   x         [M, N] elements of `dtype`, row-major; 16-byte aligned.
 *   x_scale   float [M, N/128] or NULL.  Only with MOE_FP8_E4M3, and then
 *             N % 128 == 0.
 *   send_row  int32 [M*k] from moe_dispatch_layout (any map into rows works).
 *   dedup     0 or 1: whether send_row came from a dedup layout.  Only selects the
 *             kernel shape (k single-store waves per row piece, or two waves sharing
 *             the token's distinct rows; the latter also when x is larger than the
 *             GPU's last-level cache and k > 1); the bytes written are the same.
 * Outputs:
 *   out       [out_rows, N] elements of `dtype`; rows named by send_row are written.
 *   out_scale float [out_rows, N/128]; NULL exactly when x_scale is NULL.
 *   out_rows  capacity of out in rows.  Entries of send_row outside [0, out_rows)
 *             are skipped, so an erroneous layout can never write out of bounds.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null or misaligned pointers, M < 0, N < 1,
 * k < 1, dedup not 0/1, scales with bf16, out_scale/x_scale mismatch), MOE_ERR_UNSUPPORTED (row
 * bytes not a multiple of 16, scales with N % 128 != 0, k > 16), MOE_ERR_LAUNCH.
 */
moe_status moe_dispatch(const void* x, moe_dtype dtype, int64_t M, int32_t N,
                        const float* x_scale, const int32_t* send_row, int32_t k,
                        int32_t dedup, void* out, float* out_scale, int64_t out_rows,
                        hipStream_t stream);

/*
 * moe_layout_dispatch -- moe_dispatch_layout followed by moe_dispatch, in one launch,
 * for small batches (M <= MOE_FUSED_MAX_TOKENS).
 *
 * The small-token regime of "All2all performance comparison between Triton-distributed
 * and DeepEP" ("Results (Latency in us)" and the note under it: at 128 tokens the
 * dispatch is a few tens of microseconds, so launch count and gaps, not bytes, decide
 * it).  Every output is the one the two calls would produce: the layout arrays and
 * status word of moe_dispatch_layout (same arguments, same meaning) and the send rows
 * of moe_dispatch (x, dtype, N, x_scale, out, out_scale, out_rows as there).  No
 * workspace is needed.  Within the launch every workgroup derives the layout in its
 * own on-chip memory, so no workgroup waits for another.  On MI355X it is the faster
 * form up to 256 tokens (one tile); from 257 to 512 tokens the two calls are faster,
 * since every workgroup then derives two tiles.
 * Errors: those of the two calls, and MOE_ERR_UNSUPPORTED for M > MOE_FUSED_MAX_TOKENS.
 */
#define MOE_FUSED_MAX_TOKENS 512
moe_status moe_layout_dispatch(const int32_t* topk_idx, int64_t M, int32_t k,
                               const int32_t* expert_bucket, int32_t G, int32_t B, int32_t dedup,
                               const void* x, moe_dtype dtype, int32_t N, const float* x_scale,
                               int32_t* expert_count, int32_t* expert_offset,
                               int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                               int32_t* send_row, int32_t* send_token, int32_t* status,
                               void* out, float* out_scale, int64_t out_rows,
                               hipStream_t stream);

/*
 * moe_combine -- routing-weighted top-k sum of expert outputs back in token order.
 *
 *   y[t, i] = bf16_rne( sum_{j=0..k-1} w[t, j] * expert_out[slot[t, j], i] )
 *
 * with an fp32 accumulator that starts at +0.0 and takes, for j ascending, one
 * rounded fp32 product and one rounded fp32 add (no fused multiply-add), then one
 * round-to-nearest-even to bf16.  This is the determinism rule of "Purlin:
 * Separating Orchestration from the Datapath of Collectives", section 3.3 (SCORE):
 * one owner per output element, accumulation in source order.  Results are
 * bitwise reproducible.
 *
 * Inputs:
 *   expert_out  bf16 [expert_rows, N], slot-indexed (expert-major); 16-byte
 *               aligned.
 *   weights     float [M*k], row-major [M][k]; never renormalised.
 *   slot        int32 [M*k] from moe_dispatch_layout.  Entries outside
 *               [0, expert_rows) contribute nothing.
 * Output:
 *   y           bf16 [M, N]; 16-byte aligned.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null or misaligned pointers, M < 0, N < 1,
 * k < 1), MOE_ERR_UNSUPPORTED (N % 8 != 0, k > 16), MOE_ERR_LAUNCH.
 */
moe_status moe_combine(const uint16_t* expert_out, int64_t expert_rows,
                       const float* weights, const int32_t* slot, int64_t M, int32_t k,
                       int32_t N, uint16_t* y, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------
 * The steps on either side of the path in dedup mode.  A (token, bucket) pair
 * travels as one row ("Zyphra says routing-pattern expert placement ...", the
 * copy-reduction item); the receiver turns it back into one row per expert, and on
 * the way back the token's experts inside a bucket are summed before the return, so
 * one row per (token, bucket) travels instead of one per (token, j).  The return path
 * is not described on the pages; this is its mirror image of the forward path.
 * ---------------------------------------------------------------------------------
 */

/*
 * moe_expand -- receiver-side expansion:  expert_in[slot[f]] = recv[send_row[f]] for
 * every entry f = t*k + j (raw bytes, scales follow the rows).
 *
 *   recv        [recv_rows, N] elements of `dtype` (a dedup send buffer, or what the
 *               exchange delivered), 16-byte aligned.
 *   recv_scale  float [recv_rows, N/128] or NULL (fp8 only).
 *   send_row, slot  int32 [M*k] from moe_dispatch_layout (dedup = 1).
 *   expert_in   [expert_rows, N] of `dtype`, slot-indexed; expert_scale float
 *               [expert_rows, N/128], NULL exactly when recv_scale is NULL.
 * Entries whose send row or slot is out of range are skipped.
 * Errors: as moe_dispatch (argument checks on the host).
 */
moe_status moe_expand(const void* recv, moe_dtype dtype, int64_t recv_rows, int32_t N,
                      const float* recv_scale, const int32_t* send_row, const int32_t* slot,
                      int64_t M, int32_t k, void* expert_in, float* expert_scale,
                      int64_t expert_rows, hipStream_t stream);

/*
 * moe_combine_partial -- per-(token, bucket) partial sums on the receiver:
 *
 *   partial[r] = bf16_rne( sum over j with send_row[t,j] = r, j ascending,
 *                          of w[t,j] * expert_out[slot[t,j]] )
 *
 * fp32 accumulator from +0.0, one rounded multiply and one rounded add per term (no
 * fused multiply-add), one final rounding -- the order rule of "Purlin: Separating
 * Orchestration from the Datapath of Collectives", section 3.3 (SCORE).
 *
 *   expert_out  bf16 [expert_rows, N], slot-indexed, 16-byte aligned.
 *   weights     float [M*k]; slot, send_row int32 [M*k] (dedup layout).
 *   partial     bf16 [partial_rows, N]; rows named by send_row are written.
 * Entries with a slot outside [0, expert_rows) contribute nothing; send rows outside
 * [0, partial_rows) are skipped.
 * Errors: as moe_combine.
 */
moe_status moe_combine_partial(const uint16_t* expert_out, int64_t expert_rows,
                               const float* weights, const int32_t* slot,
                               const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                               uint16_t* partial, int64_t partial_rows, hipStream_t stream);

/*
 * moe_combine_reduce -- the sender adds a token's partials:
 *
 *   y[t] = bf16_rne( sum over the distinct r in send_row[t, 0..k), ascending (that is,
 *                    ascending bucket), of f32(partial[r]) )
 *
 * fp32 accumulator from +0.0, one final rounding.
 *   partial  bf16 [partial_rows, N]; send_row int32 [M*k]; y bf16 [M, N].
 * Errors: as moe_combine.
 */
moe_status moe_combine_reduce(const uint16_t* partial, int64_t partial_rows,
                              const int32_t* send_row, int64_t M, int32_t k, int32_t N,
                              uint16_t* y, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------
 * Correlation-aware placement.  Experts that tokens choose together are placed on the
 * same destination, so the token's copies there collapse into one ("Zyphra says
 * routing-pattern expert placement speeds MoE token communication up to 2.63x on AMD
 * MI300X", the pair statistics and copy-reduction items; the page states the idea,
 * the counting and the greedy below are this library's reading of it).
 * ---------------------------------------------------------------------------------
 */

/*
 * moe_expert_pair_counts -- co-occurrence of experts over a routing batch (device):
 *   pair_counts[a*G + b] = number of tokens whose expert set holds both a and b
 *   (a token naming an expert twice counts once); pair_counts[a*G + a] = number of
 *   tokens choosing a.  Symmetric, exact integers.
 *   topk_idx     int32 [M*k]; ids outside [0, G) are ignored.
 *   pair_counts  int32 [G*G], overwritten (no prior zeroing needed).
 * Errors: MOE_ERR_INVALID_ARGUMENT (null, M < 0, k < 1, G < 1), MOE_ERR_UNSUPPORTED
 * (G > 1024, k > 16, M*k >= 2^31), MOE_ERR_LAUNCH.
 */
moe_status moe_expert_pair_counts(const int32_t* topk_idx, int64_t M, int32_t k, int32_t G,
                                  int32_t* pair_counts, hipStream_t stream);

/*
 * moe_place_experts -- greedy expert -> bucket placement from pair counts (HOST
 * pointers, synchronous, deterministic).  Every bucket gets G/B experts:
 *   1. each expert is its own cluster;
 *   2. pairs (a < b) with count > 0 are visited by count descending, ties by a then b;
 *      a pair joins its two clusters when the merged size is at most G/B;
 *   3. clusters, by size descending then smallest member, go whole into the
 *      lowest-numbered bucket with room;
 *   4. experts of clusters that fit nowhere fill the remaining places in order.
 *   pair_counts    int32 [G*G] host array (as moe_expert_pair_counts writes it).
 *   expert_bucket  int32 [G] host array, written.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null, G < 1, B < 1, G % B != 0),
 * MOE_ERR_UNSUPPORTED (G > 1024, B > 64).
 */
moe_status moe_place_experts(const int32_t* pair_counts, int32_t G, int32_t B,
                             int32_t* expert_bucket);

/*
 * ---------------------------------------------------------------------------------
 * The expert step between dispatch and combine: a grouped GEMM over the per-expert
 * layout, driven by tile metadata built on the device from the layout's offsets, with
 * no device -> host synchronisation ("Add Triton grouped-GEMM for MoE experts on
 * Ampere/Ada", "What this PR does": 2D x 3D with per-group offsets, a tile -> group
 * map computed on the device, weights in their native [E, N, K] layout).
 * ---------------------------------------------------------------------------------
 */
#define MOE_GEMM_TILE_M 256 /* rows per tile moe_grouped_gemm expects (tile_m) */

/* Host-side bound on the number of row tiles: ceil(rows / tile_m) + G. */
int32_t moe_grouped_gemm_max_tiles(int64_t rows, int32_t G, int32_t tile_m);

/*
 * moe_grouped_gemm_tiles -- row tiles of each expert's run (device):
 *   experts in ascending id; expert e's rows [expert_offset[e], +expert_count[e]) cut
 *   into tiles of tile_m rows (the last shorter).  For t < num_tiles:
 *   tile_expert[t] = e, tile_row0[t] = first row, tile_rows[t] = rows; entries
 *   t >= num_tiles (up to max_tiles) get tile_expert = -1.
 *   expert_offset, expert_count  int32 [G] from moe_dispatch_layout.
 *   tile_expert, tile_row0, tile_rows  int32 [max_tiles]; num_tiles int32 [1].
 * Errors: MOE_ERR_INVALID_ARGUMENT (null, G < 1, tile_m < 1, max_tiles < 0),
 * MOE_ERR_UNSUPPORTED (G > 1024), MOE_ERR_LAUNCH.
 */
moe_status moe_grouped_gemm_tiles(const int32_t* expert_offset, const int32_t* expert_count,
                                  int32_t G, int32_t tile_m, int32_t* tile_expert,
                                  int32_t* tile_row0, int32_t* tile_rows, int32_t max_tiles,
                                  int32_t* num_tiles, hipStream_t stream);

/*
 * moe_grouped_gemm -- y[r, n] = bf16_rne( sum_k x[r, k] * w[e, n, k] ) for every row r
 * of a tile of expert e, fp32 accumulation on the matrix cores
 * (v_mfma_f32_32x32x16_bf16).
 *   x  bf16 [rows, K] (slot-indexed expert inputs), w bf16 [G, Nout, K],
 *   tiles from moe_grouped_gemm_tiles with tile_m = MOE_GEMM_TILE_M (any tiling with at
 *   most MOE_GEMM_TILE_M rows per tile gives the same y; rows of a tile past that many
 *   are not computed),
 *   y  bf16 [rows, Nout]; rows outside every tile are not written.
 *   Every element is the same whichever launch shape and kernel body run (operands
 *   copied global -> LDS directly when K % 128 == 0 and the grid fills the chip, staged
 *   through registers otherwise): each output element is one lane's k-ordered fp32
 *   accumulation.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null or misaligned pointers, sizes < 1),
 * MOE_ERR_UNSUPPORTED (K % 64 != 0, Nout % 128 != 0, MOE_GEMM_TILE_M * K * 2 > 2^31 - 1,
 * max_tiles * Nout / 128 > 2^23),
 * MOE_ERR_LAUNCH.  Tiles are checked on the device: a tile whose expert lies outside
 * [0, G) or whose first row lies outside [0, rows) is skipped, and a tile's rows are
 * clipped to end at row `rows`, so no tile arrays can make the kernel touch memory
 * outside x, w and y.
 */
moe_status moe_grouped_gemm(const uint16_t* x, int64_t rows, int32_t K, const uint16_t* w,
                            int32_t G, int32_t Nout, const int32_t* tile_expert,
                            const int32_t* tile_row0, const int32_t* tile_rows,
                            int32_t max_tiles, uint16_t* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H_ */
