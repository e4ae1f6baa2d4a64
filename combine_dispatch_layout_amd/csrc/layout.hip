// Dispatch layout on gfx950: expert / bucket histograms, their exclusive scans and
// the stable slot map.
//
// What is computed (passages on the pages):
//  - per-destination splits and their cumulative sums for a send buffer grouped by
//    destination ("All2all performance comparison between Triton-distributed and
//    DeepEP", "Test Code Snippet");
//  - per-expert offsets that stay on the device for the grouped GEMM ("Add Triton
//    grouped-GEMM for MoE experts on Ampere/Ada", "What this PR does");
//  - one send row per (token, destination) in dedup mode ("Zyphra says
//    routing-pattern expert placement ...", the copy-reduction item).
//
// Building blocks (device functions shared by the kernels below):
//  - tile_expert_ranks (tile_load_ids, then the rank phases): one workgroup of NW
//    waves per tile of TT tokens (256 unless stated).  Each wave64 holds NC
//    consecutive 64-entry chunks of the tile's (t, j) entries in flat order.  Entries
//    of a chunk that name the same expert are found with ceil(log2 G) ballots (lanes
//    agreeing on every bit of the id), the ballots of all chunks interleaved; per
//    chunk, one leader lane per distinct expert adds the chunk's count to the wave's
//    LDS counter with an atomic that returns the old value (a wave's LDS operations
//    complete in order, so it counts the earlier chunks), and the peers fetch it from
//    the leader.  No same-address LDS atomics under skew.  That value plus the lane's
//    rank among its peers (mbcnt) is the entry's stable rank in the wave; a cross-wave
//    prefix makes it the rank in the tile.
//  - tile_dedup_ranks (in phases too): token view (lane = token).  Per-token bucket
//    bitmask; one ballot per bucket gives each token's rank among the tile's tokens
//    sending there.
//  - expert_sigma_positions / expert_order_offsets: experts ranked by (bucket, id)
//    with the same ballot matching (key = bucket), from the map alone; then a
//    block-wide exclusive scan of the counts in that order gives every expert's
//    offset; a map whose bucket never decreases with the id skips the ranking (id
//    order).
//
// Kernels:
//  - M <= 256 tokens (one tile): layout_single_kernel does everything in LDS in one
//    launch.
//  - M <= 512 with the row scatter in the same launch: layout_dispatch_small_kernel
//    (every workgroup recomputes the layout in LDS, then copies its share of rows).
//  - 2 to kOnePassMaxTiles tiles (M <= 16384): layout_onepass_kernel, one launch.
//    Each tile counts its entries and publishes the counts, ranks its entries and
//    orders the experts while the other tiles' counts arrive, waits (bounded) until
//    every tile has published, reduces the columns it needs itself and writes its
//    slots from registers.  Up to
//    kOnePassMaxTiles tiles of 1024 tokens (M <= 65536, k <= 8) take the same kernel
//    with 16 waves of one 64-token group each (tiles of 512 tokens, 8 such waves, for
//    M <= 32768); at k >= 5 it takes tiles of 64 tokens (8 waves) for 257 <= M <= 2048
//    and of 128 tokens for M <= 8192 instead.
//  - more tiles (or k > 8 above 16384 tokens): three launches, no inter-workgroup
//    waiting:
//    layout_tile_kernel (per-tile ranks and totals to the workspace),
//    layout_scan_kernel (one 1024-thread workgroup scans each expert / bucket column
//    over tiles, orders experts, writes counts, offsets and the status word),
//    layout_finalize_kernel (one thread per entry: offset + tile prefix + rank).
#include "moe_internal.h"

namespace moedl {

namespace {

constexpr int kMaxE = MOE_MAX_EXPERTS;
constexpr int kMaxB = MOE_MAX_BUCKETS;
constexpr unsigned char kBadBucket = 0xFF;
constexpr int kAbsent = -1;  // no entry (past the end, or an invalid id)
constexpr int kExpertBits = 10;  // bits of an expert id (G <= 1024)
constexpr int kBucketBits = 6;   // bits of a bucket id (B <= 64)
static_assert(kMaxE <= (1 << kExpertBits) && kMaxB <= (1 << kBucketBits), "id widths");

__device__ __forceinline__ int bits_for(int n) {  // bits needed for values in [0, n)
  return n <= 1 ? 0 : 32 - __builtin_clz((unsigned)(n - 1));
}

// Peer masks of C independent 64-entry chunks at once: peers[c] = the lanes whose
// key[c] equals the caller's, among lanes with ok[c] set (meaningless where ok[c] is
// false).  Lanes agree on a key when they agree on each of its nbits bits, one ballot
// per bit.  The bit loop is outside the chunk loop and fully unrolled, so the ballots
// of different chunks interleave instead of forming one long dependent chain.  Per bit
// and chunk: m = the bit spread over the word, the ballot, and peers &= ~(ballot ^ m)
// as one three-input logic op per half (v_bitop3; truth table 0x84 with the mask as
// the middle operand, which reads the same whichever outer operand indexes first).
template <int C, int MAXBITS>
__device__ __forceinline__ void match_peers(const bool (&ok)[C], const int (&key)[C], int nbits,
                                            uint64_t (&peers)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) peers[c] = wave_ballot(ok[c]);
#pragma unroll
  for (int bit = 0; bit < MAXBITS; ++bit) {
    if (bit < nbits) {  // uniform
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t m = (uint32_t)((int32_t)((uint32_t)key[c] << (31 - bit)) >> 31);
        const uint64_t bal = wave_ballot(m != 0u);
        const uint32_t lo = __builtin_amdgcn_bitop3_b32((uint32_t)bal, (uint32_t)peers[c], m, 0x84);
        const uint32_t hi =
            __builtin_amdgcn_bitop3_b32((uint32_t)(bal >> 32), (uint32_t)(peers[c] >> 32), m, 0x84);
        peers[c] = ((uint64_t)hi << 32) | lo;
      }
    }
  }
}

// Stable ranks of C chunks against per-key running counters in LDS (counter[key]).
// For each chunk in order, one leader lane per distinct key adds the key's count in
// the chunk with an LDS atomic that returns the previous value; a wave's LDS
// operations complete in issue order, so that value counts exactly the earlier
// chunks.  Peers fetch it from their leader (ds_bpermute) and add their rank among
// the chunk's peers: rank[c] = entries with the same key before this one, in order
// (chunk, lane).
template <int C>
__device__ __forceinline__ void stable_ranks(const bool (&ok)[C], const int (&key)[C],
                                             const uint64_t (&peers)[C], int32_t* counter,
                                             int (&rank)[C]) {
  const int lane = threadIdx.x & 63;
  int old[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    old[c] = 0;
    const int below = lanes_below(peers[c]);
    if (ok[c] && below == 0) old[c] = atomicAdd(counter + key[c], __builtin_popcountll(peers[c]));
    rank[c] = below;
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int leader = ok[c] ? __builtin_ctzll(peers[c]) : lane;
    rank[c] += __builtin_amdgcn_ds_bpermute(leader << 2, old[c]);
  }
}

// The flat (t, j) entries of a tile are split over its waves in NC chunks of 64
// entries each: wave w holds entries [tile * 256 * k + w * 64 * NC, + 64 * NC), chunk c
// lane l being the entry at offset c * 64 + l.  NC = k rounded up to a power of two
// covers a full tile; a single short tile (small M) takes the smallest NC that covers
// it, so the work is spread over all waves with no idle chunks.
template <int NC, int TT = kTileTokens>
__device__ __forceinline__ int64_t wave_first_entry(int tile, int32_t k, int w) {
  return (int64_t)tile * TT * k + (int64_t)w * 64 * NC;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes inside each row of 16 (lanes shifted in from outside
// the row read 0), then the last lane of rows 0 and 2 is added to rows 1 and 3
// (row_bcast:15), and lane 31 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive scan of src[0, n) into dst by one wave (n <= 64); dst[n] = the total when
// with_total.  src may be dst (every lane reads before any writes).  Callers put
// barriers around it.
__device__ __forceinline__ void small_exclusive_scan(const int32_t* src, int32_t* dst, int n,
                                                     bool with_total, int wave = 0) {
  if ((int)(threadIdx.x >> 6) == wave) {
    const int lane = threadIdx.x & 63;
    const int v = lane < n ? src[lane] : 0;
    const int incl = wave_inclusive_sum(v);
    if (lane < n) dst[lane] = incl - v;
    if (with_total && lane == 63) dst[n] = incl;
  }
}

// A tile of TT tokens (kTileTokens unless stated) has its tokens one per lane in its
// first TT / 64 waves (the token view of the dedup ranks); its (t, j) entries are
// spread over all NW waves of the workgroup.

template <int KC, int NW = kTileWaves, int TT = kTileTokens>  // KC: k rounded up to a power of two
struct TileLds {
  unsigned char map_s[kMaxE];
  int32_t wcnt[NW][kMaxE];                // per-wave running counts, then prefixes
  int32_t ids_s[TT * KC];                 // the tile's expert ids, flat order
  uint64_t wbal[TT / 64][kMaxB];          // dedup: per-wave ballot of each bucket
  int32_t wbcnt[TT / 64][kMaxB];          // dedup: per-wave counts, then prefixes
  int32_t err_s;                          // first bad flat index in the tile
};

// Last flat entry (exclusive) of a tile.
template <int TT = kTileTokens>
__device__ __forceinline__ int64_t tile_end_entry(int32_t M, int32_t k, int tile) {
  const int64_t Mk = (int64_t)M * k;
  const int64_t e = ((int64_t)tile + 1) * TT * k;
  return e < Mk ? e : Mk;
}

// First half of tile_expert_ranks: ec[c] = the expert id of flat entry
// wave_first_entry<NC, TT>(tile, k, w) + c*64 + lane, or kAbsent (past the end, or an
// id outside [0, G), whose first flat index goes to lds.err_s), ok[c] = present;
// lds.map_s holds the map and the per-wave counters are zero (both complete after the
// barrier inside); lds.ids_s holds the tile's ids (tile-local flat order) when
// keep_ids, written after that barrier: readers in other waves need another one.
template <int KC, int NC, int NW = kTileWaves, int TT = kTileTokens>
__device__ __forceinline__ void tile_load_ids(TileLds<KC, NW, TT>& lds, const int32_t* __restrict__ idx,
                                              int32_t M, int32_t k,
                                              const int32_t* __restrict__ ebkt, int32_t G,
                                              int32_t B, int tile, bool keep_ids,
                                              int (&ec)[NC], bool (&ok)[NC]) {
  static_assert(NC * NW <= KC * (TT / 64), "a wave's chunks must fit the tile's id store");
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int64_t wbase = wave_first_entry<NC, TT>(tile, k, w);
  const int64_t tend = tile_end_entry<TT>(M, k, tile);
  const int local0 = w * 64 * NC;  // tile-local index of the wave's first entry

  // all global loads first: clamped, unconditional, so they are in flight together
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    const bool valid = f < tend;
    const int v = idx[valid ? f : 0];
    ec[c] = valid ? v : kAbsent;
  }
  for (int e = tid; e < G; e += NT) {
    const int b = ebkt[e];
    lds.map_s[e] = (b >= 0 && b < B) ? (unsigned char)b : kBadBucket;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) lds.wcnt[ww][e] = 0;
  }
  if (tid == 0) lds.err_s = kNoError;
  __syncthreads();

  int my_err = kNoError;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int e = ec[c];
    if (e != kAbsent && (e < 0 || e >= G)) {
      my_err = min(my_err, (int)(wbase + c * 64 + lane));
      e = kAbsent;
    }
    if (keep_ids) lds.ids_s[local0 + c * 64 + lane] = e;
    ok[c] = e >= 0;
    ec[c] = e;
  }
  if (my_err != kNoError) atomicMin(&lds.err_s, my_err);
}

// Second half: the stable ranks of the loaded entries, in three phases that callers
// separate with barriers (tile_rank_entries below; the one-launch layout interleaves
// them with the dedup ranks' phases).  After the last, rc[c] is the rank inside the
// tile of entry c (meaningless where ec[c] is absent); totals[e] (global or LDS, or
// null) holds the tile's count of expert e after the second.
template <int KC, int NC, int NW, int TT>
__device__ __forceinline__ void rank_phase_match(TileLds<KC, NW, TT>& lds, int32_t G,
                                                 const bool (&ok)[NC], const int (&ec)[NC],
                                                 int (&rc)[NC]) {
  uint64_t peers[NC];
  match_peers<NC, kExpertBits>(ok, ec, bits_for(G), peers);
  stable_ranks<NC>(ok, ec, peers, lds.wcnt[wave_index()], rc);
}
template <int KC, int NW, int TT>
__device__ __forceinline__ void rank_phase_prefix(TileLds<KC, NW, TT>& lds, int32_t G,
                                                  int32_t* totals) {
  // cross-wave exclusive prefix per expert; the column total is the tile's count
  for (int e = threadIdx.x; e < G; e += NW * 64) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int v = lds.wcnt[ww][e];
      lds.wcnt[ww][e] = run;
      run += v;
    }
    if (totals != nullptr) totals[e] = run;
  }
}
template <int KC, int NC, int NW, int TT>
__device__ __forceinline__ void rank_phase_finish(TileLds<KC, NW, TT>& lds, const int (&ec)[NC],
                                                  int (&rc)[NC]) {
  const int w = wave_index();
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (ec[c] >= 0) rc[c] += lds.wcnt[w][ec[c]];
}

template <int KC, int NC, int NW = kTileWaves, int TT = kTileTokens>
__device__ __forceinline__ void tile_rank_entries(TileLds<KC, NW, TT>& lds, int32_t G,
                                                  const bool (&ok)[NC], const int (&ec)[NC],
                                                  int32_t* totals, int (&rc)[NC]) {
  rank_phase_match<KC, NC, NW, TT>(lds, G, ok, ec, rc);
  __syncthreads();
  rank_phase_prefix<KC, NW, TT>(lds, G, totals);
  __syncthreads();
  rank_phase_finish<KC, NC, NW, TT>(lds, ec, rc);
}

// Expert ranks of one tile of TT tokens (256 unless stated), NW waves of NC chunks
// each (see wave_first_entry; NW * NC = (TT / 64) * KC covers the tile).  On return
// (after a barrier): ec[c] / rc[c] hold the expert id (or kAbsent) and the rank inside
// the tile of flat entry wave_first_entry<NC, TT>(tile, k, w) + c*64 + lane; totals[e] holds the tile's
// count of expert e (totals may be global or LDS); lds.ids_s holds the tile's ids
// (tile-local flat order) when keep_ids.
template <int KC, int NC, int NW = kTileWaves, int TT = kTileTokens>
__device__ __forceinline__ void tile_expert_ranks(TileLds<KC, NW, TT>& lds, const int32_t* __restrict__ idx,
                                                  int32_t M, int32_t k,
                                                  const int32_t* __restrict__ ebkt, int32_t G,
                                                  int32_t B, int tile, bool keep_ids,
                                                  int32_t* totals, int (&ec)[NC], int (&rc)[NC]) {
  bool ok[NC];
  tile_load_ids<KC, NC, NW, TT>(lds, idx, M, k, ebkt, G, B, tile, keep_ids, ec, ok);
  tile_rank_entries<KC, NC, NW, TT>(lds, G, ok, ec, totals, rc);
}

// Dedup ranks of one tile (token view: token w*64 + lane of the tile in waves w <
// TT / 64; later waves hold no token).  Needs lds.ids_s from tile_expert_ranks.
// Three phases that callers separate with barriers (tile_dedup_ranks below).  After
// the last: eb[j] is the bucket of the lane's token's j-th entry or kBadBucket, dl[j]
// the token's rank among the tile's tokens that send to that bucket; btotals[b]
// (unless null) the tile's distinct-token count of bucket b after the second.
template <int KC, int NW, int TT>
__device__ __forceinline__ void dedup_phase_ballots(TileLds<KC, NW, TT>& lds, int32_t M, int32_t k,
                                                    int32_t B, int tile, int (&eb)[KC]) {
  constexpr int TW = TT / 64;  // token waves
  static_assert(TW <= NW, "every token has a lane");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const bool token_wave = w < TW;
  const int64_t t = (int64_t)tile * TT + (int64_t)w * 64 + lane;
  const bool tv = token_wave && t < M;
  const int* my_ids = lds.ids_s + ((token_wave ? w * 64 : 0) + lane) * k;
  // Branch-free throughout: every LDS read is unconditional (clamped index, value
  // replaced afterwards), so the reads of all j are in flight together.
  int ev[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) ev[j] = (j < k && tv) ? my_ids[j] : kAbsent;
  uint64_t bmask = 0;
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int m = lds.map_s[ev[j] >= 0 ? ev[j] : 0];
    eb[j] = ev[j] >= 0 ? m : kBadBucket;
    if (eb[j] != kBadBucket) bmask |= 1ull << eb[j];
  }
  // one ballot per bucket; lane b keeps bucket b's ballot and writes it
  uint64_t mine = 0;
  for (int b = 0; b < B; ++b) {
    const uint64_t bal = wave_ballot(tv && ((bmask >> b) & 1ull));
    mine = lane == b ? bal : mine;
  }
  if (token_wave && lane < B) {
    lds.wbal[w][lane] = mine;
    lds.wbcnt[w][lane] = __builtin_popcountll(mine);
  }
}
template <int KC, int NW, int TT>
__device__ __forceinline__ void dedup_phase_prefix(TileLds<KC, NW, TT>& lds, int32_t B,
                                                   int32_t* btotals) {
  const int tid = threadIdx.x;
  if (tid < B) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < TT / 64; ++ww) {
      const int v = lds.wbcnt[ww][tid];
      lds.wbcnt[ww][tid] = run;
      run += v;
    }
    if (btotals != nullptr) btotals[tid] = run;
  }
}
template <int KC, int NW, int TT>
__device__ __forceinline__ void dedup_phase_finish(TileLds<KC, NW, TT>& lds, const int (&eb)[KC],
                                                   int (&dl)[KC]) {
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const uint64_t below = (1ull << lane) - 1ull;
  const int wt = w < TT / 64 ? w : 0;  // waves without tokens read a valid row, unused
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int b = eb[j] != kBadBucket ? eb[j] : 0;
    const int base = lds.wbcnt[wt][b];
    const uint64_t bal = lds.wbal[wt][b];
    dl[j] = eb[j] != kBadBucket ? base + __builtin_popcountll(bal & below) : -1;
  }
}

template <int KC, int NW = kTileWaves, int TT = kTileTokens>
__device__ __forceinline__ void tile_dedup_ranks(TileLds<KC, NW, TT>& lds, int32_t M, int32_t k,
                                                 int32_t B, int tile, int32_t* btotals,
                                                 int (&eb)[KC], int (&dl)[KC]) {
  dedup_phase_ballots<KC, NW, TT>(lds, M, k, B, tile, eb);
  __syncthreads();
  dedup_phase_prefix<KC, NW, TT>(lds, B, btotals);
  __syncthreads();
  dedup_phase_finish<KC, NW, TT>(lds, eb, dl);
}

// Distinct-token counts of the tile's buckets, token view as in tile_dedup_ranks:
// bcnt[b] gains one for every token of the tile that sends to bucket b (LDS adds, no
// ranks).  bcnt must be zero and lds.ids_s / lds.map_s complete; callers put a barrier
// after it.
template <int KC, int NW, int TT>
__device__ __forceinline__ void tile_bucket_counts(TileLds<KC, NW, TT>& lds, int32_t M, int32_t k,
                                                   int tile, int32_t* bcnt) {
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  const int64_t t = (int64_t)tile * TT + (int64_t)w * 64 + lane;
  if (w >= TT / 64 || t >= M) return;
  const int* my_ids = lds.ids_s + (w * 64 + lane) * k;
  int ev[KC], m[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) ev[j] = j < k ? my_ids[j] : kAbsent;
#pragma unroll
  for (int j = 0; j < KC; ++j) m[j] = lds.map_s[ev[j] >= 0 ? ev[j] : 0];
  uint64_t seen = 0;
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (ev[j] < 0 || m[j] == kBadBucket || ((seen >> m[j]) & 1ull)) continue;
    seen |= 1ull << m[j];
    atomicAdd(bcnt + m[j], 1);
  }
}

// Exclusive scan of one int per thread over an NT-thread workgroup: a DPP scan in
// each wave, then every wave adds the totals of the waves before it (independent LDS
// reads, no serial step).
template <int NT>
__device__ int block_exclusive_scan(int v, int32_t* wave_sums /* >= NT/64 */) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int incl = wave_inclusive_sum(v);
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) base += q < w ? wave_sums[q] : 0;
  __syncthreads();  // wave_sums is reused by the next call
  return base + incl - v;
}

// LDS for expert_order_offsets.
template <int NT>
struct OrderLds {
  int32_t wbc[NT / 64][kMaxB];  // per-wave per-bucket expert counts, then prefixes
  int32_t base[kMaxB + 1];      // first sigma position of each bucket
  int32_t arr[kMaxE];           // counts in sigma order, then their exclusive scan
  int32_t wave_sums[NT / 64];
};

template <int NT>
constexpr int order_chunks() { return (kMaxE + NT - 1) / NT; }  // 64-expert chunks per wave

// Positions of the experts in (bucket, id) order, from the map alone.  NT-thread
// workgroup; wave w ranks a contiguous range of experts (w * per + c * 64 + lane) so
// the cross-wave prefix keeps id order.  On return (after a barrier) pos[c] is the
// position of expert w * per + c * 64 + lane (-1 past G) and lds.base[b] the first
// position of bucket b.  A bad map entry is ranked as bucket B - 1 (callers report
// it).
template <int NT>
__device__ void expert_sigma_positions(OrderLds<NT>& lds, const unsigned char* map_s,
                                       int32_t G, int32_t B, int (&pos)[order_chunks<NT>()]) {
  constexpr int NW = NT / 64;
  constexpr int CH = order_chunks<NT>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int per = ((G + NW - 1) / NW + 63) / 64 * 64;  // experts per wave, whole chunks
  for (int i = tid; i < NW * kMaxB; i += NT) lds.wbc[i / kMaxB][i % kMaxB] = 0;
  __syncthreads();

  const int nbits = bits_for(B);
  int rk[CH];
  int bk[CH];
  bool okc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = w * per + c * 64 + lane;
    okc[c] = c * 64 < per && e < G;
    int b = okc[c] ? (int)map_s[e] : 0;
    bk[c] = b < B ? b : B - 1;  // a bad map entry is reported by status; keep it in range
  }
  uint64_t peers[CH];
  match_peers<CH, kBucketBits>(okc, bk, nbits, peers);
  stable_ranks<CH>(okc, bk, peers, lds.wbc[w], rk);
  __syncthreads();
  if (tid < B) {
    int run = 0;
    for (int q = 0; q < NW; ++q) {
      const int v = lds.wbc[q][tid];
      lds.wbc[q][tid] = run;
      run += v;
    }
    lds.base[tid] = run;
  }
  __syncthreads();
  small_exclusive_scan(lds.base, lds.base, B, false);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CH; ++c)
    pos[c] = okc[c] ? lds.base[bk[c]] + lds.wbc[w][bk[c]] + rk[c] : -1;
}

// Offsets of expert runs laid out in (bucket, id) order, from per-expert counts
// cnt[G] (LDS).  NT-thread workgroup.  A map whose bucket never decreases with the
// id takes a fast path (id order).  Writes offset[e] (global or LDS).
template <int NT>
__device__ void expert_order_offsets(OrderLds<NT>& lds, const unsigned char* map_s,
                                     const int32_t* cnt, int32_t G, int32_t B,
                                     int32_t* offset) {
  constexpr int NW = NT / 64;
  constexpr int CH = order_chunks<NT>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int per = ((G + NW - 1) / NW + 63) / 64 * 64;  // experts per wave, whole chunks

  // Contiguous maps (the bucket never decreases with the expert id; the common case)
  // order experts by id: the ranking is skipped and the counts are scanned in place.
  // (One wave alone scanning the counts, with the map checked by a ballot in every wave
  // and no barrier before it, measured 0.2 us slower at G = 256.)
  int mono = 1;
  for (int e = tid; e + 1 < G; e += NT) mono &= map_s[e] <= map_s[e + 1];
  if (__syncthreads_and(mono)) {
    int local[CH];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = tid * CH + u;
      local[u] = i < G ? cnt[i] : 0;
      sum += local[u];
    }
    int run = block_exclusive_scan<NT>(sum, lds.wave_sums);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = tid * CH + u;
      if (i < G) offset[i] = run;
      run += local[u];
    }
    __syncthreads();
    return;
  }

  int pos[CH];
  expert_sigma_positions<NT>(lds, map_s, G, B, pos);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = w * per + c * 64 + lane;
    if (pos[c] >= 0) lds.arr[pos[c]] = cnt[e];
  }
  __syncthreads();
  // exclusive scan of arr[0, G): thread tid owns CH consecutive entries
  int local[CH];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int i = tid * CH + u;
    local[u] = i < G ? lds.arr[i] : 0;
    sum += local[u];
  }
  int run = block_exclusive_scan<NT>(sum, lds.wave_sums);
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int i = tid * CH + u;
    if (i < G) lds.arr[i] = run;
    run += local[u];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = w * per + c * 64 + lane;
    if (pos[c] >= 0) offset[e] = lds.arr[pos[c]];
  }
  __syncthreads();
}

// ------------------------------------------------------------------ M <= 256 tokens
template <int KC, int NC>
__global__ __launch_bounds__(kTileThreads) void layout_single_kernel(
    const int32_t* __restrict__ idx, int32_t M, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ bucket_count, int32_t* __restrict__ bucket_offset,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_row,
    int32_t* __restrict__ send_token, int32_t* __restrict__ status) {
  __shared__ TileLds<KC> lds;
  __shared__ OrderLds<kTileThreads> olds;
  __shared__ int32_t cnt_s[kMaxE];
  __shared__ int32_t off_s[kMaxE];
  __shared__ int32_t bsum_s[kMaxB];
  __shared__ int32_t btot_s[kMaxB];
  __shared__ int32_t boff_s[kMaxB + 1];
  __shared__ int32_t mapbad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int64_t Mk = (int64_t)M * k;
  if (tid < kMaxB) bsum_s[tid] = 0;
  if (tid == 0) mapbad_s = kNoError;

  int ec[NC], rc[NC];
  tile_expert_ranks<KC, NC>(lds, idx, M, k, ebkt, G, B, 0, dedup != 0, cnt_s, ec, rc);
  for (int e = tid; e < G; e += kTileThreads) {
    if (lds.map_s[e] == kBadBucket) atomicMin(&mapbad_s, e);
    else atomicAdd(&bsum_s[lds.map_s[e]], cnt_s[e]);
  }
  expert_order_offsets<kTileThreads>(olds, lds.map_s, cnt_s, G, B, off_s);

  int eb[KC], dl[KC];
  if (dedup) {
    tile_dedup_ranks<KC>(lds, M, k, B, 0, btot_s, eb, dl);
  } else if (tid < B) {
    btot_s[tid] = bsum_s[tid];
  }
  __syncthreads();
  small_exclusive_scan(btot_s, boff_s, B, true);
  __syncthreads();

  for (int e = tid; e < G; e += kTileThreads) {
    expert_count[e] = cnt_s[e];
    expert_offset[e] = off_s[e];
  }
  if (tid < B) bucket_count[tid] = btot_s[tid];
  if (tid <= B) bucket_offset[tid] = boff_s[tid];
  if (tid == 0)
    status[0] = mapbad_s != kNoError ? -(mapbad_s + 1)
                                     : (lds.err_s != kNoError ? lds.err_s + 1 : 0);

  const int64_t wbase = wave_first_entry<NC>(0, k, w);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (f < Mk) {
      const int s = ec[c] >= 0 ? off_s[ec[c]] + rc[c] : -1;
      slot[f] = s;
      if (!dedup) {
        send_row[f] = s;
        if (s >= 0 && s < Mk) send_token[s] = (int)(f / k);
      }
    }
  }
  if (dedup) {
    const int t = w * 64 + lane;
    const int64_t cap = (int64_t)M * (k < B ? k : B);
    if (t < M) {
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (j < k) {
          const int r = eb[j] != kBadBucket ? boff_s[eb[j]] + dl[j] : -1;
          send_row[(int64_t)t * k + j] = r;
          if (r >= 0 && r < cap) send_token[r] = t;
        }
      }
    }
  }
}

// ------------------------------------------- layout + dispatch in one launch, M <= 512
// The small-M regime is set by launches and the gaps between them, not by bytes, so
// layout and row scatter share one launch.  Every workgroup computes the complete
// layout of the (at most two) 256-token tiles in its own LDS with the building blocks
// above.  The computation is deterministic, so all workgroups hold the same layout and
// none ever waits for another; workgroup 0 alone writes the layout arrays.  Then the
// workgroups share the row copies: work item i = (token, 4 KiB piece of its row) goes to
// workgroup i mod gridDim.x, which loads the piece once (a batch of items at a time, all
// loads in flight) and stores it non-temporally to each of the token's distinct send
// rows inside the buffer.  Without dedup (and k >= 4) the items are 1 KiB pieces
// instead, and the workgroup's four waves share the token's k rows (wave w stores rows
// j = w, w + 4, ...), as the separate dispatch kernel spreads its stores over waves:
// measured (graph replay, N=7168, top-8, this call + combine of its rows) 9.8 / 12.6 /
// 18.8 us at M = 64 / 128 / 256 against 11.9 / 16.4 / 21.6 with 4 KiB items, the
// combine after it reading the rows faster (the call alone: 6.4 / 8.2 / 12.1 against
// 6.5 / 8.1 / 12.3).  In dedup mode the 4 KiB items stay: the waves would share a
// token's ~4.6 distinct rows unevenly (14.2 vs 14.1 us at M = 128, 20.3 vs 19.4 at 256),
// and compacting the distinct rows first did not help (14.5, 20.6).  The LDS row table holds each distinct row once (dedup repeats
// are marked absent while the layout is built), so the scatter reads a token's k rows
// together and needs no duplicate search.  Issuing the first batch of row loads before
// the layout work was measured slower (vector-load counters retire in order, so the
// layout's first wait on topk_idx also waited on the rows).  `idx` must be readable at
// index 0 even when M = 0.
constexpr int kFusedPieceVecs = kTileThreads;  // 16-byte vectors per work item
constexpr int kFusedBatch = 4;                  // work items loaded together
constexpr int kFusedFlatPieceVecs = 64;         // the same, 1 KiB items (no dedup, k >= 4)
constexpr int kFusedFlatBatch = 2;
// Grid cap: two workgroups per CU, which fit at once for every instantiation (41-68 KiB
// of LDS each).  Every workgroup recomputes the layout before copying, so a grid that
// does not fit at once pays that again in a second wave, while fewer workgroups give
// the copies less parallelism.  Measured (graph replay, layout + dispatch + combine,
// N=7168, top-8, dedup off): cap 128 / 256 / 512 / 1024 -> 25.5 / 22.5 / 22.5 / 28.1 us
// at M=256, 45.8 / 36.9 / 36.2 / 46.1 us at M=512; dedup on alike.
constexpr int kFusedMaxBlocks = 512;

template <int KC, int NTILE, int NC, bool ITEM1K>
__global__ __launch_bounds__(kTileThreads) void layout_dispatch_small_kernel(
    const int32_t* __restrict__ idx, int32_t M, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ bucket_count, int32_t* __restrict__ bucket_offset,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_row,
    int32_t* __restrict__ send_token, int32_t* __restrict__ status,
    const u32x4* __restrict__ x, int32_t row_vecs, int32_t pieces,
    const float* __restrict__ x_scale, int32_t scale_cols, u32x4* __restrict__ out,
    float* __restrict__ out_scale, int64_t out_rows) {
  __shared__ TileLds<KC> lds;
  __shared__ OrderLds<kTileThreads> olds;
  __shared__ int32_t tcnt_s[NTILE][kMaxE];  // per-tile expert counts
  __shared__ int32_t cnt_s[kMaxE];
  __shared__ int32_t off_s[kMaxE];
  __shared__ int32_t tb_s[NTILE][kMaxB];    // per-tile distinct-token counts (dedup)
  __shared__ int32_t bsum_s[kMaxB];
  __shared__ int32_t btot_s[kMaxB];
  __shared__ int32_t boff_s[kMaxB + 1];
  __shared__ int32_t mapbad_s, err_s;
  __shared__ int32_t row_s[NTILE * kTileTokens * KC];  // send row of flat entry t*k + j

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int64_t Mk = (int64_t)M * k;
  const bool writer = blockIdx.x == 0;

  const int64_t items = (int64_t)M * pieces;
  const int64_t stride = gridDim.x;
  u32x4 v[kFusedBatch];
  auto load_batch = [&](int64_t base) {
#pragma unroll
    for (int q = 0; q < kFusedBatch; ++q) {  // clamped, unconditional loads: all in flight
      const int64_t it = base + q * stride;
      const int64_t t = it < items ? it / pieces : 0;
      const int c = (int)(it - t * pieces) * kFusedPieceVecs + tid;
      const bool in_row = it < items && c < row_vecs;
      v[q] = x[in_row ? t * row_vecs + c : 0];
    }
  };

  if (tid < kMaxB) bsum_s[tid] = 0;
  if (tid == 0) {
    mapbad_s = kNoError;
    err_s = kNoError;
  }

  int ec[NTILE][NC], rc[NTILE][NC], eb[NTILE][KC], dl[NTILE][KC];
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    if (tile > 0) __syncthreads();  // the previous tile's LDS reads are done
    tile_expert_ranks<KC, NC>(lds, idx, M, k, ebkt, G, B, tile, dedup != 0, tcnt_s[tile], ec[tile],
                          rc[tile]);
    if (tid == 0) err_s = min(err_s, lds.err_s);
    if (dedup) tile_dedup_ranks<KC>(lds, M, k, B, tile, tb_s[tile], eb[tile], dl[tile]);
  }
  __syncthreads();
  for (int e = tid; e < G; e += kTileThreads) {
    int c = tcnt_s[0][e];
    if (NTILE > 1) c += tcnt_s[NTILE - 1][e];
    cnt_s[e] = c;
    if (lds.map_s[e] == kBadBucket) atomicMin(&mapbad_s, e);
    else atomicAdd(&bsum_s[lds.map_s[e]], c);
  }
  expert_order_offsets<kTileThreads>(olds, lds.map_s, cnt_s, G, B, off_s);
  if (tid < B) {
    int bt = bsum_s[tid];
    if (dedup) {
      bt = tb_s[0][tid];
      if (NTILE > 1) bt += tb_s[NTILE - 1][tid];
    }
    btot_s[tid] = bt;
  }
  __syncthreads();
  small_exclusive_scan(btot_s, boff_s, B, true);
  __syncthreads();

  if (writer) {
    for (int e = tid; e < G; e += kTileThreads) {
      expert_count[e] = cnt_s[e];
      expert_offset[e] = off_s[e];
    }
    if (tid < B) bucket_count[tid] = btot_s[tid];
    if (tid <= B) bucket_offset[tid] = boff_s[tid];
    if (tid == 0)
      status[0] = mapbad_s != kNoError ? -(mapbad_s + 1) : (err_s != kNoError ? err_s + 1 : 0);
  }

  const int64_t cap = dedup ? (int64_t)M * (k < B ? k : B) : Mk;
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    const int64_t wbase = wave_first_entry<NC>(tile, k, w);
    const int64_t tend = tile_end_entry(M, k, tile);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t f = wbase + (int64_t)c * 64 + lane;
      if (f < tend) {
        const int e = ec[tile][c];
        int s = -1;
        if (e >= 0) s = off_s[e] + rc[tile][c] + (tile > 0 ? tcnt_s[0][e] : 0);
        if (!dedup) row_s[f] = s;
        if (writer) {
          slot[f] = s;
          if (!dedup) {
            send_row[f] = s;
            if (s >= 0 && s < Mk) send_token[s] = (int)(f / k);
          }
        }
      }
    }
    if (dedup) {
      const int t = tile * kTileTokens + w * 64 + lane;
      if (t < M) {
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          if (j < k) {
            const int b = eb[tile][j];
            const int r = b != kBadBucket ? boff_s[b] + dl[tile][j] + (tile > 0 ? tb_s[0][b] : 0)
                                          : -1;
            // a later entry of a bucket already seen has the same row: absent here
            bool repeat = false;
#pragma unroll
            for (int jj = 0; jj < KC; ++jj) repeat |= jj < j && eb[tile][jj] == b;
            row_s[t * k + j] = repeat ? -1 : r;
            if (writer) {
              send_row[(int64_t)t * k + j] = r;
              if (r >= 0 && r < cap) send_token[r] = t;
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // row scatter
  if constexpr (ITEM1K) {  // 1 KiB items, the waves share the token's rows (no dedup)
    constexpr int NWV = kTileThreads / 64;
    for (int64_t base = blockIdx.x; base < items; base += stride * kFusedFlatBatch) {
      u32x4 u[kFusedFlatBatch];
#pragma unroll
      for (int q = 0; q < kFusedFlatBatch; ++q) {  // clamped, unconditional: all in flight
        const int64_t it = base + q * stride;
        const int64_t t = it < items ? it / pieces : 0;
        const int c = (int)(it - t * pieces) * kFusedFlatPieceVecs + lane;
        const bool in_row = it < items && c < row_vecs;
        u[q] = x[in_row ? t * row_vecs + c : 0];
      }
#pragma unroll
      for (int q = 0; q < kFusedFlatBatch; ++q) {
        const int64_t it = base + q * stride;
        if (it >= items) break;  // uniform
        const int t = (int)(it / pieces);
        const int piece = (int)(it - (int64_t)t * pieces);
        const int c = piece * kFusedFlatPieceVecs + lane;
        const int32_t* rows = row_s + t * k;
        for (int j = w; j < k; j += NWV) {
          const int r = rows[j];
          if (r < 0 || r >= out_rows) continue;  // uniform
          if (c < row_vecs) __builtin_nontemporal_store(u[q], out + (int64_t)r * row_vecs + c);
          if (x_scale != nullptr && piece == 0) {
            for (int sc = lane; sc < scale_cols; sc += 64)
              out_scale[(int64_t)r * scale_cols + sc] = x_scale[(int64_t)t * scale_cols + sc];
          }
        }
      }
    }
    return;
  }
  for (int64_t base = blockIdx.x; base < items; base += stride * kFusedBatch) {
    load_batch(base);  // x may be null only when M = 0, and then there is no item
#pragma unroll
    for (int q = 0; q < kFusedBatch; ++q) {
      const int64_t it = base + q * stride;
      if (it >= items) break;  // uniform
      const int t = (int)(it / pieces);
      const int piece = (int)(it - (int64_t)t * pieces);
      const int c = piece * kFusedPieceVecs + tid;
      const int32_t* rows = row_s + t * k;
      int rr[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) rr[j] = j < k ? rows[j] : -1;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int r = rr[j];
        if (r < 0 || r >= out_rows) continue;  // uniform
        if (c < row_vecs) __builtin_nontemporal_store(v[q], out + (int64_t)r * row_vecs + c);
        if (x_scale != nullptr && piece == 0) {
          for (int sc = tid; sc < scale_cols; sc += kTileThreads)
            out_scale[(int64_t)r * scale_cols + sc] = x_scale[(int64_t)t * scale_cols + sc];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ M > 256 tokens
template <int KC>
__global__ __launch_bounds__(kTileThreads) void layout_tile_kernel(
    const int32_t* __restrict__ idx, int32_t M, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    int32_t* __restrict__ slot_local, int32_t* __restrict__ row_local,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_bhist,
    int32_t* __restrict__ tile_err) {
  __shared__ TileLds<KC> lds;
  const int tile = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = wave_index();
  int ec[KC], rc[KC];
  tile_expert_ranks<KC, KC>(lds, idx, M, k, ebkt, G, B, tile, dedup != 0,
                            tile_hist + (int64_t)tile * G, ec, rc);
  const int64_t wbase = wave_first_entry<KC>(tile, k, w);
  const int64_t tend = tile_end_entry(M, k, tile);
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (f < tend) slot_local[f] = ec[c] >= 0 ? rc[c] : -1;
  }
  if (dedup) {
    int eb[KC], dl[KC];
    tile_dedup_ranks<KC>(lds, M, k, B, tile, tile_bhist + (int64_t)tile * B, eb, dl);
    const int64_t t = (int64_t)tile * kTileTokens + (int64_t)w * 64 + lane;
    if (t < M) {
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (j < k) row_local[t * k + j] = dl[j];
    }
  }
  if (threadIdx.x == 0) tile_err[tile] = lds.err_s;
}

// Exclusive prefix down each column of data[T][C] (row-major), in place, using the
// whole 1024-thread workgroup: P = 1024 / C threads share a column, each owning a
// contiguous run of rows, and a short serial scan joins the runs.  Each thread
// loads its run into registers once (kSegRegs rows per round trip), so a column of
// up to P * kSegRegs tiles costs one global round trip.  totals[c] gets the column
// sum.  seg must hold kScanThreads ints.
constexpr int kSegRegs = 16;

__device__ void column_exclusive_scan(int32_t* __restrict__ data, int T, int C,
                                      int32_t* totals, int32_t* seg) {
  const int tid = threadIdx.x;
  const int P = max(1, min(kScanThreads / C, 64));
  const int per = (T + P - 1) / P;
  const int col = tid % C;
  const int p = tid / C;
  const bool active = tid < P * C;
  const int t0 = active ? min(T, p * per) : T;
  const int t1 = active ? min(T, t0 + per) : T;
  int v[kSegRegs];
  int sum = 0;
  for (int b0 = t0; b0 < t1; b0 += kSegRegs) {
#pragma unroll
    for (int u = 0; u < kSegRegs; ++u) {
      const int t = b0 + u;
      v[u] = t < t1 ? data[(int64_t)t * C + col] : 0;
    }
#pragma unroll
    for (int u = 0; u < kSegRegs; ++u) sum += v[u];
  }
  if (active) seg[p * C + col] = sum;
  __syncthreads();
  if (tid < C) {
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int x = seg[q * C + tid];
      seg[q * C + tid] = run;
      run += x;
    }
    totals[tid] = run;
  }
  __syncthreads();
  if (active) {
    int run = seg[p * C + col];
    if (t1 - t0 <= kSegRegs) {  // the whole segment is still in registers
#pragma unroll
      for (int u = 0; u < kSegRegs; ++u) {
        const int t = t0 + u;
        if (t < t1) {
          data[(int64_t)t * C + col] = run;
          run += v[u];
        }
      }
    } else {
      for (int t = t0; t < t1; ++t) {
        const int x = data[(int64_t)t * C + col];
        data[(int64_t)t * C + col] = run;
        run += x;
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int32_t T, int32_t G, int32_t B, int32_t dedup, const int32_t* __restrict__ ebkt,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_bhist,
    const int32_t* __restrict__ tile_err, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ bucket_count,
    int32_t* __restrict__ bucket_offset, int32_t* __restrict__ status) {
  __shared__ int32_t seg[kScanThreads];
  __shared__ int32_t cnt_s[kMaxE];
  __shared__ unsigned char map_s[kMaxE];
  __shared__ OrderLds<kScanThreads> olds;
  __shared__ int32_t bsum_s[kMaxB];
  __shared__ int32_t btot_s[kMaxB];
  __shared__ int32_t err_s;
  __shared__ int32_t mapbad_s;

  const int tid = threadIdx.x;
  if (tid == 0) {
    err_s = kNoError;
    mapbad_s = kNoError;
  }
  if (tid < kMaxB) bsum_s[tid] = 0;

  // Issue the small loads first; they are consumed after the column scan has issued
  // its own, so all global reads of this kernel share one round trip.
  const int map_b = tid < G ? ebkt[tid] : 0;
  int terr = kNoError;
  for (int i = tid; i < T; i += kScanThreads) terr = min(terr, tile_err[i]);
  __syncthreads();

  // per-expert counts: column scan of the tile histograms
  column_exclusive_scan(tile_hist, T, G, cnt_s, seg);

  // status: bad map entries first, then the first bad expert id
  if (terr != kNoError) atomicMin(&err_s, terr);
  if (tid < G) {
    const bool bad = map_b < 0 || map_b >= B;
    if (bad) atomicMin(&mapbad_s, tid);
    map_s[tid] = bad ? kBadBucket : (unsigned char)map_b;
    atomicAdd(&bsum_s[bad ? B - 1 : map_b], cnt_s[tid]);
  }
  __syncthreads();
  expert_order_offsets<kScanThreads>(olds, map_s, cnt_s, G, B, expert_offset);
  if (tid < G) expert_count[tid] = cnt_s[tid];

  // buckets
  if (dedup) {
    column_exclusive_scan(tile_bhist, T, B, btot_s, seg);
  } else {
    if (tid < B) btot_s[tid] = bsum_s[tid];
    __syncthreads();
  }
  if (tid < 64) {  // bucket counts and their exclusive scan, one wave
    const int v = tid < B ? btot_s[tid] : 0;
    const int incl = wave_inclusive_sum(v);
    if (tid < B) {
      bucket_count[tid] = v;
      bucket_offset[tid] = incl - v;
    }
    if (tid == 63) bucket_offset[B] = incl;
    if (tid == 0)
      status[0] = mapbad_s != kNoError ? -(mapbad_s + 1) : (err_s != kNoError ? err_s + 1 : 0);
  }
}

__global__ __launch_bounds__(256) void layout_finalize_kernel(
    const int32_t* __restrict__ idx, int64_t Mk, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    const int32_t* __restrict__ tile_hist, const int32_t* __restrict__ tile_bhist,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ bucket_offset,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_row,
    int32_t* __restrict__ send_token, int64_t send_cap) {
  const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= Mk) return;
  const int e = idx[f];
  const int t = (int)(f / k);
  const int tile = t / kTileTokens;
  const int loc = slot[f];
  if (e < 0 || e >= G || loc < 0) {
    slot[f] = -1;
    send_row[f] = -1;
    return;
  }
  const int s = expert_offset[e] + tile_hist[(int64_t)tile * G + e] + loc;
  slot[f] = s;
  if (!dedup) {
    send_row[f] = s;
    if (s >= 0 && s < send_cap) send_token[s] = t;
    return;
  }
  const int b = ebkt[e];
  const int dl = send_row[f];
  if (b < 0 || b >= B || dl < 0) {
    send_row[f] = -1;
    return;
  }
  const int r = bucket_offset[b] + tile_bhist[(int64_t)tile * B + b] + dl;
  send_row[f] = r;
  if (r >= 0 && r < send_cap) send_token[r] = t;
}

// ------------------------------------------------- 2..kOnePassMaxTiles tiles, one launch
// Every tile ranks its entries as layout_tile_kernel does and publishes one row of
// counts (expert counts, then bucket counts in dedup mode) and an error word in the
// region of this call, every value stored as value + 1 with agent-scope stores (sc1:
// written through to the point where every XCD's loads see them).  The region is zero
// before the call, so each word is its own flag: a tile reads all T rows with
// agent-scope loads, polling (bounded) until every word it needs is nonzero, and sums
// each column itself -- over the rows before it (its prefix) and over all rows (the
// totals).  There is no arrival counter, no serial column scan and no second launch;
// each tile orders the experts (identically) and writes its slots and send rows from
// the ranks it still holds in registers.  Every tile is resident at once (T <=
// kOnePassMaxTiles is far below one workgroup per CU), so the polls end as soon as the
// slowest tile has published; a poll that expires anyway (about a second) makes the
// status MOE_LAYOUT_STATUS_WAIT_EXPIRED, and every store stays in bounds regardless.
//
// Two regions alternate between calls: while a call publishes in one, its tiles clear
// the rows the previous one-launch call published in the other (that call has ended,
// so nobody reads them any more), each tile a share.  The last tile to leave (header
// word 0) writes the status word, flips the region and records this call's rows for
// the next call to clear.  The regions sit at fixed offsets, so calls of any size may
// share a workspace; it must be zero-filled before its first use.
constexpr int kSpinLimit = 1 << 20;  // polls (about 1 us each) before giving up
constexpr int kWideTileTokens = 1024;  // tokens per tile above kOnePassMaxTiles 256-token tiles
constexpr int kSmallTileTokens = 128;  // tokens per tile where 128-token tiles fit one launch
constexpr int kTinyTileTokens = 64;    // tokens per tile where up to 32 such tiles cover M
constexpr int kHalfWideTileTokens = 512;  // tokens per tile where 64 such tiles cover M
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer resource: no format, no swizzle
constexpr int kSc1 = 16;  // cache policy sc1: coherent across the XCDs' L2s

__device__ __forceinline__ bool all_published(u32x4 v) {
  return v[0] != 0u && v[1] != 0u && v[2] != 0u && v[3] != 0u;
}

// pre[c] += sum over rows t < tile and tot[c] += sum over all T rows of the Cp
// columns (Cp % 4 == 0) of the row-major rows[T][Cp] (values stored + 1), into LDS
// (zero on entry), by an NT-thread workgroup whose threads [T0, NT) read: 16-byte
// quads, PB at a time, reloading those not yet fully published.  The first attempt
// uses plain loads: in one launch a word of the region is either still zero (cleared
// by the previous call, and no stale line survives the launch boundary) or holds its
// final value, so a cached copy can only show a quad as unpublished, never a wrong
// count.  Reloads use agent-scope loads, which do not hit a stale cached line.  (Threads below T0 have stores in flight; a wave's loads complete only
// after its earlier stores, so they take no part in the reads.)  When a row has fewer
// quads than there are reading threads, `stride` groups of them take interleaved
// rows; every reader adds its partial sums with LDS adds.  Ends after a barrier;
// returns false if some quad was still unpublished when the poll gave up.
template <int NT, int PB, int T0>
__device__ __forceinline__ bool poll_column_sums(const int32_t* rows, int T, int Cp, int tile,
                                                 int32_t* pre, int32_t* tot) {
  constexpr int NP = NT - T0;  // reading threads
  const int tid = threadIdx.x - T0;
  const int Q = Cp / 4;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)rows, (short)0, T * Cp * 4, kRawBufferWord3);
  const bool wide = Q >= NP;  // every reading thread owns whole columns
  const int stride = wide ? 1 : NP / Q;
  bool done = true;
  for (int q0 = 0; q0 < Q; q0 += NP) {
    const int q = wide ? q0 + tid : (tid >= 0 ? tid % Q : 0);
    const int g = wide ? 0 : (tid >= 0 ? tid / Q : 0);
    const bool active = tid >= 0 && (wide ? q < Q : g < stride);
    u32x4 p = {0, 0, 0, 0}, a = {0, 0, 0, 0};
    const int n = active ? (T - g + stride - 1) / stride : 0;  // rows g, g + stride, ...
    for (int u0 = 0; u0 < n; u0 += PB) {
      unsigned pend = 0;
#pragma unroll
      for (int i = 0; i < PB; ++i) pend |= (u0 + i < n ? 1u : 0u) << i;
      for (int spin = 0; pend != 0u && spin < kSpinLimit; ++spin) {
        u32x4 v[PB];
        if (spin == 0) {
#pragma unroll
          for (int i = 0; i < PB; ++i) {
            v[i] = u32x4{0, 0, 0, 0};
            if ((pend >> i) & 1u)
              v[i] = __builtin_bit_cast(
                  u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rs, ((g + (u0 + i) * stride) * Cp + 4 * q) * 4, 0, 0));
          }
        } else {
#pragma unroll
          for (int i = 0; i < PB; ++i) {
            v[i] = u32x4{0, 0, 0, 0};
            if ((pend >> i) & 1u)
              v[i] = __builtin_bit_cast(
                  u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rs, ((g + (u0 + i) * stride) * Cp + 4 * q) * 4, 0, kSc1));
          }
        }
#pragma unroll
        for (int i = 0; i < PB; ++i) {
          if (((pend >> i) & 1u) && all_published(v[i])) {
            const u32x4 c = v[i] - 1u;
            a += c;
            if (g + (u0 + i) * stride < tile) p += c;
            pend &= ~(1u << i);
          }
        }
        if (pend != 0u) __builtin_amdgcn_s_sleep(1);
      }
      done = done && pend == 0u;
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        atomicAdd(pre + 4 * q + i, (int)p[i]);
        atomicAdd(tot + 4 * q + i, (int)a[i]);
      }
    }
  }
  __syncthreads();
  return done;
}

// Waves of the one-launch layout's workgroup.  Tiles of 256 tokens: 16 (two 64-entry
// chunks per wave at k = 8) when k > 2, else 4 * KC so that every wave holds at least
// one chunk; tiles of 128 tokens (KC >= 8 only): 16, one chunk per wave at k = 8; tiles
// of 64 tokens (KC >= 8 only): 8, one chunk per wave at k = 8.  Tiles of 1024 tokens (more than 64 tiles of 256): 16, one per 64 tokens,
// KC chunks each.
template <int KC, int TT = kTileTokens>
constexpr int onepass_waves() {
  return TT > kTileTokens ? TT / 64 : TT == 64 ? 8 : (KC >= 4 ? 16 : 4 * KC);
}

template <int KC, int TT>
__global__ __launch_bounds__((onepass_waves<KC, TT>() * 64)) void layout_onepass_kernel(
    const int32_t* __restrict__ idx, int32_t M, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ bucket_count, int32_t* __restrict__ bucket_offset,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_row,
    int32_t* __restrict__ send_token, int32_t* __restrict__ status, uint32_t* header,
    int32_t* region0, int32_t* region1) {
  constexpr int NW = onepass_waves<KC, TT>();
  constexpr int NT = NW * 64;
  constexpr int NC = (TT / 64) * KC / NW;  // chunks per wave
  static_assert(NC >= 1 && NC * NW == (TT / 64) * KC, "the waves cover the tile");
  __shared__ TileLds<KC, NW, TT> lds;
  __shared__ OrderLds<NT> olds;
  // a tile's row: expert counts [0, G), bucket counts [Gp, Gp + B) (dedup), zero pads
  __shared__ int32_t pre_s[kRegionCols];
  __shared__ int32_t tot_s[kRegionCols];
  __shared__ int32_t off_s[kMaxE];
  __shared__ int32_t inv_s[kMaxE];       // the expert at each (bucket, id) position
  __shared__ int32_t scan_s[kMaxE + 1];  // exclusive scan of the counts in that order
  __shared__ int32_t base_s[kMaxB + 1];  // first position of each bucket
  __shared__ int32_t boff_s[kMaxB + 1];
  __shared__ int32_t err_s;
  __shared__ int32_t mapbad_s;
  __shared__ int32_t sorted_map_s;

  const int T = (int)gridDim.x;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int64_t Mk = (int64_t)M * k;
  const int Gp = (G + 3) & ~3;
  const int Cp = dedup ? Gp + ((B + 3) & ~3) : Gp;  // row pitch of this call, in ints
  // which region this call publishes in, and what the previous call left in the other.
  // Plain loads: these words were last written by an earlier launch (visible to this
  // one like any kernel's output to the next), and this launch rewrites them only
  // after every tile has published, i.e. after every tile has read them.  (Device-
  // coherent loads would take the slow path, and the in-order completion of vector
  // memory operations would make the topk_idx loads behind them wait as long.)
  const uint32_t parity = header[1] & 1u;
  const int prev_T = (int)header[2];
  const int prev_Cp = (int)header[3];
  int32_t* const rows = parity ? region1 : region0;
  int32_t* const old_rows = parity ? region0 : region1;
  if (tid == 0) {
    err_s = kNoError;
    mapbad_s = kNoError;
  }
  for (int c = tid; c < Cp; c += NT) pre_s[c] = 0;

  // The counts go out first: per-tile histograms are cheap (LDS adds), while the
  // stable ranks (ballot matching) are the tile's longest compute.  So the ranks, and
  // the (bucket, id) order of the experts, run while the other tiles' counts travel.
  int ec[NC];
  bool ok[NC];
  tile_load_ids<KC, NC, NW, TT>(lds, idx, M, k, ebkt, G, B, tile, dedup != 0, ec, ok);
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (ok[c]) atomicAdd(pre_s + ec[c], 1);
  if (dedup) {
    __syncthreads();  // lds.ids_s complete
    tile_bucket_counts<KC, NW, TT>(lds, M, k, tile, pre_s + Gp);
  }
  __syncthreads();

  // Wave 0 publishes (value + 1; nobody waits for these stores, readers poll the
  // words) and then clears this tile's share of the previous call's rows.
  if (w == 0) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rows + (int64_t)tile * Cp), (short)0, Cp * 4, kRawBufferWord3);
    for (int q = lane; q < Cp / 4; q += 64) {
      const u32x4 v = {(uint32_t)pre_s[4 * q] + 1u, (uint32_t)pre_s[4 * q + 1] + 1u,
                       (uint32_t)pre_s[4 * q + 2] + 1u, (uint32_t)pre_s[4 * q + 3] + 1u};
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, q * 16, 0, kSc1);
    }
    if (lane == 0)
      __hip_atomic_store(rows + kRegionErrOffset + tile, (int32_t)((uint32_t)lds.err_s + 1u),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t words = (int64_t)prev_T * prev_Cp;  // a multiple of 4
    const int64_t q_lo = words / 4 * tile / T, q_hi = words / 4 * (tile + 1) / T;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)old_rows, (short)0, (int)(words * 4), kRawBufferWord3);
    for (int64_t q = q_lo + lane; q < q_hi; q += 64)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, ro, (int)(q * 16), 0, kSc1);
    if (tile == 0 && lane < prev_T)
      __hip_atomic_store(old_rows + kRegionErrOffset + lane, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  if (w == NW - 1) {  // is the map in range and nondecreasing in the expert id?
    bool good = true;
#pragma unroll 4
    for (int e = lane; e < G; e += 64) {
      const int m = lds.map_s[e];
      const int m1 = lds.map_s[e + 1 < G ? e + 1 : e];
      good &= (m != kBadBucket) & (m <= m1);
    }
    const bool sorted = wave_ballot(!good) == 0;
    if (lane == 0) sorted_map_s = sorted;  // read after the barriers below
  }

  // While the counts travel (a store and a load across the chip take longer than
  // the work below): this tile's ranks (the first barrier also orders the
  // publication's reads of pre_s before it is overwritten below).  With dedup, the
  // tokens' bucket ranks run in the same phases, between the same barriers, instead
  // of after them ...
  int rc[NC];
  int eb[KC], dl[KC];
  rank_phase_match<KC, NC, NW, TT>(lds, G, ok, ec, rc);
  if (dedup) dedup_phase_ballots<KC, NW, TT>(lds, M, k, B, tile, eb);
  __syncthreads();
  rank_phase_prefix<KC, NW, TT>(lds, G, nullptr);
  if (dedup) dedup_phase_prefix<KC, NW, TT>(lds, B, nullptr);
  __syncthreads();
  rank_phase_finish<KC, NC, NW, TT>(lds, ec, rc);
  if (dedup) dedup_phase_finish<KC, NW, TT>(lds, eb, dl);
  // ... and the experts' (bucket, id) order: id order for a contiguous map, where the
  // buckets (map[e-1], map[e]] start at expert e; else ranked by bucket
  if (sorted_map_s) {
    for (int e = tid; e < G; e += NT) {
      const int b1 = lds.map_s[e];
      for (int b = e == 0 ? 0 : lds.map_s[e - 1] + 1; b <= b1; ++b) base_s[b] = e;
      if (e == G - 1)
        for (int b = b1 + 1; b <= B; ++b) base_s[b] = G;
    }
  } else {
    for (int e = tid; e < G; e += NT)
      if (lds.map_s[e] == kBadBucket) atomicMin(&mapbad_s, e);
    constexpr int CH = order_chunks<NT>();
    const int per = ((G + NW - 1) / NW + 63) / 64 * 64;
    int pos[CH];
    expert_sigma_positions<NT>(olds, lds.map_s, G, B, pos);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (pos[c] >= 0) inv_s[pos[c]] = w * per + c * 64 + lane;
    if (tid <= B) base_s[tid] = tid < B ? olds.base[tid] : G;
  }
  for (int c = tid; c < Cp; c += NT) {  // the published row is no longer read
    pre_s[c] = 0;
    tot_s[c] = 0;
  }
  __syncthreads();

  // column sums over all tiles' rows: this tile's prefix and the totals.  The error
  // words are polled too.
  bool done = true;
  if (w == 1 && lane < T) {
    uint32_t e = 0;
    for (int spin = 0; spin < kSpinLimit; ++spin) {
      e = (uint32_t)__hip_atomic_load(rows + kRegionErrOffset + lane, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      if (e != 0u) break;
      __builtin_amdgcn_s_sleep(1);
    }
    done = e != 0u;
    if (done && (int)(e - 1u) != kNoError) atomicMin(&err_s, (int)(e - 1u));
  }
  constexpr int PB = (KC >= 16 || TT > kTileTokens) ? 4 : 8;  // quads polled at once (registers)
  done = poll_column_sums<NT, PB, 64>(rows, T, Cp, tile, pre_s, tot_s) && done;
  const bool expired = __syncthreads_or(!done);
  const int32_t* bpre_s = pre_s + Gp;  // dedup: this tile's prefix of each bucket

  // leave: this tile's reads of the region are complete.  The count of tiles whose
  // poll expired rides in the high half.  The returned count is looked at only at the
  // end, so the round trip overlaps the offsets and the slots (the library builds this
  // file without the atomic optimizer, which would wait for it here).
  const uint32_t mine = 1u + (expired ? 0x10000u : 0u);
  uint32_t before = 0;
  if (tid == 0)
    before = __hip_atomic_fetch_add(header, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // expert offsets: wave 0 scans the totals in (bucket, id) order, 8 positions per
  // lane and round (all LDS reads of a round in flight together); bucket offsets are
  // the scan at each bucket's first position (dedup: wave 1 scans the bucket totals,
  // columns Gp.. of the sums)
  if (w == 0) {
    constexpr int kPer = 8;
    const bool sorted = sorted_map_s;
    int carry = 0;
    for (int r0 = 0; r0 < G; r0 += 64 * kPer) {
      int ex[kPer], v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = r0 + lane * kPer + u;
        const int ic = i < G ? i : G - 1;
        ex[u] = sorted ? ic : inv_s[ic];
      }
      int sum = 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        v[u] = r0 + lane * kPer + u < G ? tot_s[ex[u]] : 0;
        sum += v[u];
      }
      const int incl = wave_inclusive_sum(sum);
      int run = carry + incl - sum;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = r0 + lane * kPer + u;
        if (i < G) {
          off_s[ex[u]] = run;
          scan_s[i] = run;
        }
        run += v[u];
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) scan_s[G] = carry;
  }
  if (dedup) small_exclusive_scan(tot_s + Gp, boff_s, B, true, 1);
  __syncthreads();
  if (!dedup && tid <= B) boff_s[tid] = scan_s[base_s[tid]];
  __syncthreads();

  if (tile == 0) {
    for (int e = tid; e < G; e += NT) {
      expert_count[e] = tot_s[e];
      expert_offset[e] = off_s[e];
    }
    if (tid < B) bucket_count[tid] = boff_s[tid + 1] - boff_s[tid];
    if (tid <= B) bucket_offset[tid] = boff_s[tid];
  }

  const int64_t wbase = wave_first_entry<NC, TT>(tile, k, w);
  const int64_t tend = tile_end_entry<TT>(M, k, tile);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (f < tend) {
      const int s = ec[c] >= 0 ? off_s[ec[c]] + pre_s[ec[c]] + rc[c] : -1;
      slot[f] = s;
      if (!dedup) {
        send_row[f] = s;
        if (s >= 0 && s < Mk) send_token[s] = (int)(f / k);
      }
    }
  }
  if (dedup) {
    // send rows are found in the token view; they go through LDS (the tile's id store,
    // no longer read) so that they are stored in flat order, like the slots
    if (w < TT / 64) {
      const int64_t t = (int64_t)tile * TT + (int64_t)w * 64 + lane;
      const int64_t cap = (int64_t)M * (k < B ? k : B);
      if (t < M) {
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          if (j < k) {
            const int r = eb[j] != kBadBucket ? boff_s[eb[j]] + bpre_s[eb[j]] + dl[j] : -1;
            lds.ids_s[(w * 64 + lane) * k + j] = r;
            if (r >= 0 && r < cap) send_token[r] = (int)t;
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t f = wbase + (int64_t)c * 64 + lane;
      if (f < tend) send_row[f] = lds.ids_s[w * 64 * NC + c * 64 + lane];
    }
  }

  // the last tile to leave writes the status and hands the region to the next call
  const uint32_t now = before + mine;
  if (tid == 0 && (now & 0xFFFFu) == (uint32_t)T) {
    status[0] = (now >> 16) ? MOE_LAYOUT_STATUS_WAIT_EXPIRED
                : mapbad_s != kNoError ? -(mapbad_s + 1)
                : (err_s != kNoError ? err_s + 1 : 0);
    __hip_atomic_store(header + 1, parity ^ 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(header + 2, (uint32_t)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(header + 3, (uint32_t)Cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(header, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Chunks of 64 entries per wave that cover one tile of `entries` entries with all
// four waves (rounded up to a power of two by the callers' instantiations).
inline int chunks_per_wave(int64_t entries) {
  return (int)((entries + kTileThreads - 1) / kTileThreads);
}

template <int KC>
void launch_tiles(const int32_t* topk_idx, int64_t M, int32_t k, const int32_t* expert_bucket,
                  int32_t G, int32_t B, int32_t dedup, int32_t* expert_count,
                  int32_t* expert_offset, int32_t* bucket_count, int32_t* bucket_offset,
                  int32_t* slot, int32_t* send_row, int32_t* send_token, int32_t* status,
                  const LayoutWorkspace& ws, hipStream_t stream) {
  const int T = (int)layout_tiles(M);
  const int64_t Mk = M * k;
  if (T == 1) {
#define MOEDL_SINGLE(NC)                                                                        \
  hipLaunchKernelGGL((layout_single_kernel<KC, NC>), dim3(1), dim3(kTileThreads), 0, stream,        \
                     topk_idx, (int32_t)M, k, expert_bucket, G, B, dedup, expert_count,            \
                     expert_offset, bucket_count, bucket_offset, slot, send_row, send_token, status)
    const int nc = chunks_per_wave(Mk);
    if (nc <= 1 || KC == 1) MOEDL_SINGLE(1);
    else if (nc <= 2 || KC == 2) MOEDL_SINGLE(KC >= 2 ? 2 : 1);
    else if (nc <= 4 || KC == 4) MOEDL_SINGLE(KC >= 4 ? 4 : 1);
    else if (nc <= 8 || KC == 8) MOEDL_SINGLE(KC >= 8 ? 8 : 1);
    else MOEDL_SINGLE(KC >= 16 ? 16 : 1);
#undef MOEDL_SINGLE
    return;
  }
  // Smaller tiles where at most kOnePassMaxTiles of them cover M (k >= 5, so that every
  // wave still holds one 64-entry chunk): less ranking work per workgroup for more
  // published rows read.  Measured on MI355X (graph replay, outputs identical), 256 /
  // 128 / 64-token tiles: M = 1,000 8.5 / 7.6 / 7.1 us, 2,048 8.6 / 7.8 / 7.4, 4,096 9.0 /
  // 8.1 / 8.8 (64 rows read: the 64-token tiles lose there), 8,192 9.3 / 8.6; dedup
  // layouts likewise.  So 64-token tiles up to 32 of them, 128-token tiles up to 64.
  if constexpr (KC >= 8) {
    const int64_t T64 = (M + kTinyTileTokens - 1) / kTinyTileTokens;
    if (T64 >= 2 && T64 <= kOnePassMaxTiles / 2) {
      hipLaunchKernelGGL((layout_onepass_kernel<KC, kTinyTileTokens>), dim3((unsigned)T64),
                         dim3(onepass_waves<KC, kTinyTileTokens>() * 64), 0, stream, topk_idx,
                         (int32_t)M, k, expert_bucket, G, B, dedup, expert_count, expert_offset,
                         bucket_count, bucket_offset, slot, send_row, send_token, status,
                         ws.header, ws.region[0], ws.region[1]);
      return;
    }
    const int64_t T128 = (M + kSmallTileTokens - 1) / kSmallTileTokens;
    if (T128 >= 3 && T128 <= kOnePassMaxTiles) {
      hipLaunchKernelGGL((layout_onepass_kernel<KC, kSmallTileTokens>), dim3((unsigned)T128),
                         dim3(onepass_waves<KC, kSmallTileTokens>() * 64), 0, stream, topk_idx,
                         (int32_t)M, k, expert_bucket, G, B, dedup, expert_count, expert_offset,
                         bucket_count, bucket_offset, slot, send_row, send_token, status,
                         ws.header, ws.region[0], ws.region[1]);
      return;
    }
  }
  if (T >= 2 && T <= kOnePassMaxTiles) {  // (M = 0: no tiles, the scan kernel writes zeros)
    hipLaunchKernelGGL((layout_onepass_kernel<KC, kTileTokens>), dim3(T),
                       dim3(onepass_waves<KC, kTileTokens>() * 64), 0, stream, topk_idx,
                       (int32_t)M, k, expert_bucket, G, B, dedup, expert_count, expert_offset,
                       bucket_count, bucket_offset, slot, send_row, send_token, status,
                       ws.header, ws.region[0], ws.region[1]);
    return;
  }
  // up to 64 tiles of 512 tokens (M <= 32,768), else of 1024 tokens (M <= 65,536), k <= 8:
  // the same single launch with more tokens per workgroup (k = 16 would not fit the
  // ids of a 1024-token tile in LDS).  Measured on MI355X (graph replay, outputs
  // identical), 1024- against 512-token tiles: M = 16,385 15.9 -> 11.9 us, 20,000 16.1
  // -> 12.5, 32,768 16.4 -> 13.9 (Zipf 15.5 -> 13.6); dedup layouts 3-5 us faster.
  const int64_t T4 = (M + kWideTileTokens - 1) / kWideTileTokens;
  if constexpr (KC <= 8) {
    const int64_t T2 = (M + kHalfWideTileTokens - 1) / kHalfWideTileTokens;
    if (T2 >= 2 && T2 <= kOnePassMaxTiles) {
      hipLaunchKernelGGL((layout_onepass_kernel<KC, kHalfWideTileTokens>), dim3((unsigned)T2),
                         dim3(onepass_waves<KC, kHalfWideTileTokens>() * 64), 0, stream,
                         topk_idx, (int32_t)M, k, expert_bucket, G, B, dedup, expert_count,
                         expert_offset, bucket_count, bucket_offset, slot, send_row,
                         send_token, status, ws.header, ws.region[0], ws.region[1]);
      return;
    }
    if (T4 >= 2 && T4 <= kOnePassMaxTiles) {
      hipLaunchKernelGGL((layout_onepass_kernel<KC, kWideTileTokens>), dim3((unsigned)T4),
                         dim3(onepass_waves<KC, kWideTileTokens>() * 64), 0, stream, topk_idx,
                         (int32_t)M, k, expert_bucket, G, B, dedup, expert_count, expert_offset,
                         bucket_count, bucket_offset, slot, send_row, send_token, status,
                         ws.header, ws.region[0], ws.region[1]);
      return;
    }
  }
  if (T > 1) {
    hipLaunchKernelGGL(layout_tile_kernel<KC>, dim3(T), dim3(kTileThreads), 0, stream, topk_idx,
                       (int32_t)M, k, expert_bucket, G, B, dedup, slot, send_row, ws.tile_hist,
                       ws.tile_bhist, ws.tile_err);
  }
  hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, T, G, B, dedup,
                     expert_bucket, ws.tile_hist, ws.tile_bhist, ws.tile_err, expert_count,
                     expert_offset, bucket_count, bucket_offset, status);
  if (Mk > 0) {
    const int64_t blocks = (Mk + 255) / 256;
    hipLaunchKernelGGL(layout_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       topk_idx, Mk, k, expert_bucket, G, B, dedup, ws.tile_hist,
                       ws.tile_bhist, expert_offset, bucket_offset, slot, send_row, send_token,
                       dedup ? M * (int64_t)(k < B ? k : B) : Mk);
  }
}

template <int KC>
hipError_t launch_fused(const int32_t* topk_idx, int64_t M, int32_t k, const int32_t* expert_bucket,
                        int32_t G, int32_t B, int32_t dedup, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* bucket_count, int32_t* bucket_offset,
                        int32_t* slot, int32_t* send_row, int32_t* send_token, int32_t* status,
                        const void* x, int64_t row_bytes, const float* x_scale,
                        int32_t scale_cols, void* out, float* out_scale, int64_t out_rows,
                        hipStream_t stream) {
  const int32_t row_vecs = (int32_t)(row_bytes / 16);
  const bool item1k = dedup == 0 && k >= 4;
  const int32_t piece_vecs = item1k ? kFusedFlatPieceVecs : kFusedPieceVecs;
  const int32_t pieces = (row_vecs + piece_vecs - 1) / piece_vecs;
  const int64_t items = M * pieces;
  const unsigned grid = (unsigned)(items < 1 ? 1 : (items < kFusedMaxBlocks ? items : kFusedMaxBlocks));
  const int32_t* idx = M > 0 ? topk_idx : expert_bucket;  // read at index 0 only
#define MOEDL_FUSED_AS(NT, NC, ITEM1K)                                                          \
  hipLaunchKernelGGL((layout_dispatch_small_kernel<KC, NT, NC, ITEM1K>), dim3(grid),               \
                     dim3(kTileThreads), 0, stream, idx, (int32_t)M, k, expert_bucket, G, B, dedup, \
                     expert_count, expert_offset, bucket_count, bucket_offset, slot, send_row,     \
                     send_token, status, (const u32x4*)x, row_vecs, pieces, x_scale, scale_cols,   \
                     (u32x4*)out, out_scale, out_rows)
  // (k >= 4 implies KC >= 4: the 1 KiB item shape is compiled only there)
#define MOEDL_FUSED(NT, NC)                                     \
  do {                                                          \
    if constexpr (KC >= 4) {                                    \
      if (item1k) {                                             \
        MOEDL_FUSED_AS(NT, NC, true);                           \
        break;                                                  \
      }                                                         \
    }                                                           \
    MOEDL_FUSED_AS(NT, NC, false);                              \
  } while (0)
  if (M > kTileTokens) {
    MOEDL_FUSED(2, KC);
  } else {
    const int nc = chunks_per_wave(M * k);
    if (nc <= 1 || KC == 1) MOEDL_FUSED(1, 1);
    else if (nc <= 2 || KC == 2) MOEDL_FUSED(1, KC >= 2 ? 2 : 1);
    else if (nc <= 4 || KC == 4) MOEDL_FUSED(1, KC >= 4 ? 4 : 1);
    else if (nc <= 8 || KC == 8) MOEDL_FUSED(1, KC >= 8 ? 8 : 1);
    else MOEDL_FUSED(1, KC >= 16 ? 16 : 1);
  }
#undef MOEDL_FUSED
#undef MOEDL_FUSED_AS
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// [sync words | tile_hist | tile_bhist | tile_err], each part 256-byte aligned.
// [header | region 0 | region 1 | tile_hist | tile_bhist | tile_err], each part
// 256-byte aligned.  The regions (one-launch layout) sit at fixed offsets whatever the
// sizes; the per-tile arrays of the three-launch layout follow only when it is used.
size_t layout_workspace_bytes(int64_t M, int32_t G, int32_t B) {
  const size_t T = (size_t)layout_tiles(M);
  size_t bytes = 256 + 2 * kRegionBytes;
  if (T > (size_t)kOnePassMaxTiles || T == 0)
    bytes += align256(T * G * 4) + align256(T * B * 4) + align256(T * 4);
  return bytes;
}

LayoutWorkspace carve_layout_workspace(void* base, int64_t M, int32_t G, int32_t B) {
  const size_t T = (size_t)layout_tiles(M);
  char* p = (char*)base;
  LayoutWorkspace ws;
  ws.header = (uint32_t*)p;
  p += 256;
  ws.region[0] = (int32_t*)p;
  p += kRegionBytes;
  ws.region[1] = (int32_t*)p;
  p += kRegionBytes;
  ws.tile_hist = (int32_t*)p;
  p += align256(T * G * 4);
  ws.tile_bhist = (int32_t*)p;
  p += align256(T * B * 4);
  ws.tile_err = (int32_t*)p;
  return ws;
}

hipError_t launch_layout(const int32_t* topk_idx, int64_t M, int32_t k,
                         const int32_t* expert_bucket, int32_t G, int32_t B, int32_t dedup,
                         int32_t* expert_count, int32_t* expert_offset,
                         int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                         int32_t* send_row, int32_t* send_token, int32_t* status,
                         const LayoutWorkspace& ws, hipStream_t stream) {
#define MOEDL_ARGS                                                                          \
  topk_idx, M, k, expert_bucket, G, B, dedup, expert_count, expert_offset, bucket_count,    \
      bucket_offset, slot, send_row, send_token, status, ws, stream
  if (k <= 1) launch_tiles<1>(MOEDL_ARGS);
  else if (k <= 2) launch_tiles<2>(MOEDL_ARGS);
  else if (k <= 4) launch_tiles<4>(MOEDL_ARGS);
  else if (k <= 8) launch_tiles<8>(MOEDL_ARGS);
  else launch_tiles<16>(MOEDL_ARGS);
#undef MOEDL_ARGS
  return hipGetLastError();
}

}  // namespace moedl

namespace moedl {

hipError_t launch_layout_dispatch(const int32_t* topk_idx, int64_t M, int32_t k,
                                  const int32_t* expert_bucket, int32_t G, int32_t B,
                                  int32_t dedup, int32_t* expert_count, int32_t* expert_offset,
                                  int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot,
                                  int32_t* send_row, int32_t* send_token, int32_t* status,
                                  const void* x, int64_t row_bytes, const float* x_scale,
                                  int32_t scale_cols, void* out, float* out_scale,
                                  int64_t out_rows, hipStream_t stream) {
  if (M > kFusedMaxTokens) return hipErrorInvalidValue;
#define MOEDL_ARGS                                                                          \
  topk_idx, M, k, expert_bucket, G, B, dedup, expert_count, expert_offset, bucket_count,    \
      bucket_offset, slot, send_row, send_token, status, x, row_bytes, x_scale, scale_cols, \
      out, out_scale, out_rows, stream
  if (k <= 1) return launch_fused<1>(MOEDL_ARGS);
  if (k <= 2) return launch_fused<2>(MOEDL_ARGS);
  if (k <= 4) return launch_fused<4>(MOEDL_ARGS);
  if (k <= 8) return launch_fused<8>(MOEDL_ARGS);
  return launch_fused<16>(MOEDL_ARGS);
#undef MOEDL_ARGS
}

}  // namespace moedl
