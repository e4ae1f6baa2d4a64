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
//  - tile_expert_ranks: one 256-thread workgroup, 256 tokens.  Each wave64 holds NC
//    consecutive 64-entry chunks of the tile's (t, j) entries in flat order.  Entries
//    of a chunk that name the same expert are found with ceil(log2 G) ballots (lanes
//    agreeing on every bit of the id), the ballots of all chunks interleaved; per
//    chunk, one leader lane per distinct expert adds the chunk's count to the wave's
//    LDS counter with an atomic that returns the old value (a wave's LDS operations
//    complete in order, so it counts the earlier chunks), and the peers fetch it from
//    the leader.  No same-address LDS atomics under skew.  That value plus the lane's
//    rank among its peers (mbcnt) is the entry's stable rank in the wave; a cross-wave
//    prefix makes it the rank in the tile.
//  - tile_dedup_ranks: token view (lane = token).  Per-token bucket bitmask; one
//    ballot per bucket gives each token's rank among the tile's tokens sending there.
//  - expert_order_offsets: experts ranked by (bucket, id) with the same ballot
//    matching (key = bucket), then a block-wide exclusive scan of the counts in that
//    order gives every expert's offset; a map whose bucket never decreases with the
//    id skips the ranking (id order).
//
// Kernels:
//  - M <= 256 tokens (one tile): layout_single_kernel does everything in LDS in one
//    launch.
//  - M <= 512 with the row scatter in the same launch: layout_dispatch_small_kernel
//    (every workgroup recomputes the layout in LDS, then copies its share of rows).
//  - otherwise three launches, no inter-workgroup waiting and no initialised state:
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
// of different chunks interleave instead of forming one long dependent chain.
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
        const bool set = (key[c] >> bit) & 1;
        const uint64_t bal = wave_ballot(set);
        peers[c] &= set ? bal : ~bal;
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
template <int NC>
__device__ __forceinline__ int64_t wave_first_entry(int tile, int32_t k, int w) {
  return (int64_t)tile * kTileTokens * k + (int64_t)w * 64 * NC;
}

// Exclusive scan of src[0, n) into dst by one thread; dst[n] = the total when
// with_total.  src may be dst.  For the short arrays here (n <= 64, usually a handful)
// the independent LDS reads issue together, which beats a shuffle-based wave scan.
// Callers put barriers around it.
__device__ __forceinline__ void serial_exclusive_scan(const int32_t* src, int32_t* dst, int n,
                                                      bool with_total) {
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < n; ++i) {
      const int v = src[i];
      dst[i] = run;
      run += v;
    }
    if (with_total) dst[n] = run;
  }
}

template <int KC>  // KC: k rounded up to a power of two (chunks per wave)
struct TileLds {
  unsigned char map_s[kMaxE];
  int32_t wcnt[kTileWaves][kMaxE];        // per-wave running counts, then prefixes
  int32_t ids_s[kTileTokens * KC];        // the tile's expert ids, flat order
  uint64_t wbal[kTileWaves][kMaxB];       // dedup: per-wave ballot of each bucket
  int32_t wbcnt[kTileWaves][kMaxB];       // dedup: per-wave counts, then prefixes
  int32_t err_s;                          // first bad flat index in the tile
};

// Last flat entry (exclusive) of a tile.
__device__ __forceinline__ int64_t tile_end_entry(int32_t M, int32_t k, int tile) {
  const int64_t Mk = (int64_t)M * k;
  const int64_t e = ((int64_t)tile + 1) * kTileTokens * k;
  return e < Mk ? e : Mk;
}

// Expert ranks of one 256-token tile, NC chunks per wave (see wave_first_entry).  On
// return (after a barrier): ec[c] / rc[c] hold the expert id (or kAbsent) and the rank
// inside the tile of flat entry wave_first_entry<NC>(tile, k, w) + c*64 + lane;
// totals[e] holds the tile's count of expert e (totals may be global or LDS);
// lds.ids_s holds the tile's ids (tile-local flat order) when keep_ids.
template <int KC, int NC>
__device__ __forceinline__ void tile_expert_ranks(TileLds<KC>& lds, const int32_t* __restrict__ idx,
                                                  int32_t M, int32_t k,
                                                  const int32_t* __restrict__ ebkt, int32_t G,
                                                  int32_t B, int tile, bool keep_ids,
                                                  int32_t* totals, int (&ec)[NC], int (&rc)[NC]) {
  static_assert(NC <= KC, "a wave's chunks must fit the tile's id store");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int nbits = bits_for(G);
  const int64_t wbase = wave_first_entry<NC>(tile, k, w);
  const int64_t tend = tile_end_entry(M, k, tile);
  const int local0 = w * 64 * NC;  // tile-local index of the wave's first entry

  // all global loads first: clamped, unconditional, so they are in flight together
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    const bool valid = f < tend;
    const int v = idx[valid ? f : 0];
    ec[c] = valid ? v : kAbsent;
  }
  for (int e = tid; e < G; e += kTileThreads) {
    const int b = ebkt[e];
    lds.map_s[e] = (b >= 0 && b < B) ? (unsigned char)b : kBadBucket;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) lds.wcnt[ww][e] = 0;
  }
  if (tid == 0) lds.err_s = kNoError;
  __syncthreads();

  int my_err = kNoError;
  bool ok[NC];
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
  uint64_t peers[NC];
  match_peers<NC, kExpertBits>(ok, ec, nbits, peers);
  stable_ranks<NC>(ok, ec, peers, lds.wcnt[w], rc);
  if (my_err != kNoError) atomicMin(&lds.err_s, my_err);
  __syncthreads();

  // cross-wave exclusive prefix per expert; the column total is the tile's count
  for (int e = tid; e < G; e += kTileThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) {
      const int v = lds.wcnt[ww][e];
      lds.wcnt[ww][e] = run;
      run += v;
    }
    totals[e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (ec[c] >= 0) rc[c] += lds.wcnt[w][ec[c]];
}

// Dedup ranks of one tile (token view).  Needs lds.ids_s from tile_expert_ranks.  On
// return (after a barrier): eb[j] is the bucket of token (lane)'s j-th entry or
// kBadBucket, dl[j] the token's rank among the tile's tokens that send to that
// bucket; btotals[b] the tile's distinct-token count of bucket b.
template <int KC>
__device__ __forceinline__ void tile_dedup_ranks(TileLds<KC>& lds, int32_t M, int32_t k, int32_t B, int tile,
                                 int32_t* btotals, int (&eb)[KC], int (&dl)[KC]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t t = (int64_t)tile * kTileTokens + (int64_t)w * 64 + lane;
  const bool tv = t < M;
  const int* my_ids = lds.ids_s + (w * 64 + lane) * k;
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
  if (lane < B) {
    lds.wbal[w][lane] = mine;
    lds.wbcnt[w][lane] = __builtin_popcountll(mine);
  }
  __syncthreads();
  if (tid < B) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) {
      const int v = lds.wbcnt[ww][tid];
      lds.wbcnt[ww][tid] = run;
      run += v;
    }
    btotals[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int b = eb[j] != kBadBucket ? eb[j] : 0;
    const int base = lds.wbcnt[w][b];
    const uint64_t bal = lds.wbal[w][b];
    dl[j] = eb[j] != kBadBucket ? base + __builtin_popcountll(bal & below) : -1;
  }
}

// Exclusive scan of one int per thread over an NT-thread workgroup.
template <int NT>
__device__ int block_exclusive_scan(int v, int32_t* wave_sums /* >= NT/64 */) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  serial_exclusive_scan(wave_sums, wave_sums, NT / 64, false);
  __syncthreads();
  const int r = wave_sums[w] + incl - v;
  __syncthreads();
  return r;
}

// LDS for expert_order_offsets.
template <int NT>
struct OrderLds {
  int32_t wbc[NT / 64][kMaxB];  // per-wave per-bucket expert counts, then prefixes
  int32_t base[kMaxB + 1];      // first sigma position of each bucket
  int32_t arr[kMaxE];           // counts in sigma order, then their exclusive scan
  int32_t wave_sums[NT / 64];
};

// Offsets of expert runs laid out in (bucket, id) order, from per-expert counts
// cnt[G] (LDS).  NT-thread workgroup; wave w handles a contiguous range of experts so
// the cross-wave prefix keeps id order.  A map whose bucket never decreases with the
// id takes a fast path (id order).  Writes offset[e] (global or LDS).
template <int NT>
__device__ void expert_order_offsets(OrderLds<NT>& lds, const unsigned char* map_s,
                                     const int32_t* cnt, int32_t G, int32_t B,
                                     int32_t* offset) {
  constexpr int NW = NT / 64;
  constexpr int CH = (kMaxE + NT - 1) / NT;  // chunks of 64 experts per wave, at most
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
  serial_exclusive_scan(lds.base, lds.base, B, false);
  __syncthreads();
  int pos[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = w * per + c * 64 + lane;
    pos[c] = -1;
    if (c * 64 < per && e < G) {
      pos[c] = lds.base[bk[c]] + lds.wbc[w][bk[c]] + rk[c];
      lds.arr[pos[c]] = cnt[e];
    }
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
  serial_exclusive_scan(btot_s, boff_s, B, true);
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
// rows inside the buffer.  The LDS row table holds each distinct row once (dedup repeats
// are marked absent while the layout is built), so the scatter reads a token's k rows
// together and needs no duplicate search.  Issuing the first batch of row loads before
// the layout work was measured slower (vector-load counters retire in order, so the
// layout's first wait on topk_idx also waited on the rows).  `idx` must be readable at
// index 0 even when M = 0.
constexpr int kFusedPieceVecs = kTileThreads;  // 16-byte vectors per work item
constexpr int kFusedBatch = 4;                  // work items loaded together
// Grid cap: two workgroups per CU, which fit at once for every instantiation (41-68 KiB
// of LDS each).  Every workgroup recomputes the layout before copying, so a grid that
// does not fit at once pays that again in a second wave, while fewer workgroups give
// the copies less parallelism.  Measured (graph replay, layout + dispatch + combine,
// N=7168, top-8, dedup off): cap 128 / 256 / 512 / 1024 -> 25.5 / 22.5 / 22.5 / 28.1 us
// at M=256, 45.8 / 36.9 / 36.2 / 46.1 us at M=512; dedup on alike.
constexpr int kFusedMaxBlocks = 512;

template <int KC, int NTILE, int NC>
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
  serial_exclusive_scan(btot_s, boff_s, B, true);
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
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
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
  const int32_t pieces = (row_vecs + kFusedPieceVecs - 1) / kFusedPieceVecs;
  const int64_t items = M * pieces;
  const unsigned grid = (unsigned)(items < 1 ? 1 : (items < kFusedMaxBlocks ? items : kFusedMaxBlocks));
  const int32_t* idx = M > 0 ? topk_idx : expert_bucket;  // read at index 0 only
#define MOEDL_FUSED(NT, NC)                                                                     \
  hipLaunchKernelGGL((layout_dispatch_small_kernel<KC, NT, NC>), dim3(grid), dim3(kTileThreads), 0, \
                     stream, idx, (int32_t)M, k, expert_bucket, G, B, dedup, expert_count,         \
                     expert_offset, bucket_count, bucket_offset, slot, send_row, send_token,      \
                     status, (const u32x4*)x, row_vecs, pieces, x_scale, scale_cols, (u32x4*)out, \
                     out_scale, out_rows)
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
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t layout_workspace_bytes(int64_t M, int32_t G, int32_t B) {
  const size_t T = (size_t)layout_tiles(M);
  return align256(T * G * 4) + align256(T * B * 4) + align256(T * 4) + 256;
}

LayoutWorkspace carve_layout_workspace(void* base, int64_t M, int32_t G, int32_t B) {
  const size_t T = (size_t)layout_tiles(M);
  char* p = (char*)base;
  LayoutWorkspace ws;
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
