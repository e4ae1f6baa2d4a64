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
//  - tile_expert_ranks: one 256-thread workgroup, 256 tokens.  Each wave64 walks its
//    64 tokens' k*64 (t, j) entries in flat order, 64 at a time.  Entries of one
//    64-entry chunk that name the same expert are found with ceil(log2 G) ballots
//    (lanes agreeing on every bit of the id); one leader lane per distinct expert
//    bumps the wave's LDS counter, so there are no same-address LDS atomics under
//    skew.  The lane's rank among its peers (mbcnt) plus the counter's old value is
//    the entry's stable rank in the wave; a cross-wave prefix makes it the rank in the
//    tile.
//  - tile_dedup_ranks: token view (lane = token).  Per-token bucket bitmask; one
//    ballot per bucket gives each token's rank among the tile's tokens sending there.
//  - expert_order_offsets: experts ranked by (bucket, id) with the same ballot
//    matching (key = bucket), then a block-wide exclusive scan of the counts in that
//    order gives every expert's offset.
//
// Kernels:
//  - M <= 256 tokens (one tile): layout_single_kernel does everything in LDS in one
//    launch.
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

__device__ __forceinline__ int bits_for(int n) {  // bits needed for values in [0, n)
  return n <= 1 ? 0 : 32 - __builtin_clz((unsigned)(n - 1));
}

// Lanes of the wave whose `key` equals the caller's, among lanes with `ok` set.
__device__ __forceinline__ uint64_t match_peers(bool ok, int key, int nbits) {
  uint64_t peers = wave_ballot(ok);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (key >> bit) & 1;
    const uint64_t bal = wave_ballot(ok && set);
    peers &= set ? bal : ~bal;
  }
  return peers;
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

// Expert ranks of one 256-token tile.  On return (after a barrier): ec[c] / rc[c]
// hold the expert id (or kAbsent) and the rank inside the tile of flat entry
// wbase + c*64 + lane; totals[e] holds the tile's count of expert e (totals may be
// global or LDS); lds.ids_s holds the tile's ids when keep_ids.
template <int KC>
__device__ void tile_expert_ranks(TileLds<KC>& lds, const int32_t* __restrict__ idx, int32_t M,
                                  int32_t k, const int32_t* __restrict__ ebkt, int32_t G,
                                  int32_t B, int tile, bool keep_ids, int32_t* totals,
                                  int (&ec)[KC], int (&rc)[KC]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int64_t Mk = (int64_t)M * k;
  const int nbits = bits_for(G);
  const int64_t wbase = ((int64_t)tile * kTileTokens + (int64_t)w * 64) * k;

  // all global loads first: clamped, unconditional, so they are in flight together
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    const bool valid = c < k && f < Mk;
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
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    int e = ec[c];
    if (e != kAbsent && (e < 0 || e >= G)) {
      my_err = min(my_err, (int)(wbase + c * 64 + lane));
      e = kAbsent;
    }
    if (keep_ids && c < k) lds.ids_s[w * 64 * k + c * 64 + lane] = e;
    const bool ok = e >= 0;
    const uint64_t peers = match_peers(ok, e, nbits);
    const int r = lanes_below(peers);
    int old = 0;
    if (ok) old = lds.wcnt[w][e];
    if (ok && r == 0) lds.wcnt[w][e] = old + __builtin_popcountll(peers);
    ec[c] = e;
    rc[c] = old + r;
  }
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
  for (int c = 0; c < KC; ++c)
    if (ec[c] >= 0) rc[c] += lds.wcnt[w][ec[c]];
}

// Dedup ranks of one tile (token view).  Needs lds.ids_s from tile_expert_ranks.  On
// return (after a barrier): eb[j] is the bucket of token (lane)'s j-th entry or
// kBadBucket, dl[j] the token's rank among the tile's tokens that send to that
// bucket; btotals[b] the tile's distinct-token count of bucket b.
template <int KC>
__device__ void tile_dedup_ranks(TileLds<KC>& lds, int32_t M, int32_t k, int32_t B, int tile,
                                 int32_t* btotals, int (&eb)[KC], int (&dl)[KC]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t t = (int64_t)tile * kTileTokens + (int64_t)w * 64 + lane;
  const bool tv = t < M;
  const int* my_ids = lds.ids_s + (w * 64 + lane) * k;
  uint64_t bmask = 0;
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    eb[j] = kBadBucket;
    if (j < k && tv) {
      const int e = my_ids[j];
      if (e >= 0) {
        eb[j] = lds.map_s[e];
        if (eb[j] != kBadBucket) bmask |= 1ull << eb[j];
      }
    }
  }
  for (int b = 0; b < B; ++b) {
    const uint64_t bal = wave_ballot(tv && ((bmask >> b) & 1ull));
    if (lane == 0) {
      lds.wbal[w][b] = bal;
      lds.wbcnt[w][b] = __builtin_popcountll(bal);
    }
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
    const int b = eb[j];
    dl[j] = b != kBadBucket ? lds.wbcnt[w][b] + __builtin_popcountll(lds.wbal[w][b] & below)
                            : -1;
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
  if (threadIdx.x == 0) {
    int run = 0;
    for (int q = 0; q < NT / 64; ++q) {
      const int s = wave_sums[q];
      wave_sums[q] = run;
      run += s;
    }
  }
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
// the cross-wave prefix keeps id order.  Writes offset[e] (global or LDS).
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
  for (int i = tid; i < NW * kMaxB; i += NT) lds.wbc[i / kMaxB][i % kMaxB] = 0;
  __syncthreads();

  const int nbits = bits_for(B);
  int rk[CH];
  int bk[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = w * per + c * 64 + lane;
    const bool ok = c * 64 < per && e < G;
    int b = ok ? (int)map_s[e] : 0;
    b = b < B ? b : B - 1;  // a bad map entry is reported by status; keep it in range
    const uint64_t peers = match_peers(ok, b, nbits);
    const int r = lanes_below(peers);
    int old = 0;
    if (ok) old = lds.wbc[w][b];
    if (ok && r == 0) lds.wbc[w][b] = old + __builtin_popcountll(peers);
    rk[c] = old + r;
    bk[c] = b;
  }
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
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < B; ++b) {
      const int v = lds.base[b];
      lds.base[b] = run;
      run += v;
    }
  }
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
template <int KC>
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

  int ec[KC], rc[KC];
  tile_expert_ranks<KC>(lds, idx, M, k, ebkt, G, B, 0, dedup != 0, cnt_s, ec, rc);
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
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < B; ++b) {
      boff_s[b] = run;
      run += btot_s[b];
    }
    boff_s[B] = run;
  }
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

  const int64_t wbase = (int64_t)w * 64 * k;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (c < k && f < Mk) {
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
  const int64_t Mk = (int64_t)M * k;
  int ec[KC], rc[KC];
  tile_expert_ranks<KC>(lds, idx, M, k, ebkt, G, B, tile, dedup != 0,
                        tile_hist + (int64_t)tile * G, ec, rc);
  const int64_t wbase = ((int64_t)tile * kTileTokens + (int64_t)w * 64) * k;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (c < k && f < Mk) slot_local[f] = ec[c] >= 0 ? rc[c] : -1;
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
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < B; ++b) {
      bucket_count[b] = btot_s[b];
      bucket_offset[b] = run;
      run += btot_s[b];
    }
    bucket_offset[B] = run;
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

template <int KC>
void launch_tiles(const int32_t* topk_idx, int64_t M, int32_t k, const int32_t* expert_bucket,
                  int32_t G, int32_t B, int32_t dedup, int32_t* expert_count,
                  int32_t* expert_offset, int32_t* bucket_count, int32_t* bucket_offset,
                  int32_t* slot, int32_t* send_row, int32_t* send_token, int32_t* status,
                  const LayoutWorkspace& ws, hipStream_t stream) {
  const int T = (int)layout_tiles(M);
  const int64_t Mk = M * k;
  if (T == 1) {
    hipLaunchKernelGGL(layout_single_kernel<KC>, dim3(1), dim3(kTileThreads), 0, stream, topk_idx,
                       (int32_t)M, k, expert_bucket, G, B, dedup, expert_count, expert_offset,
                       bucket_count, bucket_offset, slot, send_row, send_token, status);
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
