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
// Structure (three launches, no inter-workgroup waiting, no initialised state):
//  1. layout_tile_kernel: one workgroup per 256-token tile.  Each wave64 walks its
//     64 tokens' k*64 (t, j) entries in flat order, 64 at a time.  Entries of one
//     64-entry chunk that name the same expert are found with ceil(log2 G) ballots
//     (lanes agreeing on every bit of the id), so one leader lane per distinct
//     expert bumps the wave's LDS counter -- no same-address LDS atomics under skew.
//     The lane's rank among its peers (mbcnt) plus the counter's old value is the
//     entry's stable rank inside the wave; a cross-wave prefix turns it into the
//     rank inside the tile.  Tile totals go to the workspace.  Dedup bucket masks
//     are per token; one ballot per bucket gives each token's rank among the
//     tile's tokens that send to that bucket.
//  2. layout_scan_kernel: one 1024-thread workgroup scans the per-tile counts down
//     each expert / bucket column, orders experts by (bucket, id), and writes the
//     counts, offsets and the status word.
//  3. layout_finalize_kernel: one thread per entry adds the expert offset and the
//     tile prefix to the tile-local rank, and scatters send_token.
#include "moe_internal.h"

namespace moedl {

namespace {

constexpr int kMaxE = MOE_MAX_EXPERTS;
constexpr int kMaxB = MOE_MAX_BUCKETS;
constexpr int kMaxK = MOE_MAX_TOPK;
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
__global__ __launch_bounds__(kTileThreads) void layout_tile_kernel(
    const int32_t* __restrict__ idx, int32_t M, int32_t k,
    const int32_t* __restrict__ ebkt, int32_t G, int32_t B, int32_t dedup,
    int32_t* __restrict__ slot_local, int32_t* __restrict__ row_local,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_bhist,
    int32_t* __restrict__ tile_err) {
  __shared__ unsigned char map_s[kMaxE];
  __shared__ int32_t wcnt[kTileWaves][kMaxE];
  __shared__ int32_t ids_s[kTileTokens * KC];  // the tile's expert ids, flat order
  __shared__ uint64_t wbal[kTileWaves][kMaxB];
  __shared__ int32_t wbcnt[kTileWaves][kMaxB];
  __shared__ int32_t err_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_index();
  const int tile = blockIdx.x;
  const int64_t Mk = (int64_t)M * k;
  const int nbits = bits_for(G);
  const uint64_t below = (1ull << lane) - 1ull;

  // ---- all global loads first: KC chunks of 64 flat entries per wave.  Loads are
  // unconditional (clamped index) so they are all in flight together.
  const int64_t tbase = (int64_t)tile * kTileTokens * k;  // first flat entry of the tile
  const int64_t wbase = tbase + (int64_t)w * 64 * k;
  int ec[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    const bool valid = c < k && f < Mk;
    const int v = idx[valid ? f : 0];
    ec[c] = valid ? v : kAbsent;
  }
  for (int e = tid; e < G; e += kTileThreads) {
    const int b = ebkt[e];
    map_s[e] = (b >= 0 && b < B) ? (unsigned char)b : kBadBucket;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) wcnt[ww][e] = 0;
  }
  if (tid == 0) err_s = kNoError;
  __syncthreads();

  // ---- stable ranks inside the wave: chunk c covers flat entries wbase + c*64 + lane
  int rc[KC];
  int my_err = kNoError;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    int e = ec[c];
    if (e != kAbsent && (e < 0 || e >= G)) {
      my_err = min(my_err, (int)(wbase + c * 64 + lane));
      e = kAbsent;
    }
    if (dedup && c < k) ids_s[w * 64 * k + c * 64 + lane] = e;
    const bool ok = e >= 0;
    const uint64_t peers = match_peers(ok, e, nbits);
    const int r = lanes_below(peers);
    int old = 0;
    if (ok) old = wcnt[w][e];
    if (ok && r == 0) wcnt[w][e] = old + __builtin_popcountll(peers);
    ec[c] = e;
    rc[c] = old + r;
  }
  if (my_err != kNoError) atomicMin(&err_s, my_err);
  __syncthreads();

  // cross-wave exclusive prefix per expert; the column total is the tile's count
  for (int e = tid; e < G; e += kTileThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) {
      const int v = wcnt[ww][e];
      wcnt[ww][e] = run;
      run += v;
    }
    tile_hist[(int64_t)tile * G + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int64_t f = wbase + (int64_t)c * 64 + lane;
    if (c < k && f < Mk) slot_local[f] = ec[c] >= 0 ? wcnt[w][ec[c]] + rc[c] : -1;
  }

  // ---- dedup rows: token view (lane = token), ids read back from LDS
  if (dedup) {
    const int64_t t = (int64_t)tile * kTileTokens + (int64_t)w * 64 + lane;
    const bool tv = t < M;
    const int* my_ids = ids_s + (w * 64 + lane) * k;
    int eb[KC];
    uint64_t bmask = 0;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      eb[j] = kBadBucket;
      if (j < k && tv) {
        const int e = my_ids[j];
        if (e >= 0) {
          eb[j] = map_s[e];
          if (eb[j] != kBadBucket) bmask |= 1ull << eb[j];
        }
      }
    }
    for (int b = 0; b < B; ++b) {
      const uint64_t bal = wave_ballot(tv && ((bmask >> b) & 1ull));
      if (lane == 0) {
        wbal[w][b] = bal;
        wbcnt[w][b] = __builtin_popcountll(bal);
      }
    }
    __syncthreads();
    if (tid < B) {
      int run = 0;
#pragma unroll
      for (int ww = 0; ww < kTileWaves; ++ww) {
        const int v = wbcnt[ww][tid];
        wbcnt[ww][tid] = run;
        run += v;
      }
      tile_bhist[(int64_t)tile * B + tid] = run;
    }
    __syncthreads();
    if (tv) {
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (j < k) {
          const int b = eb[j];
          row_local[t * k + j] =
              b != kBadBucket ? wbcnt[w][b] + __builtin_popcountll(wbal[w][b] & below) : -1;
        }
      }
    }
  }
  if (tid == 0) tile_err[tile] = err_s;
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
  // pass 1: segment sums (the last batch stays in registers)
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
  // pass 2: prefixes; a segment of one batch is still in registers
  if (active) {
    int run = seg[p * C + col];
    if (t1 - t0 <= kSegRegs) {
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

// Exclusive scan of one int per thread over the 1024-thread workgroup.
__device__ int block_exclusive_scan(int v, int32_t* wave_sums /* >= 16 */) {
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
    for (int q = 0; q < kScanThreads / 64; ++q) {
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

__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int32_t T, int32_t G, int32_t B, int32_t dedup, const int32_t* __restrict__ ebkt,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_bhist,
    const int32_t* __restrict__ tile_err, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ bucket_count,
    int32_t* __restrict__ bucket_offset, int32_t* __restrict__ status) {
  __shared__ int32_t seg[kScanThreads];
  __shared__ int32_t cnt_s[kMaxE];
  __shared__ int32_t arr_s[kMaxE];
  __shared__ int32_t wbc[kScanThreads / 64][kMaxB];
  __shared__ int32_t nexp_s[kMaxB + 1];
  __shared__ int32_t bsum_s[kMaxB];
  __shared__ int32_t btot_s[kMaxB];
  __shared__ int32_t wave_sums[kScanThreads / 64];
  __shared__ int32_t err_s;
  __shared__ int32_t mapbad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  if (tid == 0) {
    err_s = kNoError;
    mapbad_s = kNoError;
  }
  for (int i = tid; i < (kScanThreads / 64) * kMaxB; i += kScanThreads) wbc[i / kMaxB][i % kMaxB] = 0;
  if (tid < kMaxB) bsum_s[tid] = 0;
  __syncthreads();

  // Issue the small loads first; they are consumed after the column scan has issued
  // its own, so all global reads of this kernel share one round trip.
  const int map_b = tid < G ? ebkt[tid] : 0;
  int terr = kNoError;
  for (int i = tid; i < T; i += kScanThreads) terr = min(terr, tile_err[i]);

  // per-expert counts: column scan of the tile histograms
  column_exclusive_scan(tile_hist, T, G, cnt_s, seg);

  // status: bad map entries first, then the first bad expert id
  if (terr != kNoError) atomicMin(&err_s, terr);
  int b_of_e = 0;
  if (tid < G) {
    if (map_b < 0 || map_b >= B) atomicMin(&mapbad_s, tid);
    b_of_e = min(max(map_b, 0), B - 1);
  }

  // memory order of experts: sigma = sorted by (bucket, id).  Rank inside the wave
  // among experts of the same bucket, then per-(wave, bucket) prefixes.
  const bool ev = tid < G;
  const uint64_t peers = match_peers(ev, b_of_e, bits_for(B));
  const int rw = lanes_below(peers);
  if (ev && rw == 0) wbc[w][b_of_e] = __builtin_popcountll(peers);
  if (ev) atomicAdd(&bsum_s[b_of_e], cnt_s[tid]);
  __syncthreads();
  if (tid < B) {
    int run = 0;
    for (int q = 0; q < kScanThreads / 64; ++q) {
      const int v = wbc[q][tid];
      wbc[q][tid] = run;
      run += v;
    }
    nexp_s[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < B; ++b) {
      const int v = nexp_s[b];
      nexp_s[b] = run;
      run += v;
    }
  }
  __syncthreads();
  int pos = 0;
  if (ev) {
    pos = nexp_s[b_of_e] + wbc[w][b_of_e] + rw;
    arr_s[pos] = cnt_s[tid];
  }
  __syncthreads();
  const int v = tid < G ? arr_s[tid] : 0;
  const int ex = block_exclusive_scan(v, wave_sums);
  if (tid < G) arr_s[tid] = ex;
  __syncthreads();
  if (ev) {
    expert_count[tid] = cnt_s[tid];
    expert_offset[tid] = arr_s[pos];
  }

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
  (void)lane;
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
  const int T = (int)layout_tiles(M);
  const int64_t Mk = M * k;
  if (T > 0) {
#define MOEDL_TILE(KC)                                                                        \
  hipLaunchKernelGGL(layout_tile_kernel<KC>, dim3(T), dim3(kTileThreads), 0, stream, topk_idx, \
                     (int32_t)M, k, expert_bucket, G, B, dedup, slot, send_row, ws.tile_hist,  \
                     ws.tile_bhist, ws.tile_err)
    if (k <= 1) MOEDL_TILE(1);
    else if (k <= 2) MOEDL_TILE(2);
    else if (k <= 4) MOEDL_TILE(4);
    else if (k <= 8) MOEDL_TILE(8);
    else MOEDL_TILE(16);
#undef MOEDL_TILE
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
  return hipGetLastError();
}

}  // namespace moedl
