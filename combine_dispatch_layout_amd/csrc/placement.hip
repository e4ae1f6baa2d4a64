// Correlation-aware expert placement: the expert pair co-occurrence histogram on
// gfx950 and the greedy expert -> bucket packing on the host.
//
// "Zyphra says routing-pattern expert placement speeds MoE token communication up
// to 2.63x on AMD MI300X": experts that tokens choose together are placed on the
// same destination, so a token's copies there collapse into one (the pair statistics
// and copy-reduction items).  The page states the idea only; the counting and the
// greedy below are this library's reading of it.
//
// pair counts: C[a][b] = number of tokens whose expert set holds both a and b (a
// repeated expert counts once); C[a][a] = tokens choosing a.  The G x G matrix does not
// fit LDS for large G, so the grid is (token chunk) x (row block): a workgroup keeps
// rows [r0, r0 + RB) of the matrix in LDS (RB * G <= 8192 counters), walks its 256
// tokens (one per thread, the token's k ids in registers, deduplicated), adds its
// pairs with LDS atomics, and flushes the nonzero counters with device-scope global
// atomics.  Integer counts: the result is exact and order independent.
//
// greedy placement (host): clusters grow by visiting pairs (a < b) with C > 0 in
// count-descending order (ties by a, then b), joining two clusters when the merged
// size stays within G/B; clusters (size descending, ties by smallest member) go whole
// into the first bucket with room; leftovers fill free places expert by expert.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "moe_internal.h"

namespace moedl {
namespace {

constexpr int kPairLds = 8192;   // LDS counters per workgroup (32 KiB)
constexpr int kPairTokens = 256;  // tokens per workgroup, one per thread

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int KC>
__global__ __launch_bounds__(256) void pair_counts_kernel(const int32_t* __restrict__ idx,
                                                          int64_t M, int32_t k, int32_t G,
                                                          int32_t rows_per_block,
                                                          int32_t* __restrict__ counts) {
  __shared__ int32_t hist[kPairLds];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * rows_per_block;
  const int r1 = min(G, r0 + rows_per_block);
  const int n = (r1 - r0) * G;
  for (int i = tid; i < n; i += 256) hist[i] = 0;

  const int64_t t = (int64_t)blockIdx.x * kPairTokens + tid;
  int e[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const bool in = t < M && j < k;
    const int v = in ? idx[t * k + j] : -1;
    e[j] = (v >= 0 && v < G) ? v : -1;
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {  // keep the first occurrence of each expert
#pragma unroll
    for (int jj = 0; jj < j; ++jj)
      if (e[jj] == e[j]) e[j] = -1;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (e[j] < r0 || e[j] >= r1) continue;  // also skips -1
    int32_t* row = hist + (e[j] - r0) * G;
#pragma unroll
    for (int jj = 0; jj < KC; ++jj)
      if (e[jj] >= 0) atomicAdd(row + e[jj], 1);
  }
  __syncthreads();
  int32_t* out = counts + (int64_t)r0 * G;
  for (int i = tid; i < n; i += 256) {
    const int v = hist[i];
    if (v) atomicAdd(out + i, v);
  }
}

}  // namespace

hipError_t launch_pair_counts(const int32_t* topk_idx, int64_t M, int32_t k, int32_t G,
                              int32_t* counts, hipStream_t stream) {
  const int64_t n = (int64_t)G * G;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     counts, n);
  if (M > 0) {
    const int rows = std::max(1, std::min<int>(G, kPairLds / G));
    const dim3 grid((unsigned)((M + kPairTokens - 1) / kPairTokens), (unsigned)((G + rows - 1) / rows));
#define MOEDL_PAIRS(KC)                                                                        \
  hipLaunchKernelGGL(pair_counts_kernel<KC>, grid, dim3(256), 0, stream, topk_idx, M, k, G, rows, \
                     counts)
    if (k <= 1) MOEDL_PAIRS(1);
    else if (k <= 2) MOEDL_PAIRS(2);
    else if (k <= 4) MOEDL_PAIRS(4);
    else if (k <= 8) MOEDL_PAIRS(8);
    else MOEDL_PAIRS(16);
#undef MOEDL_PAIRS
  }
  return hipGetLastError();
}

void place_experts_greedy(const int32_t* C, int32_t G, int32_t B, int32_t* bucket) {
  const int cap = G / B;
  std::vector<int> parent(G), size(G, 1);
  for (int e = 0; e < G; ++e) parent[e] = e;
  auto find = [&](int a) {  // with path halving; the roots, hence the result, are unchanged
    while (parent[a] != a) {
      parent[a] = parent[parent[a]];
      a = parent[a];
    }
    return a;
  };

  struct Pair {
    int32_t count, a, b;
  };
  std::vector<Pair> pairs;
  for (int a = 0; a < G; ++a)
    for (int b = a + 1; b < G; ++b)
      if (C[(int64_t)a * G + b] > 0) pairs.push_back({C[(int64_t)a * G + b], a, b});
  std::sort(pairs.begin(), pairs.end(), [](const Pair& x, const Pair& y) {
    if (x.count != y.count) return x.count > y.count;
    if (x.a != y.a) return x.a < y.a;
    return x.b < y.b;
  });
  for (const Pair& p : pairs) {
    const int ra = find(p.a), rb = find(p.b);
    if (ra != rb && size[ra] + size[rb] <= cap) {
      const int lo = std::min(ra, rb), hi = std::max(ra, rb);
      parent[hi] = lo;
      size[lo] += size[hi];
    }
  }

  std::vector<std::vector<int>> clusters;
  std::vector<int> slot_of_root(G, -1);
  for (int e = 0; e < G; ++e) {  // ascending e: members come out sorted
    const int r = find(e);
    if (slot_of_root[r] < 0) {
      slot_of_root[r] = (int)clusters.size();
      clusters.emplace_back();
    }
    clusters[slot_of_root[r]].push_back(e);
  }
  std::stable_sort(clusters.begin(), clusters.end(),
                   [](const std::vector<int>& x, const std::vector<int>& y) {
                     if (x.size() != y.size()) return x.size() > y.size();
                     return x[0] < y[0];
                   });

  std::vector<int> fill(B, 0);
  std::vector<const std::vector<int>*> waiting;
  for (const auto& m : clusters) {
    int dst = -1;
    for (int b = 0; b < B && dst < 0; ++b)
      if (fill[b] + (int)m.size() <= cap) dst = b;
    if (dst < 0) {
      waiting.push_back(&m);
      continue;
    }
    for (int e : m) bucket[e] = dst;
    fill[dst] += (int)m.size();
  }
  for (const auto* m : waiting)
    for (int e : *m) {
      int b = 0;
      while (fill[b] >= cap) ++b;
      bucket[e] = b;
      ++fill[b];
    }
}

}  // namespace moedl
