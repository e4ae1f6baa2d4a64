// Combine on gfx950: y[t] = bf16( sum_j w[t,j] * expert_out[slot[t,j]] ).
//
// Determinism follows "Purlin: Separating Orchestration from the Datapath of
// Collectives", section 3.3 (SCORE): exactly one lane owns each output element and
// accumulates its k sources in source order (j ascending), each step one rounded
// fp32 multiply and one rounded fp32 add (this file is built without FP
// contraction), starting from +0.0, then one round-to-nearest-even to bf16
// (v_cvt_pk_bf16_f32).  The result is bitwise reproducible and independent of the
// launch geometry.  Keeping several sources in flight while accumulating in order
// is the same idea as that section's pipelined, ordered reduction; here the k
// loads of a column group are all issued before the first add.
//
// Mapping: one wave64 per token, four tokens per 256-thread workgroup.  The k slots
// and weights are wave-uniform scalar loads.  The row is walked in groups of GV
// 16-byte vectors per lane (8 bf16 each); for each group the k source rows' vectors
// are loaded (k*GV loads in flight per lane), accumulated in fp32 in j order, and
// the 16-byte bf16 result is stored.  Loads and stores are non-temporal: each
// expert row is read exactly once.
#include "moe_internal.h"

#pragma clang fp contract(off)

namespace moedl {
namespace {

constexpr int kTokensPerBlock = 4;
constexpr int kGroupVecs = 2;  // 16-byte vectors per lane per column group

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int K>
__global__ __launch_bounds__(256) void combine_kernel(
    const u32x4* __restrict__ eo, int64_t expert_rows, const float* __restrict__ wts,
    const int32_t* __restrict__ slot, int64_t M, int32_t row_vecs, u32x4* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + wave_index();
  if (t >= M) return;

  int64_t row[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int s = slot[t * K + j];
    row[j] = (s >= 0 && s < expert_rows) ? (int64_t)s * row_vecs : -1;
    w[j] = wts[t * K + j];
  }

  for (int base = 0; base < row_vecs; base += 64 * kGroupVecs) {
    u32x4 d[K][kGroupVecs];
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int i = 0; i < kGroupVecs; ++i) {
        const int c = base + lane + 64 * i;
        d[j][i] = (u32x4){0u, 0u, 0u, 0u};
        if (row[j] >= 0 && c < row_vecs) d[j][i] = __builtin_nontemporal_load(eo + row[j] + c);
      }
    }
#pragma unroll
    for (int i = 0; i < kGroupVecs; ++i) {
      const int c = base + lane + 64 * i;
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if (row[j] < 0) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = d[j][i][q];
          const float lo = __builtin_bit_cast(float, u << 16);
          const float hi = __builtin_bit_cast(float, u & 0xFFFF0000u);
          const float plo = w[j] * lo;
          const float phi = w[j] * hi;
          acc[2 * q] = acc[2 * q] + plo;
          acc[2 * q + 1] = acc[2 * q + 1] + phi;
        }
      }
      if (c < row_vecs) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        __builtin_nontemporal_store(o, y + t * row_vecs + c);
      }
    }
  }
}

template <int K>
hipError_t launch_k(const uint16_t* expert_out, int64_t expert_rows, const float* weights,
                    const int32_t* slot, int64_t M, int32_t row_vecs, uint16_t* y,
                    hipStream_t stream) {
  const int64_t blocks = (M + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(combine_kernel<K>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4*)expert_out, expert_rows, weights, slot, M, row_vecs,
                     (u32x4*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* expert_out, int64_t expert_rows, const float* weights,
                          const int32_t* slot, int64_t M, int32_t k, int32_t N, uint16_t* y,
                          hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int32_t row_vecs = N / 8;
#define MOEDL_CASE(K) \
  case K:             \
    return launch_k<K>(expert_out, expert_rows, weights, slot, M, row_vecs, y, stream);
  switch (k) {
    MOEDL_CASE(1) MOEDL_CASE(2) MOEDL_CASE(3) MOEDL_CASE(4) MOEDL_CASE(5) MOEDL_CASE(6)
    MOEDL_CASE(7) MOEDL_CASE(8) MOEDL_CASE(9) MOEDL_CASE(10) MOEDL_CASE(11) MOEDL_CASE(12)
    MOEDL_CASE(13) MOEDL_CASE(14) MOEDL_CASE(15) MOEDL_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOEDL_CASE
}

}  // namespace moedl
