// Test and measurement helpers beside the dispatch/combine path (libmoedl_harness):
// the expert stand-ins that produce combine's inputs, and a plain streaming copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_harness.h"

#pragma clang fp contract(off)

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// OCP fp8 e4m3 ("fn") code -> float, from the format's definition: bias 7, three
// mantissa bits, exponent field 0 subnormal (m * 2^-9), S.1111.111 NaN.
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t ex = (b >> 3) & 0xFu;
  const uint32_t man = b & 0x7u;
  float v;
  if (ex == 0) {
    v = (float)man * 0x1p-9f;
  } else if (ex == 0xFu && man == 0x7u) {
    v = __builtin_nanf("");
  } else {
    v = __builtin_bit_cast(float, ((ex + 120u) << 23) | (man << 20));
  }
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | sign);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// One wave64 per (t, j) entry; lane c handles elements [8c', 8c'+8) of the row.
__global__ __launch_bounds__(256) void standin_kernel(
    int32_t kind, const uint8_t* __restrict__ sent, const float* __restrict__ sent_scale,
    int64_t sent_rows, int32_t N, const int32_t* __restrict__ send_row,
    const int32_t* __restrict__ slot, const int32_t* __restrict__ topk_idx, int64_t Mk,
    uint16_t* __restrict__ eo, int64_t expert_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= Mk) return;
  const int src = send_row[f];
  const int dst = slot[f];
  const int e = topk_idx[f];
  if (src < 0 || src >= sent_rows || dst < 0 || dst >= expert_rows) return;
  uint16_t* out = eo + (int64_t)dst * N;
  if (kind == MOE_STANDIN_DEQUANT) {
    const uint8_t* in = sent + (int64_t)src * N;
    const float* sc = sent_scale + (int64_t)src * (N / 128);
    for (int i = lane * 8; i < N; i += 64 * 8) {
      const float s = sc[i / 128];
#pragma unroll
      for (int q = 0; q < 8; ++q) out[i + q] = to_bf16(e4m3_to_float(in[i + q]) * s);
    }
  } else {
    const uint16_t* in = (const uint16_t*)sent + (int64_t)src * N;
    const float factor = 1.0f + (float)e / 256.0f;
    for (int i = lane * 8; i < N; i += 64 * 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint16_t v = in[i + q];
        out[i + q] = kind == MOE_STANDIN_IDENTITY
                         ? v
                         : to_bf16(__builtin_bit_cast(float, (uint32_t)v << 16) * factor);
      }
    }
  }
}

// One 16-byte vector per thread over a full grid: the fastest plain copy shape
// measured on MI355X (a persistent grid-stride loop reaches ~4.8 TB/s).  The launch
// requests kCopyLds bytes of (unused) dynamic LDS per workgroup, which caps residency
// at five workgroups per CU: fastest at 2 GiB, 6.74 TB/s read+write against 6.56 with
// no cap (sweep of the reservation: 24-30 KiB best, 32 KiB and more slower).
constexpr unsigned kCopyLds = 30 * 1024;

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" int moe_harness_expert_outputs(int32_t kind, const void* sent, const float* sent_scale,
                                          int64_t sent_rows, int32_t N, const int32_t* send_row,
                                          const int32_t* slot, const int32_t* topk_idx, int64_t M,
                                          int32_t k, uint16_t* expert_out, int64_t expert_rows,
                                          hipStream_t stream) {
  if (kind < 0 || kind > 2 || M < 0 || k < 1 || N < 8 || N % 8 != 0) return 1;
  if (kind == MOE_STANDIN_DEQUANT && (N % 128 != 0 || !sent_scale)) return 1;
  const int64_t Mk = M * k;
  if (Mk == 0) return 0;
  if (!sent || !send_row || !slot || !topk_idx || !expert_out) return 1;
  hipLaunchKernelGGL(standin_kernel, dim3((unsigned)((Mk + 3) / 4)), dim3(256), 0, stream, kind,
                     (const uint8_t*)sent, sent_scale, sent_rows, N, send_row, slot, topk_idx,
                     Mk, expert_out, expert_rows);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_harness_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0 || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return 1;
  if (bytes == 0) return 0;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), kCopyLds, stream,
                     (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
