// Device helpers shared by the libmsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

namespace msa {

constexpr int kBlock = 128;   // B_k, tokens per KV block
constexpr int kWave = 64;

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].
// Lane l supplies A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32], e = 0..7,
// and holds D[8*(j/4) + 4*(l/32) + j%4][l%32] in accumulator j = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held by lane half `h` in register j.
__device__ __forceinline__ constexpr int acc_row(int j, int h) {
  return 8 * (j >> 2) + 4 * h + (j & 3);
}

__device__ __forceinline__ float bf2f(__bf16 x) { return static_cast<float>(x); }

// Round-to-nearest-even fp32 -> bf16.
__device__ __forceinline__ __bf16 f2bf(float x) { return static_cast<__bf16>(x); }

// Monotone map of fp32 onto uint32: a < b  <=>  ord(a) < ord(b) (no NaNs).
__device__ __forceinline__ uint32_t ord_f32(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int o) {
  uint32_t lo = __shfl_xor((uint32_t)x, o, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(x >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t y = shfl_xor_u64(x, o);
    x = y > x ? y : x;
  }
  return x;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace msa
