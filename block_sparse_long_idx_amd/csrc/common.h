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

__device__ __forceinline__ uint64_t join_u64(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | lo;
}

// max(x, x of the lane that the DPP control CTRL maps onto this one)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint64_t y = join_u64((uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false),
                              (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false));
  return y > x ? y : x;
}

// Maximum over the 64 lanes, returned wave-uniform, without LDS traffic:
// DPP quad_perm pairs lanes 1 and then 2 apart (every lane then holds its
// quad's maximum), row_half_mirror pairs the two quads of each 8-lane
// group, row_mirror the two 8-lane groups of each 16-lane row, ds_swizzle
// (bit mode, xor 16) the two rows of each 32-lane half, and readlane joins
// the halves.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = dpp_max_u64<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_max_u64<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_max_u64<0x141>(x);  // row_half_mirror
  x = dpp_max_u64<0x140>(x);  // row_mirror
  {
    const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
    const uint64_t y = join_u64((uint32_t)__builtin_amdgcn_ds_swizzle(lo, 0x401F),
                                (uint32_t)__builtin_amdgcn_ds_swizzle(hi, 0x401F));
    x = y > x ? y : x;
  }
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint64_t a = join_u64((uint32_t)__builtin_amdgcn_readlane(lo, 0),
                              (uint32_t)__builtin_amdgcn_readlane(hi, 0));
  const uint64_t b = join_u64((uint32_t)__builtin_amdgcn_readlane(lo, 32),
                              (uint32_t)__builtin_amdgcn_readlane(hi, 32));
  return a > b ? a : b;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace msa
