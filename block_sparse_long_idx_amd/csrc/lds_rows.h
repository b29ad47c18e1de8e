// Shared by the kernels that keep 128-row blocks of keys in LDS.
#pragma once

namespace msa {

constexpr int kMaxItem = 2048;  // max query positions per KV-outer work item
constexpr int kMaxK = 32;       // max selected blocks per (query, group)

// XOR swizzle of the 16-byte chunks of row `row` of a [128][D] bf16 block in
// LDS.  A fragment read has 16 lanes (16 consecutive rows, one chunk index)
// in flight per LDS cycle; the swizzle sends them to 16 distinct 4-bank
// groups.  D = 128: a row spans all 64 banks, so rows differ in their low 4
// bits.  D = 64: two rows share a bank row (row & 1 picks the half), the
// next 3 bits pick the chunk.  D = 32: four rows share a bank row.
template <int D>
__device__ __forceinline__ int row_swz(int row) {
  return D == 128 ? (row & 15) : D == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

}  // namespace msa
