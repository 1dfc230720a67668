// Register types, the K-row permutation and the LDS swizzles shared by the
// forward and backward attention kernels.
#ifndef BSGA_TILE_COMMON_HPP
#define BSGA_TILE_COMMON_HPP

#include "bsga_internal.hpp"

namespace bsga {

constexpr float kScaleLog2 = 0.18033688011112042f;  // log2(e) / sqrt(64)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rows i = 8a + 4hh + c of a 32x32 accumulator become operand keys (or
// queries) 16m + 8hh + e when the A-operand row i is loaded from row pi(i):
// pi swaps bits 2 and 3 (an involution).
__device__ inline int pi_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// LDS swizzles (16-byte chunk index XOR a row function) so that the MFMA
// operand reads touch distinct banks: swz_k for 64-dim rows (8 chunks),
// swz_v<T> for transposed tiles (T/8 chunks per dim row).
__device__ inline int swz_k(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 1); }
template <int KT>
__device__ inline int swz_v(int d) {
  if constexpr (KT == 128) return d & 15;
  else return ((d >> 1) & 7) ^ ((d & 1) << 2);
}

}  // namespace bsga

#endif
