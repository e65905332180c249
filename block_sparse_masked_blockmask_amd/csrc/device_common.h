// Device-side helpers shared by the BlockMask builder and the forward kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flexattn.h"
#include "tile_class.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// mask_mod for one (query, key) pair (the predicate itself is mask_pair_flags in tile_class.h).
// Flags are wave-uniform.
struct MaskSpec {
  int flags;
  int window;
  int prefix_len;
};

__device__ __forceinline__ bool mask_pair(const MaskSpec& m, int i, int j, int qdoc, int kvdoc) {
  return mask_pair_flags(m.flags, m.window, m.prefix_len, i, j, qdoc, kvdoc);
}

// Cross-half exchange inside a wave64: v_permlane32_swap swaps the upper half of the first
// operand with the lower half of the second. Called with the same value twice, one of the
// two results is the caller's own value and the other is the value of lane (l ^ 32), so a
// max or sum of both results combines the two halves.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x) = 1 - 2 / (exp(2x) + 1), with hardware exp2 and reciprocal; saturates to +-1 for
// large |x| (exp2 gives inf or 0). Absolute error is a few fp32 ulps of 1.
__device__ __forceinline__ float fast_tanh(float x) {
  float e = __builtin_amdgcn_exp2f(x * (2.0f * kLog2e));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// 16-byte-chunk XOR swizzle of a [rows][128] bf16 tile in LDS (256 bytes per row, 16 chunks).
// Row r stores chunk c at position c ^ swz(r). swz mixes r%4 into bits 2-3 and (r/4)%4 into
// bits 0-1, so that (a) 16 consecutive rows read at one chunk hit 16 distinct positions
// (K operand reads, ds_read_b128) and (b) 4 consecutive rows read at 4 consecutive chunks
// hit 16 distinct positions (V operand transposed reads, ds_read_b64_tr_b16).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * 256 + ((chunk ^ swz(r)) << 4); }

// Map a linear workgroup id onto a logical work id so that each of the 8 XCDs (which receive
// workgroups round-robin) processes one contiguous range of logical ids: neighbouring work
// items share K/V tiles, and this keeps them in one XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int per = n / 8, rem = n % 8;
  const int x = wg % 8, s = wg / 8;
  return x * per + (x < rem ? x : rem) + s;
}

}  // namespace fa
