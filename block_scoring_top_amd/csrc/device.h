// device.h - gfx950 device helpers shared by the indexer kernels.
//
// Wavefronts are 64 lanes.  DPP row operations act within 16-lane rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/blockscore.h"

namespace bs {

constexpr int kHeads = BS_HEADS;
constexpr int kDim = BS_DIM;
constexpr int kPage = BS_PAGE_TOKENS;
constexpr int kKmax = BS_KMAX;
constexpr int kBins = 1024;  // 10-bit coarse histogram (TopK-V2, Figure 3)

// fl32(1/sqrt(128)): sqrt(128) = 8*sqrt(2), so 1/sqrt(128) = sqrt(2)/16.
constexpr float kScale = 0.08838834764831845f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Two bf16 products summed into an FP32 accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// DPP lane moves inside a 16-lane row.  Every control used here is a
// permutation of the row, so no lane reads outside it.
enum : int {
  kDppQuadXor1 = 0xB1,     // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,     // quad_perm [2,3,0,1]
  kDppRowMirror = 0x140,   // lane i <- lane 15-i
  kDppRowHalfMirror = 0x141  // lane i <- lane 7-i within each 8-lane half
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Order-preserving keys.  -0.0 is folded to +0.0 first so that equal values
// get equal keys; non-negative patterns get the sign bit set and negative
// patterns are inverted, so unsigned key order equals numeric order.
__device__ __forceinline__ uint32_t key32_of(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// FP32 -> FP16 with the hardware conversion (round to nearest even, overflow
// to infinity), then the 16-bit order-preserving key; the coarse bin is its
// upper 10 bits.
__device__ __forceinline__ uint32_t bin_of(float v) {
  _Float16 h = (_Float16)v;
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  b = (b == 0x8000u) ? 0u : b;
  uint32_t key = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  return key >> 6;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

}  // namespace bs
