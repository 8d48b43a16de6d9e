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

// Integer DPP move: lanes whose source is outside the row (bound_ctrl) or
// whose row is masked out read 0.
enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,  // lane 15 of each row -> the next row
  kDppRowBcast31 = 0x143   // lane 31 -> rows 2 and 3
};

template <int CTRL, int ROW_MASK = 0xF, bool BOUND = true>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, BOUND);
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active):
// Hillis-Steele within each 16-lane row, then the row carries.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<kDppRowShr1>(x);
  x += dpp_u32<kDppRowShr2>(x);
  x += dpp_u32<kDppRowShr4>(x);
  x += dpp_u32<kDppRowShr8>(x);
  x += dpp_u32<kDppRowBcast15, 0xA, false>(x);
  x += dpp_u32<kDppRowBcast31, 0xC, false>(x);
  return x;
}

__device__ __forceinline__ uint32_t readlane(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Bitwise AND / OR of a 64-bit value over the wave, in every lane: the four
// DPP row permutations reach all 16 lanes of a row, readlane joins the rows.
template <bool AND>
__device__ __forceinline__ uint32_t wave_bits32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return AND ? (a & b) : (a | b); };
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor2, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowHalfMirror, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowMirror, 0xF, 0xF, false));
  return op(op(readlane(x, 0), readlane(x, 16)), op(readlane(x, 32), readlane(x, 48)));
}

__device__ __forceinline__ uint64_t wave_and64(uint64_t x) {
  return ((uint64_t)wave_bits32<true>((uint32_t)(x >> 32)) << 32) | wave_bits32<true>((uint32_t)x);
}

__device__ __forceinline__ uint64_t wave_or64(uint64_t x) {
  return ((uint64_t)wave_bits32<false>((uint32_t)(x >> 32)) << 32) | wave_bits32<false>((uint32_t)x);
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
// After the conversion -0 is folded to +0 by an FP16 add of +0 (round to
// nearest: -0 + +0 = +0, every other value unchanged).  The key flips all 16
// bits of a negative pattern and only the sign bit of a non-negative one:
// b ^ 0x8000 ^ (the sign bit smeared over bits 14..0).
__device__ __forceinline__ uint32_t bin_of(float v) {
  const _Float16 h = (_Float16)v + (_Float16)0.0f;
  const uint32_t b = __builtin_bit_cast(uint16_t, h);
  const uint32_t smear = (uint32_t)__builtin_amdgcn_sbfe((int)b, 15, 1) & 0x7FFFu;
  return ((b ^ smear) ^ 0x8000u) >> 6;
}

// bin_of for two values at once (the same mapping, entry a in the low 16
// bits of the result, b in the high 16): one packed FP32 -> FP16 conversion
// (round to nearest even), one packed FP16 add of +0, and the key transform
// on both 16-bit halves.
typedef _Float16 bs_half2 __attribute__((ext_vector_type(2)));
typedef float bs_float2 __attribute__((ext_vector_type(2)));
typedef uint16_t bs_ushort2 __attribute__((ext_vector_type(2)));
typedef int16_t bs_short2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bin_pair(float a, float b) {
  const bs_half2 h = __builtin_convertvector((bs_float2){a, b}, bs_half2) + (bs_half2){0, 0};
  const bs_ushort2 u = __builtin_bit_cast(bs_ushort2, h);
  const bs_short2 sign = __builtin_bit_cast(bs_short2, u) >> 15;
  const bs_ushort2 key = u ^ (__builtin_bit_cast(bs_ushort2, sign) | (bs_ushort2){0x8000, 0x8000});
  return __builtin_bit_cast(uint32_t, (bs_ushort2)(key >> 6));
}

// Per 16-bit half: 1 if the half of `codes` exceeds the same half of `t`,
// else 0 (a saturating packed subtract, then a packed min with 1).
__device__ __forceinline__ uint32_t pk_gt_flags(uint32_t codes, uint32_t t) {
  uint32_t g;
  asm("v_pk_sub_u16 %0, %1, %2 clamp\n\tv_pk_min_u16 %0, %0, 1 op_sel_hi:[1,0]" : "=&v"(g) : "v"(codes), "v"(t));
  return g;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Blocks visible to a query row at position t (it sees tokens 0..t): those
// whose c tokens all lie at or before t, floor((t+1)/c), capped at the
// caller's bound max_vis and at 0 for an invalid position.
__device__ __forceinline__ int visible_blocks(int t, int c, int max_vis) { return max(0, min((t + 1) / c, max_vis)); }

// Reads FP32 entries of one row through a raw buffer resource: one lane
// offset per load (no 64-bit address registers), and the hardware range check
// returns 0 for entries at or past n, so reads past the row never fault.
struct RowReader {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ RowReader(const float* row, int n)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, n > 0 ? n * 4 : 0,
                                               0x00020000)) {}
  __device__ __forceinline__ float operator[](int idx) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, idx * 4, 0, 0));
  }
  // Entry lane_idx + uniform_idx, the uniform part passed as the scalar
  // offset, so that loads strided by a constant share one lane offset
  // register.
  __device__ __forceinline__ float at(int lane_idx, int uniform_idx) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_idx * 4, uniform_idx * 4, 0));
  }
};

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Loads 64 lanes x 16 bytes from a buffer straight into LDS (no VGPRs): lane
// i reads at byte `voffset` of the resource and writes LDS bytes
// lds_addr + 16*i .. +15 (M0 holds the wave-uniform LDS address).  The
// transfer is counted by vmcnt; the caller waits with s_waitcnt before a
// barrier publishes the data.  Out-of-range lanes of the resource write zeros.
__device__ __forceinline__ void lds_dma_b128(const u32x4_t& rsrc, uint32_t voffset, uint32_t lds_addr) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)rsrc.y << 32) | rsrc.x), (short)0, rsrc.z, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds_addr, 16, voffset, 0, 0, 0);
}

// vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace bs
