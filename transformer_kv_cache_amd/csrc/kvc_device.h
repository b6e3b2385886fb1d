// kvc_device.h -- small device helpers shared by the attention kernels of
// libkvcache.so: the softmax's exp2 and state rescale, and the gfx950
// cross-lane moves the split kernels reduce with.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the transcendental unit (log2(e) is folded into the score scale).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight of a softmax state with max m when merged under a common max M
// (0 for an empty state, m = -inf).
__device__ __forceinline__ float rescale(float m, float M) {
  return m == kNegInf ? 0.f : fast_exp2(m - M);
}

// DPP controls (GFX9 encoding), all inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane ^ 7 inside 8
constexpr int kDppRowMirror = 0x140;  // row_mirror: lane ^ 15
constexpr int kDppRowRor8 = 0x128;    // row_ror:8: lane ^ 8

// The value of lane CTRL(lane), every lane valid.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// x combined (sum, or max with MAX) with the value OFF lanes away, OFF in
// {8, 16, 32}, every lane getting the result.  OFF = 8 is a DPP rotate inside
// the 16-lane row; OFF = 16 and 32 use the gfx950 permlane swaps, which trade
// rows (or half-waves) between two registers: swapping x with itself leaves
// the two partners' values in the two results, so combining them gives the
// pair's total in every lane, in VALU latency rather than an LDS round trip.
template <int OFF, bool MAX = false>
__device__ __forceinline__ float xor_combine(float x) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "partner distance");
  float y0, y1;
  if constexpr (OFF == 8) {
    y0 = x;
    y1 = dpp_mov<kDppRowRor8>(x);
  } else {
    const uint32_t u = __float_as_uint(x);
    const auto r = (OFF == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                               : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    y0 = __uint_as_float(r[0]);
    y1 = __uint_as_float(r[1]);
  }
  return MAX ? fmaxf(y0, y1) : y0 + y1;
}

}  // namespace kvc
