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


// ---- split-state merge shared by the split kernels and the combine pass ----

// Reads of split states written by other workgroups of the same launch.
// A workgroup-scope load is coherent only within the workgroup, so the CU's
// L1 may serve it from a copy of the line taken earlier.  Partial outputs
// are whole lines of one (split, row), read once by the row's one merging
// workgroup after their writers finished, so no earlier copy can exist; the
// (max, sum) pairs of 16 rows share a line, so those are read by an atomic
// (an add of 0), which the L2 the writers stored to performs.
__device__ __forceinline__ float state_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t state_fetch_ml(const float *p) {
  // The zero is hidden from the compiler, which would otherwise turn the
  // no-op atomic into a plain load.
  uint64_t zero = 0;
  asm volatile("" : "+v"(zero));
  return __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), zero, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of a query row's split states into the running state (M, L, o) of
// one wave (lane j holds output elements j, j + 64, ...):
//   o = sum_s 2^(m_s - M') o_s + 2^(M - M') o,  L likewise,  M' = max(M, m_s)
// over splits 0 .. nsplit-1, in chunks of CH whose loads are all issued
// before any is used (lane t < CH fetches split s0 + t's pair, which every
// lane then takes from it).  The fused kernel's last workgroup and
// combine_kernel both run exactly this, so their outputs are bit-identical.
template <int D>
__device__ __forceinline__ void merge_states(const float *ws_o, const float *ws_ml, int64_t ws_rows,
                                             int64_t row, int nsplit, int lane, float &M, float &L,
                                             float (&o)[D / 64]) {
  constexpr int EPL = D / 64;
  constexpr int CH = 16;
  for (int s0 = 0; s0 < nsplit; s0 += CH) {
    float mv[CH], lv[CH], ov[CH][EPL];
    uint64_t ml = 0;
    if (lane < CH && s0 + lane < nsplit)
      ml = state_fetch_ml(ws_ml + ((size_t)(s0 + lane) * (size_t)ws_rows + (size_t)row) * 2);
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int sp = (s0 + t < nsplit) ? s0 + t : nsplit - 1;
      const size_t ws = (size_t)sp * (size_t)ws_rows + (size_t)row;
#pragma unroll
      for (int j = 0; j < EPL; ++j) ov[t][j] = state_load(ws_o + ws * D + lane + 64 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t ml_lo = (uint32_t)ml, ml_hi = (uint32_t)(ml >> 32);
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      mv[t] = __uint_as_float(__builtin_amdgcn_readlane(ml_lo, t));
      lv[t] = __uint_as_float(__builtin_amdgcn_readlane(ml_hi, t));
    }
    float Mc = M;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      if (s0 + t >= nsplit) mv[t] = kNegInf;
      Mc = fmaxf(Mc, mv[t]);
    }
    const float fr = rescale(M, Mc);
    L *= fr;
#pragma unroll
    for (int j = 0; j < EPL; ++j) o[j] *= fr;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const float f = rescale(mv[t], Mc);
      L = fmaf(f, lv[t], L);
#pragma unroll
      for (int j = 0; j < EPL; ++j) o[j] = fmaf(f, ov[t][j], o[j]);
    }
    M = Mc;
  }
}

// Count a split workgroup's state (already stored) on its unit's 64-bit
// arrival counter and tell whether it arrived last.  The caller has waited
// until the L2 acknowledged the state stores (s_waitcnt vmcnt(0)) in every
// wave that stored; one lane calls this.  The count also sums each
// writer's XCD id x and x^2: with n earlier writers, sum x = n y and sum
// x^2 = n y^2 hold for this workgroup's id y only if every x equals y
// (their variance about y is zero), i.e. only if every state went through
// this XCD's L2 -- `misplaced` reports otherwise.
__device__ __forceinline__ bool arrive_last(uint64_t *counter, int nsplit, bool &misplaced) {
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  xcc &= 0xFu;
  const uint64_t mark = 1ull | ((uint64_t)xcc << 16) | ((uint64_t)(xcc * xcc) << 36);
  const uint64_t prev = __hip_atomic_fetch_add(counter, mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t n = prev & 0xFFFFu;
  misplaced = ((prev >> 16) & 0xFFFFFu) != n * xcc || (prev >> 36) != n * xcc * xcc;
  return n == (uint64_t)(nsplit - 1);
}

// The merging workgroup leaves the counter zero for the next call.
__device__ __forceinline__ void reset_counter(uint64_t *counter) {
  __hip_atomic_store(counter, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvc
