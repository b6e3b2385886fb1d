// kvc_decode_rows.hip -- split-K decode for a few query rows per KV head on
// the vector ALUs, streaming K/V in the access pattern of the single-row
// kernel.
//
// Same computation as kvc_decode.hip and kvc_decode_mfma.hip ([KV-4]
// jennyma11.github.io/infra/ch07-01.html, "Decode 阶段", listing 1-2; [KV-2]
// openai-hub.com/news/2435, "一个很容易漏掉的错误": row i of N new rows sees keys
// 0 .. P+i), for a KV head that serves R = G * N query rows -- GQA groups
// and short chunks: 2 <= R <= 8, fp32 with D = 64 or bf16 with D = 128 or 64.
//
// Streaming.  A workgroup (256 lanes) owns one (layer, sequence, KV head,
// split of 256 / LPR * KPL consecutive keys).  A key row is LPR lanes wide
// (16 for 256-byte rows: one DPP row; 8 for 128-byte rows: half of one); a
// workgroup-wide load covers 256 / LPR consecutive rows (4 KB), so every
// wave instruction reads 1 KB of contiguous memory, and each lane issues its
// KPL K loads and KPL V loads before any arithmetic, as the single-row
// kernel does.
//
// Scores.  Each lane forms its 16-byte slice of the dot product with each of
// the RP (R padded to a power of two) query rows, then the RP partial sums
// are reduced over the LPR lanes of the key by a butterfly reduce-scatter:
// at each of the first log2(RP) steps a lane keeps half of its values and
// adds the partner's other half, the remaining steps add single values.  The
// partner pairs are DPP lane swaps inside the row (xor 8 = rotate by 8,
// xor 7 = half-row mirror, xor 2 and xor 1 = quad permutes).  Register j of
// lane c holds the partial of query row j ^ f(c), with f linear and chosen
// so that the half the partner gives away always holds the rows the lane
// keeps: no selects, RP - 1 + (4 - log2 RP) adds per key instead of 4 RP.
// Lane c ends with the score of row f(c).
// Softmax.  Per row over the wave: a row's scores sit in its lanes' KPL
// registers and in the wave's four DPP rows (xor 16 / 32 permlane swaps).
// P.V.  The weights are gathered back over the 16 lanes (the reverse
// butterfly, RP - 1 moves), so every lane holds all rows' weights of its key
// and accumulates RP rows of its 16-byte slice of V, in its permuted row
// order; the wave's four DPP rows (four keys per load) are then summed by a
// reduce-scatter with the gfx950 permlane32 / permlane16 swaps, each row
// keeping a quarter of the accumulators.  With 8 fp32 rows the product runs
// on the matrix cores instead: the contiguous V slices are already the A
// operand of v_mfma_f32_16x16x4f32 with the four keys of a load as the
// contraction, and each lane's own weight is its B element, so neither the
// gather nor the cross-row sum is needed.
// Merge.  The four waves through LDS, then as in the other split kernels:
// the output directly for a single split, else (max, sum, partial output)
// per row into the workspace for the combine.
//   decode_rows_loop_kernel (below) runs the same rows with one workgroup per
// KV head over the whole key range, for calls whose heads about fill the GPU.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Partner of butterfly step S inside a 16-lane row: lane c ^ 8, c ^ 7, c ^ 2,
// c ^ 1 (DPP row_ror:8, row_half_mirror, quad_perm [2,3,0,1], [1,0,3,2]).
// A key row of 16 lanes takes steps 0-3; one of 8 lanes (128-byte rows)
// takes steps 1-3, all of which stay inside its 8 lanes.
constexpr int kStepCtrl[4] = {kDppRowRor8, kDppHalfMirror, kDppQuadXor2, kDppQuadXor1};
template <int S>
__device__ __forceinline__ float step_partner(float x) {
  return dpp_mov<kStepCtrl[S]>(x);
}

// First butterfly step for key rows of LPR lanes.
template <int LPR>
constexpr int first_step() {
  return LPR == 16 ? 0 : 1;
}

// Row order of lane c: register j holds query row j ^ row_perm<RP, LPR>(c).
// Writing c in the basis {8, 7, 2, 1} of the step masks, c = a0*8 ^ a1*7 ^
// a2*2 ^ a3*1 with a0 = c3, a1 = c2, a2 = c1 ^ c2, a3 = c0 ^ c2, and
// f(c) = sum over the halving steps S (the first log2(RP) steps from
// first_step) of a_S * (RP >> (S - first + 1)).  Then f(c ^ mask_S) =
// f(c) ^ (RP >> (S - first + 1)) for a halving step (the partner's upper
// half holds this lane's lower-half rows) and f(c ^ mask_S) = f(c) for the
// steps after them (partners hold the same row).  With 8-lane rows c < 8,
// so a0 = 0 and step 0 is not taken.
template <int RP, int LPR>
__device__ __forceinline__ int row_perm(int c) {
  constexpr int F = first_step<LPR>();
  const int c3 = (c >> 3) & 1, c2 = (c >> 2) & 1, c1 = (c >> 1) & 1, c0 = c & 1;
  const int a[4] = {c3, c2, c1 ^ c2, c0 ^ c2};
  int f = 0;
#pragma unroll
  for (int s = F; (RP >> (s - F + 1)) > 0; ++s) f |= a[s] * (RP >> (s - F + 1));
  return f;
}

// Butterfly reduce-scatter of v[0 .. RP) over the LPR lanes of a key row,
// steps F .. 3; returns the full sum of row f(c).
template <int RP, int F, int S = F>
__device__ __forceinline__ float reduce_rows(float *v) {
  if constexpr (S == 4) {
    return v[0];
  } else {
    constexpr int n = RP >> (S - F);
    if constexpr (n >= 2) {
#pragma unroll
      for (int j = 0; j < n / 2; ++j) v[j] += step_partner<S>(v[j + n / 2]);
    } else {
      v[0] += step_partner<S>(v[0]);
    }
    return reduce_rows<RP, F, S + 1>(v);
  }
}

// Reverse butterfly: from u[0] = value of row f(c), fill u[0 .. RP) with the
// values of rows j ^ f(c) held by the other lanes of the key row (steps
// S down to F).
template <int RP, int F, int S>
__device__ __forceinline__ void gather_rows(float *u) {
  if constexpr (S >= F) {
    constexpr int n = RP >> (S - F + 1);
#pragma unroll
    for (int j = 0; j < n; ++j) u[j + n] = step_partner<S>(u[j]);
    gather_rows<RP, F, S - 1>(u);
  }
}

template <int RP>
constexpr int log2_of() {
  return RP == 2 ? 1 : RP == 4 ? 2 : RP == 8 ? 3 : 4;
}

// Sum of a and b's partners in the paired DPP rows: permlane32 pairs lanes
// l and l + 32 (rows 0-2, 1-3), permlane16 rows 0-1 and 2-3.  Swapping the
// upper half of a with the lower half of b and adding gives, in the lower
// half, a summed over the pair, and in the upper half, b summed over it.
template <int OFF>
__device__ __forceinline__ float swap_add(float a, float b) {
  const auto r = (OFF == 32)
                     ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                     : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K/V rows are read once per call: non-temporal loads, as in the single-row
// kernel.
__device__ __forceinline__ u32x4 stream_load(const u32x4 *p) { return __builtin_nontemporal_load(p); }

template <int DT, int LPR, int RP, int KPL, bool MPV, bool FUSED, bool PAGED, bool DEVLEN>
__global__ __launch_bounds__(256) void decode_rows_kernel(DecodeArgs a) {
  constexpr int EV = Dtype<DT>::kPer16B;  // elements per 16-byte vector
  constexpr int D = LPR * EV;             // LPR * 16-byte rows
  constexpr int F = first_step<LPR>();    // first butterfly step
  constexpr int NRG = 256 / LPR;          // key rows per workgroup load
  constexpr int SPLIT = NRG * KPL;        // keys per workgroup
  constexpr int NV = RP * EV;             // accumulators per lane
  static_assert(LPR == 8 || LPR == 16, "key row width");
  static_assert(RP >= 2 && RP <= 16 && (RP & (RP - 1)) == 0, "rows");
  static_assert(!MPV || (DT == KVC_F32 && RP == 8 && LPR == 16), "matrix-core P.V: fp32, 8 rows");

  __shared__ float sh_o[4][RP * D];
  __shared__ float sh_m[4][RP], sh_l[4][RP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & (LPR - 1);  // 16-byte slice of the key row
  const int kg = lane / LPR;       // key row within the wave load
  const int rg = tid / LPR;        // key row within a workgroup load

  // Grid: x = (layer, KV head), y = split, z = sequence in the batch slice.
  // With the head count a multiple of 8 every split of one head runs on the
  // same XCD (workgroups are dealt round-robin to the 8 XCDs), and the
  // workgroups past a short sequence's last split sit together at the end
  // of its slice (batched GQA decode 36.0 -> 35.2 us against split-major).
  const int lh = blockIdx.x;
  const int split = blockIdx.y;
  const int bb = blockIdx.z;
  const int P = seq_hist<DEVLEN>(a, bb);
  const int Hkv = a.Hkv, B = a.B, Tmax = a.Tmax, layer0 = a.layer0, N = a.N, rows = a.rows;
  const int Hq = a.Hq;
  const uint32_t hkv_div = a.hkv_div;
  asm volatile("" ::"s"(P), "s"(Hkv), "s"(B), "s"(Tmax), "s"(layer0), "s"(N), "s"(rows), "s"(Hq),
               "s"(hkv_div));
  const int nkeys = P + N;
  const int nsplit = (nkeys + SPLIT - 1) / SPLIT;
  if (split >= nsplit) return;
  const int l = div_magic(lh, Hkv, hkv_div);
  const int hkv = lh - l * Hkv;
  const int b = a.b0 + bb;

  const size_t crow0 = (((size_t)(layer0 + l) * B + b) * Hkv + hkv) * (size_t)Tmax;
  const char *kc = a.k_cache + crow0 * (LPR * 16);
  const char *vc = a.v_cache + crow0 * (LPR * 16);
  const size_t nrow0 = (((size_t)l * B + b) * Hkv + hkv) * (size_t)N;
  // Query rows of this (layer, sequence, KV head): rr = g * N + i, contiguous.
  const long long qrow0 = (((long long)l * B + b) * Hq + (long long)hkv * a.group) * N;

  // This lane's row order, and the last key its own row f(c) may see (-1 for
  // padding rows: nothing visible).
  const int f = row_perm<RP, LPR>(c);
  const int lim = f < rows ? P + f % N : -1;

  // 1. Query slices (row j ^ f; padding rows read the last real row), then
  //    every K and V load of the split.
  u32x4 qw[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int rr = j ^ f;
    qw[j] = reinterpret_cast<const u32x4 *>(a.q)[(qrow0 + (rr < rows ? rr : rows - 1)) * LPR + c];
  }
  const int key0 = split * SPLIT;
  u32x4 kw[KPL], vw[KPL];
  size_t prow[KPL];
  if constexpr (PAGED) {
    if (a.pg.bs_log2 >= (LPR == 16 ? 4 : 5)) {
      // blocks of at least NRG positions: one scalar id lookup per load
      paged_rows_grouped<KPL, NRG>(a.pg, b, key0, nkeys - 1, rg, layer0 + l, hkv, Hkv, prow);
    } else {
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int key = key0 + kk * NRG + rg;
        prow[kk] = paged_row(a.pg, b, key < nkeys ? key : nkeys - 1, layer0 + l, hkv, Hkv);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    const int key = key0 + kk * NRG + rg;
    const int kidx = key < nkeys ? key : nkeys - 1;
    const u32x4 *kp, *vp;
    if (FUSED && kidx >= P) {
      kp = reinterpret_cast<const u32x4 *>(a.k_new) + (nrow0 + (kidx - P)) * LPR + c;
      vp = reinterpret_cast<const u32x4 *>(a.v_new) + (nrow0 + (kidx - P)) * LPR + c;
    } else if constexpr (PAGED) {
      kp = reinterpret_cast<const u32x4 *>(a.k_cache) + prow[kk] * LPR + c;
      vp = reinterpret_cast<const u32x4 *>(a.v_cache) + prow[kk] * LPR + c;
    } else {
      const uint32_t off = (uint32_t)(kidx * LPR + c) * 16u;
      kp = reinterpret_cast<const u32x4 *>(kc + off);
      vp = reinterpret_cast<const u32x4 *>(vc + off);
    }
    kw[kk] = stream_load(kp);
    vw[kk] = stream_load(vp);
  }
  __builtin_amdgcn_sched_barrier(0);

  // Fused step: the workgroup holding keys [P, P + N) writes them to their
  // cache slots (no workgroup reads those slots during the call).
  if constexpr (FUSED) {
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      const int key = key0 + kk * NRG + rg;
      if (key >= P && key < nkeys) {
        u32x4 *kd, *vd;
        if constexpr (PAGED) {
          kd = reinterpret_cast<u32x4 *>(a.k_cache) + prow[kk] * LPR + c;
          vd = reinterpret_cast<u32x4 *>(a.v_cache) + prow[kk] * LPR + c;
        } else {
          kd = reinterpret_cast<u32x4 *>(a.k_cache) + (crow0 + key) * LPR + c;
          vd = reinterpret_cast<u32x4 *>(a.v_cache) + (crow0 + key) * LPR + c;
        }
        *kd = kw[kk];
        *vd = vw[kk];
      }
    }
  }

  // 2. Scores of row f in the log2 domain, one per key load.
  float s[KPL];
  {
    float qf[RP][EV];
#pragma unroll
    for (int j = 0; j < RP; ++j) unpack16<DT>(qw[j], qf[j]);
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      float kf[EV];
      unpack16<DT>(kw[kk], kf);
      float part[RP];
#pragma unroll
      for (int j = 0; j < RP; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) d = fmaf(qf[j][e], kf[e], d);
        part[j] = d;
      }
      const float dot = reduce_rows<RP, F>(part);
      s[kk] = (key0 + kk * NRG + rg <= lim) ? dot * a.scale_log2 : kNegInf;
    }
  }

  // 3. Row max over the wave, weights, row sums.
  float m = s[0];
#pragma unroll
  for (int kk = 1; kk < KPL; ++kk) m = fmaxf(m, s[kk]);
  if constexpr (LPR == 8) m = xor_combine<8, true>(m);
  m = xor_combine<16, true>(m);
  m = xor_combine<32, true>(m);
  float lsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    s[kk] = (m == kNegInf) ? 0.f : fast_exp2(s[kk] - m);
    lsum += s[kk];
  }
  if constexpr (LPR == 8) lsum = xor_combine<8>(lsum);
  lsum = xor_combine<16>(lsum);
  lsum = xor_combine<32>(lsum);

  // 4. P.V summed over the wave, into this wave's LDS slice.
  if constexpr (MPV) {
    // On the matrix cores: per key load, O^T[d][col] += sum over the load's
    // four keys k of V[k][d] P[row f(col)][k], v_mfma_f32_16x16x4f32 with
    // A[i][k] = V[key k][4 i + t] (lane (i, k) = (c, kg): element t of its
    // own V slice) and B[k][col] = the weight lane (col, k) holds.  Lane
    // (c, kg) ends with row f(c), elements d = 16 kg + 4 r + t.
    f32x4 acc4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      float vf[EV];
      unpack16<DT>(vw[kk], vf);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc4[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[t], s[kk], acc4[t], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4 *>(&sh_o[wave][f * D + 16 * kg + 4 * r]) =
          f32x4{acc4[0][r], acc4[1][r], acc4[2][r], acc4[3][r]};
  } else {
    // On the vector ALUs: weights gathered over the key row, acc[j][e] =
    // row j ^ f, element c * EV + e; then summed over the wave's key rows --
    // for 8-lane rows first the two halves of each DPP row (all values),
    // then over the four DPP rows, lane (c, kg) of DPP row q = kg * LPR / 16
    // keeping accumulators [q * NV / 4, (q + 1) * NV / 4).
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      float u[RP];
      u[0] = s[kk];
      gather_rows<RP, F, F + log2_of<RP>() - 1>(u);
      float vf[EV];
      unpack16<DT>(vw[kk], vf);
#pragma unroll
      for (int j = 0; j < RP; ++j)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[j * EV + e] = fmaf(u[j], vf[e], acc[j * EV + e]);
    }
    if constexpr (LPR == 8) {
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = xor_combine<8>(acc[i]);
    }
    float half[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) half[i] = swap_add<32>(acc[i], acc[i + NV / 2]);
    const int q = lane >> 4;  // DPP row
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      const int idx = q * (NV / 4) + i;
      const int j = idx / EV, e = idx % EV;
      const float v = swap_add<16>(half[i], half[i + NV / 4]);
      // both 8-lane halves of a DPP row hold the same sums: one writes
      if (LPR == 16 || (kg & 1) == 0) sh_o[wave][(j ^ f) * D + c * EV + e] = v;
    }
  }

  // 5. Merge the four waves; write the output or the split state.
  if (kg == 0) {
    sh_m[wave][f] = m;
    sh_l[wave][f] = lsum;
  }
  __syncthreads();

  // Four consecutive elements per thread: 16-byte state stores (streaming
  // them past the caches as non-temporal stores measured slower).
  for (int t = tid; t < rows * (D / 4); t += 256) {
    const int r = t / (D / 4);
    const int d = (t % (D / 4)) * 4;
    float M = sh_m[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh_m[w][r]);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float fw = rescale(sh_m[w][r], M);
      o += fw * *reinterpret_cast<const f32x4 *>(&sh_o[w][r * D + d]);
      L = fmaf(fw, sh_l[w][r], L);
    }
    const long long row = qrow0 + r;
    if (nsplit == 1) {
      const float inv = 1.f / L;
      const float val[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      store_elems<DT>(a.o, (size_t)row * D + d, val, 4);
    } else {
      const size_t ws = ws_slot(a, row, split);
      *reinterpret_cast<f32x4 *>(a.ws_o + ws * D + d) = o;
      if (d == 0) {
        a.ws_ml[ws * 2] = M;
        a.ws_ml[ws * 2 + 1] = L;
      }
    }
  }
}

// The same rows, one workgroup per (layer, sequence, KV head) streaming the
// whole key range [0, P + N), for calls whose KV heads alone about fill the
// chip (the 12-layer chunked step has 144).  Chunks of NRG * KPL keys are
// laid out as one split above and go two register buffers deep (the next
// chunk's loads in flight while the current one is reduced, two chunks per
// loop trip with no branch inside: a chunk past the end is clamped to the
// last key and masked).  Per query row the wave keeps a running max and sum
// (wave-uniform after the cross-lane reductions) and each lane its partial
// outputs; when a row's max grows, its partial outputs are rescaled by
// 2^(m_old - m_new) -- on the matrix-core path a lane's accumulators all
// belong to its own row f(c), on the vector path lane c holds rows j ^ f(c)
// and gathers their factors over the key row with the reverse butterfly.
// The sums over the wave's key rows and the merge of the waves run once,
// after the last chunk, and the output is written directly: no split
// states, no combine pass.
// Block ids of one sequence the paged loop kernel stages in LDS (8 KB).
constexpr int kRowsLoopMaxBlocks = 2048;

template <int DT, int LPR, int RP, int KPL, int NT, bool MPV, bool FUSED, bool PAGED, bool DEVLEN>
__global__ __launch_bounds__(NT) void decode_rows_loop_kernel(DecodeArgs a) {
  constexpr int EV = Dtype<DT>::kPer16B;
  constexpr int D = LPR * EV;
  constexpr int F = first_step<LPR>();
  constexpr int NW = NT / 64;
  constexpr int NRG = NT / LPR;
  constexpr int CH = NRG * KPL;
  constexpr int NV = RP * EV;
  static_assert(LPR == 8 || LPR == 16, "key row width");
  static_assert(RP >= 2 && RP <= 16 && (RP & (RP - 1)) == 0, "rows");
  static_assert(!MPV || (DT == KVC_F32 && RP == 8 && LPR == 16), "matrix-core P.V: fp32, 8 rows");

  __shared__ float sh_o[NW][RP * D];
  __shared__ float sh_m[NW][RP], sh_l[NW][RP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & (LPR - 1);
  const int kg = lane / LPR;
  const int rg = tid / LPR;

  const int lh = blockIdx.x;
  const int bb = blockIdx.z;
  const int P = seq_hist<DEVLEN>(a, bb);
  const int Hkv = a.Hkv, B = a.B, Tmax = a.Tmax, layer0 = a.layer0, N = a.N, rows = a.rows;
  const int Hq = a.Hq;
  const uint32_t hkv_div = a.hkv_div;
  const float scale_log2 = a.scale_log2;
  asm volatile("" ::"s"(P), "s"(Hkv), "s"(B), "s"(Tmax), "s"(layer0), "s"(N), "s"(rows), "s"(Hq),
               "s"(hkv_div), "s"(scale_log2));
  const int nkeys = P + N;
  const int nch = (nkeys + CH - 1) / CH;
  const int l = div_magic(lh, Hkv, hkv_div);
  const int hkv = lh - l * Hkv;
  const int b = a.b0 + bb;

  const size_t crow0 = (((size_t)(layer0 + l) * B + b) * Hkv + hkv) * (size_t)Tmax;
  const char *kc = a.k_cache + crow0 * (LPR * 16);
  const char *vc = a.v_cache + crow0 * (LPR * 16);
  const size_t nrow0 = (((size_t)l * B + b) * Hkv + hkv) * (size_t)N;
  const long long qrow0 = (((long long)l * B + b) * Hq + (long long)hkv * a.group) * N;

  const int f = row_perm<RP, LPR>(c);
  const int lim = f < rows ? P + f % N : -1;

  u32x4 qw[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int rr = j ^ f;
    qw[j] = reinterpret_cast<const u32x4 *>(a.q)[(qrow0 + (rr < rows ? rr : rows - 1)) * LPR + c];
  }

  // A paged cache's block ids of this sequence, staged in LDS once (the host
  // sends tables longer than kRowsLoopMaxBlocks to the split kernel).
  __shared__ int32_t sh_blk[PAGED ? kRowsLoopMaxBlocks : 1];
  if constexpr (PAGED) {
    const int bsl = a.pg.bs_log2;
    const int nblk = (nkeys + (1 << bsl) - 1) >> bsl;
    const int32_t *tbl = a.pg.block_table + (size_t)b * a.pg.max_blocks;
    for (int i = tid; i < nblk; i += NT) {
      const int blk = tbl[i];
      sh_blk[i] = blk < 0 ? 0 : (blk >= a.pg.num_blocks ? a.pg.num_blocks - 1 : blk);
    }
    __syncthreads();
  }

  // Chunk ch's K loads, then its V loads; keys past the last clamped to it,
  // keys [P, P + N) from the new rows in the fused step.
  auto load_chunk = [&](int ch, u32x4 (&kw)[KPL], u32x4 (&vw)[KPL]) {
    const int key0 = ch * CH;
    size_t prow[KPL];
    if constexpr (PAGED) {
      const int bsl = a.pg.bs_log2;
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int pos0 = key0 + kk * NRG + rg;
        const int pos = pos0 < nkeys - 1 ? pos0 : nkeys - 1;
        prow[kk] = ((((size_t)(layer0 + l) * a.pg.num_blocks + sh_blk[pos >> bsl]) * Hkv + hkv) << bsl) +
                   (size_t)(pos & ((1 << bsl) - 1));
      }
    }
    const u32x4 *vp[KPL];
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      const int key = key0 + kk * NRG + rg;
      const int kidx = key < nkeys ? key : nkeys - 1;
      const u32x4 *kp;
      if (FUSED && kidx >= P) {
        kp = reinterpret_cast<const u32x4 *>(a.k_new) + (nrow0 + (kidx - P)) * LPR + c;
        vp[kk] = reinterpret_cast<const u32x4 *>(a.v_new) + (nrow0 + (kidx - P)) * LPR + c;
      } else if constexpr (PAGED) {
        kp = reinterpret_cast<const u32x4 *>(a.k_cache) + prow[kk] * LPR + c;
        vp[kk] = reinterpret_cast<const u32x4 *>(a.v_cache) + prow[kk] * LPR + c;
      } else {
        const uint32_t off = (uint32_t)(kidx * LPR + c) * 16u;
        kp = reinterpret_cast<const u32x4 *>(kc + off);
        vp[kk] = reinterpret_cast<const u32x4 *>(vc + off);
      }
      kw[kk] = stream_load(kp);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) vw[kk] = stream_load(vp[kk]);
  };

  float qf[RP][EV];
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc4[4];
  float acc[MPV ? 1 : NV];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (MPV ? 1 : NV); ++i) acc[i] = 0.f;

  auto reduce_chunk = [&](int ch, const u32x4 (&kw)[KPL], const u32x4 (&vw)[KPL]) {
    const int key0 = ch * CH;
    float s[KPL];
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      float kf[EV];
      unpack16<DT>(kw[kk], kf);
      float part[RP];
#pragma unroll
      for (int j = 0; j < RP; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) d = fmaf(qf[j][e], kf[e], d);
        part[j] = d;
      }
      const float dot = reduce_rows<RP, F>(part);
      s[kk] = (key0 + kk * NRG + rg <= lim) ? dot : kNegInf;
    }
    float mc = s[0];
#pragma unroll
    for (int kk = 1; kk < KPL; ++kk) mc = fmaxf(mc, s[kk]);
    if constexpr (LPR == 8) mc = xor_combine<8, true>(mc);
    mc = xor_combine<16, true>(mc);
    mc = xor_combine<32, true>(mc);
    const float mn = fmaxf(m_run, mc);
    const float fac = rescale(m_run, mn);
    float lc = 0.f;
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      s[kk] = (mn == kNegInf) ? 0.f : fast_exp2(s[kk] - mn);
      lc += s[kk];
    }
    if constexpr (LPR == 8) lc = xor_combine<8>(lc);
    lc = xor_combine<16>(lc);
    lc = xor_combine<32>(lc);
    l_run = fmaf(l_run, fac, lc);
    m_run = mn;
    if constexpr (MPV) {
#pragma unroll
      for (int t = 0; t < 4; ++t) acc4[t] *= fac;
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        float vf[EV];
        unpack16<DT>(vw[kk], vf);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc4[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[t], s[kk], acc4[t], 0, 0, 0);
      }
    } else {
      float fr[RP];
      fr[0] = fac;
      gather_rows<RP, F, F + log2_of<RP>() - 1>(fr);
#pragma unroll
      for (int j = 0; j < RP; ++j)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[j * EV + e] *= fr[j];
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        float u[RP];
        u[0] = s[kk];
        gather_rows<RP, F, F + log2_of<RP>() - 1>(u);
        float vf[EV];
        unpack16<DT>(vw[kk], vf);
#pragma unroll
        for (int j = 0; j < RP; ++j)
#pragma unroll
          for (int e = 0; e < EV; ++e) acc[j * EV + e] = fmaf(u[j], vf[e], acc[j * EV + e]);
      }
    }
  };

  {
    u32x4 kA[KPL], vA[KPL], kB[KPL], vB[KPL];
    load_chunk(0, kA, vA);
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      unpack16<DT>(qw[j], qf[j]);
#pragma unroll
      for (int e = 0; e < EV; ++e) qf[j][e] *= scale_log2;
    }
    for (int ch = 0; ch < nch; ch += 2) {
      load_chunk(ch + 1, kB, vB);
      __builtin_amdgcn_sched_barrier(0);
      reduce_chunk(ch, kA, vA);
      load_chunk(ch + 2, kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      reduce_chunk(ch + 1, kB, vB);
    }
  }

  // Fused step: the new rows to their cache slots, after the loop so that no
  // store sits in it (no workgroup reads those slots during the call).
  if constexpr (FUSED) {
    if (tid < N * LPR) {  // N * LPR <= 8 * 16 <= NT
      const int i = tid / LPR, cc = tid % LPR;
      const u32x4 kv = reinterpret_cast<const u32x4 *>(a.k_new)[(nrow0 + i) * LPR + cc];
      const u32x4 vv = reinterpret_cast<const u32x4 *>(a.v_new)[(nrow0 + i) * LPR + cc];
      const size_t dst = PAGED ? paged_row(a.pg, b, P + i, layer0 + l, hkv, Hkv) : crow0 + P + i;
      reinterpret_cast<u32x4 *>(a.k_cache)[dst * LPR + cc] = kv;
      reinterpret_cast<u32x4 *>(a.v_cache)[dst * LPR + cc] = vv;
    }
  }
  // Sums over the wave's key rows into this wave's LDS slice, as in the
  // split kernel, then the merge of the waves and the output.
  if constexpr (MPV) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4 *>(&sh_o[wave][f * D + 16 * kg + 4 * r]) =
          f32x4{acc4[0][r], acc4[1][r], acc4[2][r], acc4[3][r]};
  } else {
    if constexpr (LPR == 8) {
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = xor_combine<8>(acc[i]);
    }
    float half[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) half[i] = swap_add<32>(acc[i], acc[i + NV / 2]);
    const int q = lane >> 4;
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      const int idx = q * (NV / 4) + i;
      const int j = idx / EV, e = idx % EV;
      const float v = swap_add<16>(half[i], half[i + NV / 4]);
      if (LPR == 16 || (kg & 1) == 0) sh_o[wave][(j ^ f) * D + c * EV + e] = v;
    }
  }
  if (kg == 0) {
    sh_m[wave][f] = m_run;
    sh_l[wave][f] = l_run;
  }
  __syncthreads();
  for (int t = tid; t < rows * (D / 4); t += NT) {
    const int r = t / (D / 4);
    const int d = (t % (D / 4)) * 4;
    float M = sh_m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sh_m[w][r]);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float fw = rescale(sh_m[w][r], M);
      o += fw * *reinterpret_cast<const f32x4 *>(&sh_o[w][r * D + d]);
      L = fmaf(fw, sh_l[w][r], L);
    }
    const float inv = 1.f / L;
    const float val[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    store_elems<DT>(a.o, (size_t)(qrow0 + r) * D + d, val, 4);
  }
}

constexpr int kRowsLoopThreads = 256;

template <int DT, int LPR, int RP>
hipError_t launch_loop_rp(const DecodeArgs &a, bool fused, hipStream_t s) {
  constexpr bool MPV = DT == KVC_F32 && RP == 8 && LPR == 16;
  // 4 keys per lane group and chunk: chunked step 17.2 us against 17.9 at 8,
  // 18.1 at 3, 20.1 at 2 (a shorter last chunk, fewer registers)
  constexpr int KPL = 4;
  constexpr int NT = kRowsLoopThreads;
  const dim3 grid((unsigned)(a.n_layers * a.Hkv), 1u, (unsigned)a.nb);
  const bool paged = a.pg.block_table != nullptr;
  if (paged && a.pg.max_blocks > kRowsLoopMaxBlocks) return hipErrorInvalidValue;
  if (a.hist_dev) {
    if (!fused) return hipErrorInvalidValue;  // device lengths: the fused step only
    if (paged)
      hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, true, true, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, true, false, true>), grid, dim3(NT), 0, s, a);
  } else if (fused && paged)
    hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, true, true, false>), grid, dim3(NT), 0, s, a);
  else if (fused)
    hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, true, false, false>), grid, dim3(NT), 0, s, a);
  else if (paged)
    hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, false, true, false>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((decode_rows_loop_kernel<DT, LPR, RP, KPL, NT, MPV, false, false, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int DT, int LPR>
hipError_t launch_loop_dt(const DecodeArgs &a, bool fused, hipStream_t s) {
  if (a.rows <= 2) return launch_loop_rp<DT, LPR, 2>(a, fused, s);
  if (a.rows <= 4) return launch_loop_rp<DT, LPR, 4>(a, fused, s);
  if constexpr (DT == KVC_BF16 || LPR == 16) return launch_loop_rp<DT, LPR, 8>(a, fused, s);
  return hipErrorInvalidValue;
}

// Keys each lane group loads per split (a split covers 256 / LPR times as
// many): 8 measured best for the chunked fp32 and the bf16 GQA decode
// workloads (2, 4, 6, 12 and 16 were slower or equal).
constexpr int kRowsKpl = 8;

template <int DT, int LPR, int RP>
hipError_t launch_rp(const DecodeArgs &a, int splits, bool fused, hipStream_t s) {
  // P.V of 8 fp32 rows on the matrix cores (the vector-ALU form measured equal)
  constexpr bool MPV = DT == KVC_F32 && RP == 8 && LPR == 16;
  const dim3 grid((unsigned)(a.n_layers * a.Hkv), (unsigned)splits, (unsigned)a.nb);
  const bool paged = a.pg.block_table != nullptr;
  if (a.hist_dev) {
    if (!fused) return hipErrorInvalidValue;  // device lengths: the fused step only
    if (paged)
      hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, true, true, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, true, false, true>), grid, dim3(256), 0, s, a);
  } else if (fused && paged)
    hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, true, true, false>), grid, dim3(256), 0, s, a);
  else if (fused)
    hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, true, false, false>), grid, dim3(256), 0, s, a);
  else if (paged)
    hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, false, true, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_rows_kernel<DT, LPR, RP, kRowsKpl, MPV, false, false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int LPR>
hipError_t launch_dt(const DecodeArgs &a, int splits, bool fused, hipStream_t s) {
  if (a.rows <= 2) return launch_rp<DT, LPR, 2>(a, splits, fused, s);
  if (a.rows <= 4) return launch_rp<DT, LPR, 4>(a, splits, fused, s);
  if constexpr (DT == KVC_BF16 || LPR == 16) return launch_rp<DT, LPR, 8>(a, splits, fused, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_rows_fits(int dtype, int D, int rows) {
  if (rows < 2) return false;
  if (dtype == KVC_F32) return D == 64 && rows <= 8;
  return (D == 128 || D == 64) && rows <= 8;
}

int decode_rows_split_keys(int dtype, int D) {
  const int lpr = D * (dtype == KVC_BF16 ? 2 : 4) / 16;
  return (256 / lpr) * kRowsKpl;
}

hipError_t launch_decode_rows(const DecodeArgs &a, int dtype, int D, int splits, bool fused,
                              hipStream_t s) {
  if (!decode_rows_fits(dtype, D, a.rows) || a.row_tiles != 1) return hipErrorInvalidValue;
  if (dtype == KVC_F32) return launch_dt<KVC_F32, 16>(a, splits, fused, s);
  return D == 128 ? launch_dt<KVC_BF16, 16>(a, splits, fused, s)
                  : launch_dt<KVC_BF16, 8>(a, splits, fused, s);
}

hipError_t launch_decode_rows_loop(const DecodeArgs &a, int dtype, int D, bool fused, hipStream_t s) {
  if (!decode_rows_fits(dtype, D, a.rows) || a.row_tiles != 1) return hipErrorInvalidValue;
  if (dtype == KVC_F32) return launch_loop_dt<KVC_F32, 16>(a, fused, s);
  return D == 128 ? launch_loop_dt<KVC_BF16, 16>(a, fused, s) : launch_loop_dt<KVC_BF16, 8>(a, fused, s);
}

int decode_rows_loop_max_blocks() { return kRowsLoopMaxBlocks; }

}  // namespace kvc
