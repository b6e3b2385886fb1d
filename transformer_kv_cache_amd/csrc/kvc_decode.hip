// kvc_decode.hip -- split-K ("flash-decode") attention of N new query rows
// against the KV cache.
//
// What it computes ([KV-4] jennyma11.github.io/infra/ch07-01.html, "Decode
// 阶段", listing 1-2; [KV-2] openai-hub.com/news/2435, "一个很容易漏掉的错误"):
// for each (layer, sequence b, query head, new row i) the softmax of
// scale * q . K_j over keys j = 0 .. P_b + i, applied to V.  Decode reads every
// cached K/V byte once and does ~1 flop per byte, so it is bound by HBM
// bandwidth ([KV-2] "千倍计算量为何只换来6倍速度").
//
// Work split.  This vector kernel serves the case of one query row per KV
// head (plain multi-head single-token decode); several rows per KV head (GQA
// groups, chunked decode) go to the matrix-core kernel in kvc_decode_mfma.hip.
// A workgroup (256 lanes, 4 waves) owns one (layer, sequence, KV head, split
// of SPLIT consecutive keys); the code is written for a tile of RT rows but
// instantiated with RT = 1.  Inside the workgroup:
//   * a key row of D elements is LPR = D*elem/16 lanes wide; each lane loads
//     one 16-byte vector of it (global_load_dwordx4).  Consecutive lane groups
//     take consecutive rows, so one wave-wide load covers 64*16 contiguous
//     bytes.  Every K and V load of the split is issued before any arithmetic
//     so the whole split is in flight at once.
//   * the dot product is a per-lane partial over its 16 bytes followed by a
//     butterfly across the LPR lanes of the row with DPP lane permutes
//     (quad_perm, row_half_mirror, row_mirror); no LDS traffic.
//   * each row group keeps a private softmax state (max, sum, partial P.V)
//     over its keys; the states are merged across the wave with cross-lane
//     exchanges and across the 4 waves through LDS, rescaling by exp2 of
//     the max difference (log2(e) is folded into the scale).
// Fused step.  kvc_decode_step also performs the append: keys at positions
// [P, P+N) are read straight from the new K/V rows instead of the cache, and
// the workgroups of row tile 0 that hold them write them to their cache slots.
// No workgroup reads those slots during the call, so the write is race-free,
// and the step needs no separate append launch.
// Combine.  With more than one split, each workgroup writes its (max, sum,
// P.V) state to the workspace and a second, small kernel merges the splits of
// every query row (rescaling by exp2 of the max difference) and writes the
// output; with a single split the workgroup writes the output itself.  The
// merge is a separate launch rather than a last-workgroup ticket: the ticket
// needs a device-scope release fence in every workgroup, which on gfx950 is an
// L2 write-back (buffer_wbl2), and that measured about ten times slower than
// the extra launch.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR lanes that hold one key row; every lane gets the total.
// Lane groups are aligned blocks of LPR lanes.  After the two quad steps a
// quad is uniform, so mirroring inside 8 (then 16) lanes pairs uniform blocks.
template <int LPR>
__device__ __forceinline__ float row_allreduce(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row width");
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  if (LPR >= 16) x += dpp_mov<kDppRowMirror>(x);
  if (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// K/V rows are read exactly once per call: non-temporal loads keep them from
// displacing reusable lines in the caches.
#ifndef KVC_DECODE_NONTEMPORAL
#define KVC_DECODE_NONTEMPORAL 1
#endif
__device__ __forceinline__ u32x4 stream_load(const u32x4 *p) {
#if KVC_DECODE_NONTEMPORAL
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Weight of a softmax state with max m when merged under a common max M.
__device__ __forceinline__ float rescale(float m, float M) {
  return m == kNegInf ? 0.f : fast_exp2(m - M);
}

template <int DT, int D, int RT, int KPL, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int EV = Dtype<DT>::kPer16B;        // elements per 16-byte vector
  constexpr int LPR = D * Dtype<DT>::kBytes / 16;  // lanes per key row
  constexpr int NRG = 256 / LPR;                 // key rows per wave-group load
  constexpr int SPLIT = NRG * KPL;               // keys per workgroup
  static_assert(LPR * EV == D, "row layout");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = tid / LPR;
  const int c = tid % LPR;

  // Grid: x = split, y = (layer, KV head, row tile), z = sequence in the
  // batch slice.  The sequence comes straight from blockIdx.z so its length
  // can be fetched while the other indices are still being computed.
  const int split = blockIdx.x;
  const int bb = blockIdx.z;
  const int P = a.hist[bb];
  const int rt = (RT == 1) ? 0 : (int)blockIdx.y % a.row_tiles;
  const int lh = (RT == 1) ? (int)blockIdx.y : (int)blockIdx.y / a.row_tiles;
  const int hkv = lh % a.Hkv;
  const int l = lh / a.Hkv;
  const int b = a.b0 + bb;
  const int nkeys = P + a.N;
  const int nsplit = (nkeys + SPLIT - 1) / SPLIT;
  if (split >= nsplit) return;
  const size_t crow0 = (((size_t)(a.layer0 + l) * a.B + b) * a.Hkv + hkv) * (size_t)a.Tmax;
  const long long qrow0 = (((long long)l * a.B + b) * a.Hq + (long long)hkv * a.group) * a.N;

  const int key0 = split * SPLIT;
  const u32x4 *kc = reinterpret_cast<const u32x4 *>(a.k_cache) + crow0 * LPR + c;
  const u32x4 *vc = reinterpret_cast<const u32x4 *>(a.v_cache) + crow0 * LPR + c;
  const size_t nrow0 = (((size_t)l * a.B + b) * a.Hkv + hkv) * (size_t)a.N * LPR + c;
  const u32x4 *kn = FUSED ? reinterpret_cast<const u32x4 *>(a.k_new) + nrow0 : nullptr;
  const u32x4 *vn = FUSED ? reinterpret_cast<const u32x4 *>(a.v_new) + nrow0 : nullptr;

  // 1. Issue the query loads and every K and V load of this split up front.
  //    Key indices past the sequence are clamped to its last row (always
  //    valid) so that no load sits behind a branch; their scores are masked.
  const int rr0 = rt * RT;
  u32x4 qw[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int rr = (rr0 + r < a.rows) ? rr0 + r : a.rows - 1;
    qw[r] = reinterpret_cast<const u32x4 *>(a.q)[(qrow0 + rr) * LPR + c];
  }
  u32x4 kw[KPL], vw[KPL];
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    const int key = key0 + kk * NRG + rg;
    const int kidx = key < nkeys ? key : nkeys - 1;
    const bool fresh = FUSED && kidx >= P;  // a new row: read it from k_new / v_new
    const size_t nidx = (size_t)(fresh ? kidx - P : 0);
    kw[kk] = stream_load(fresh ? kn + nidx * LPR : kc + (size_t)kidx * LPR);
    vw[kk] = stream_load(fresh ? vn + nidx * LPR : vc + (size_t)kidx * LPR);
  }
  // Keep the scheduler from interleaving arithmetic (and its waits) into the
  // load burst: all loads of the split are in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);

  // 2. Query fragments of the tile's rows (row rr = g*N + i of this KV head).
  float qf[RT][EV];
#pragma unroll
  for (int r = 0; r < RT; ++r) unpack16<DT>(qw[r], qf[r]);

  // 3. Scores in the log2 domain, masked keys at -inf.
  float s[RT][KPL];
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    float kf[EV];
    unpack16<DT>(kw[kk], kf);
    const int key = key0 + kk * NRG + rg;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EV; ++e) dot = fmaf(qf[r][e], kf[e], dot);
      dot = row_allreduce<LPR>(dot);
      const int i = (rr0 + r) % a.N;
      const bool visible = (key < nkeys) && (key <= P + i) && (rr0 + r < a.rows);
      s[r][kk] = visible ? dot * a.scale_log2 : kNegInf;
    }
  }

  // 4. Per-row-group softmax state over its KPL keys.
  float m[RT], lsum[RT], acc[RT][EV];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float mx = s[r][0];
#pragma unroll
    for (int kk = 1; kk < KPL; ++kk) mx = fmaxf(mx, s[r][kk]);
    m[r] = mx;
    lsum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[r][e] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    float vf[EV];
    unpack16<DT>(vw[kk], vf);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float p = (m[r] == kNegInf) ? 0.f : fast_exp2(s[r][kk] - m[r]);
      lsum[r] += p;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[r][e] = fmaf(p, vf[e], acc[r][e]);
    }
  }

  // 5. Merge the row groups of this wave (lanes with the same c).
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float M = m[r];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = rescale(m[r], M);
    lsum[r] *= f;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[r][e] *= f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      lsum[r] += __shfl_xor(lsum[r], off);
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[r][e] += __shfl_xor(acc[r][e], off);
    }
    m[r] = M;
  }

  // Fused step: row tile 0 writes the new rows it holds into their slots.
  if constexpr (FUSED) {
    if (rt == 0) {
      u32x4 *kd = reinterpret_cast<u32x4 *>(a.k_cache) + crow0 * LPR + c;
      u32x4 *vd = reinterpret_cast<u32x4 *>(a.v_cache) + crow0 * LPR + c;
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int key = key0 + kk * NRG + rg;
        if (key >= P && key < nkeys) {
          kd[(size_t)key * LPR] = kw[kk];
          vd[(size_t)key * LPR] = vw[kk];
        }
      }
    }
  }

  // 6. Merge the four waves through LDS.
  __shared__ float sh_o[4][RT][D];
  __shared__ float sh_m[4][RT];
  __shared__ float sh_l[4][RT];
  if (lane < LPR) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int e = 0; e < EV; ++e) sh_o[wave][r][c * EV + e] = acc[r][e];
      if (c == 0) {
        sh_m[wave][r] = m[r];
        sh_l[wave][r] = lsum[r];
      }
    }
  }
  __syncthreads();

  for (int t = tid; t < RT * D; t += 256) {
    const int r = t / D;
    const int d = t % D;
    if (rr0 + r >= a.rows) continue;
    float M = sh_m[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh_m[w][r]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = rescale(sh_m[w][r], M);
      o = fmaf(f, sh_o[w][r][d], o);
      L = fmaf(f, sh_l[w][r], L);
    }
    const long long row = qrow0 + rr0 + r;
    if (nsplit == 1) {
      const float val = o / L;
      store_elems<DT>(a.o, (size_t)row * D + d, &val, 1);
    } else {
      const size_t ws = (size_t)row * a.max_splits + split;
      a.ws_o[ws * D + d] = o;
      if (d == 0) {
        a.ws_ml[ws * 2] = M;
        a.ws_ml[ws * 2 + 1] = L;
      }
    }
  }
}

// Merge of the split-K states of every query row whose sequence needed more
// than one split: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  D lanes
// per row, one output element per lane.  Splits are read in chunks of 8 with
// every load of a chunk issued before any is used (indices clamped, extra
// splits masked), merged online across chunks.
// Merge of one query row's split states, element d of the output row.
// Splits are read in chunks of 16 with every load of a chunk issued before any
// is used (indices clamped, extra splits masked), merged online across chunks.
template <int DT, int D>
__device__ __forceinline__ void combine_row(const DecodeArgs &a, long long row, int nsplit, int d) {
  constexpr int CH = 16;
  const size_t ws0 = (size_t)row * a.max_splits;
  float M = kNegInf, o = 0.f, L = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += CH) {
    float mv[CH], lv[CH], ov[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int sp = (s0 + j < nsplit) ? s0 + j : nsplit - 1;
      mv[j] = a.ws_ml[(ws0 + sp) * 2];
      lv[j] = a.ws_ml[(ws0 + sp) * 2 + 1];
      ov[j] = a.ws_o[(ws0 + sp) * D + d];
    }
    __builtin_amdgcn_sched_barrier(0);
    float Mc = M;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (s0 + j >= nsplit) mv[j] = kNegInf;
      Mc = fmaxf(Mc, mv[j]);
    }
    const float fr = rescale(M, Mc);
    o *= fr;
    L *= fr;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float f = rescale(mv[j], Mc);
      o = fmaf(f, ov[j], o);
      L = fmaf(f, lv[j], L);
    }
    M = Mc;
  }
  const float val = o / L;
  store_elems<DT>(a.o, (size_t)row * D + d, &val, 1);
}

// Merge of the split-K states of every query row whose sequence needed more
// than one split: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  D lanes
// per row, one output element per lane.
template <int DT, int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int RPW = 256 / D;  // rows per workgroup
  const int d = threadIdx.x % D;
  const long long t = (long long)blockIdx.x * RPW + threadIdx.x / D;  // (l, bb, hq, i)
  const long long rows_here = (long long)a.n_layers * a.nb * a.Hq * a.N;
  if (t >= rows_here) return;
  const int i = (int)(t % a.N);
  const int hq = (int)((t / a.N) % a.Hq);
  const int bb = (int)((t / ((long long)a.N * a.Hq)) % a.nb);
  const int l = (int)(t / ((long long)a.N * a.Hq * a.nb));
  const int b = a.b0 + bb;
  const int nsplit = (a.hist[bb] + a.N + a.split_keys - 1) / a.split_keys;
  if (nsplit <= 1) return;  // written by the split kernel
  combine_row<DT, D>(a, (((long long)l * a.B + b) * a.Hq + hq) * a.N + i, nsplit, d);
}

// Keys each lane group loads per split: a split covers 256 / LPR * this many
// keys (64 for fp32 D=64).  Build-time tuning constant; 4 measured best
// across the fp32, bf16 and GQA decode workloads.
#ifndef KVC_DECODE_KEYS_PER_LANE
#define KVC_DECODE_KEYS_PER_LANE 4
#endif
constexpr int kKeysPerLane = KVC_DECODE_KEYS_PER_LANE;

template <int DT, int D, int RT>
hipError_t launch_one(const DecodeArgs &a, int splits, bool fused, hipStream_t s) {
  const dim3 grid((unsigned)splits, (unsigned)(a.n_layers * a.Hkv * a.row_tiles), (unsigned)a.nb);
  if (fused)
    hipLaunchKernelGGL((decode_kernel<DT, D, RT, kKeysPerLane, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, RT, kKeysPerLane, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Several query rows per KV head run on the matrix-core kernel, so the vector
// kernel is instantiated for one row per workgroup only.
template <int DT, int D>
hipError_t launch_rt(const DecodeArgs &a, int /*rt*/, int splits, bool fused, hipStream_t s) {
  return launch_one<DT, D, 1>(a, splits, fused, s);
}

}  // namespace

int decode_row_tile(int /*rows*/) { return 1; }

int decode_split_keys(int dtype, int D) {
  const int lpr = D * (dtype == KVC_BF16 ? 2 : 4) / 16;
  return (256 / lpr) * kKeysPerLane;
}

hipError_t launch_combine(const DecodeArgs &a, int dtype, int D, hipStream_t s) {
  const long long rows = (long long)a.n_layers * a.nb * a.Hq * a.N;
  const long long blocks = (rows + 256 / D - 1) / (256 / D);
  const dim3 grid((unsigned)blocks);
  if (dtype == KVC_F32) {
    if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_F32, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<KVC_F32, 128>), grid, dim3(256), 0, s, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_BF16, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<KVC_BF16, 128>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int D, int row_tile, int splits,
                         bool fused_append, hipStream_t s) {
  if (dtype == KVC_F32) {
    if (D == 64) return launch_rt<KVC_F32, 64>(a, row_tile, splits, fused_append, s);
    return launch_rt<KVC_F32, 128>(a, row_tile, splits, fused_append, s);
  }
  if (D == 64) return launch_rt<KVC_BF16, 64>(a, row_tile, splits, fused_append, s);
  return launch_rt<KVC_BF16, 128>(a, row_tile, splits, fused_append, s);
}

}  // namespace kvc
