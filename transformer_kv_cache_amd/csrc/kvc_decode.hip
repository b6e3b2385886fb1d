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
// of SPLIT consecutive keys) and the head's single query row.  Inside the
// workgroup:
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
// Combine.  Each workgroup writes its (max, sum, P.V) state to the
// workspace and a second, small kernel merges the states of every query row
// (rescaling by exp2 of the max difference) and writes the output.  The
// split kernel covers keys [0, P); the combine kernel adds the last key P as
// one more state, read from the new K/V row in the fused step (kvc_decode_step,
// which also writes that row to its cache slot there) and from the cache
// otherwise, so the fused and the two-call forms do the same arithmetic.
// Every split workgroup thus runs one uniform code path: none waits on the
// new row or on a store before its arithmetic, which would lengthen the
// slowest workgroup.  The merge is a separate launch rather than a
// last-workgroup ticket: the ticket needs a device-scope release fence in
// every workgroup, which on gfx950 is an L2 write-back (buffer_wbl2), and
// that measured about ten times slower than the extra launch.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

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
  if (LPR >= 32) x = xor_combine<16>(x);
  return x;
}

template <int NRG>
constexpr int kLog2Nrg = NRG == 8 ? 3 : NRG == 16 ? 4 : NRG == 32 ? 5 : 6;

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

template <int DT, int D, int KPL, bool PAGED, bool DEVLEN>
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

  // Grid: x = split, y = (layer, KV head), z = sequence in the batch slice.
  // The sequence comes straight from blockIdx.z so its length can be fetched
  // while the other indices are still being computed.  One query row per KV
  // head (G = N = 1), so the query row index equals the KV head index.
  const int split = blockIdx.x;
  const int bb = blockIdx.z;
  const int lh = blockIdx.y;
  // Every kernel argument the prologue needs, fetched in one scalar round:
  // the empty asm takes them all as operands, so none of their loads can be
  // deferred behind the early exit or the index arithmetic.
  const int P = seq_hist<DEVLEN>(a, bb);
  const int Hkv = a.Hkv, B = a.B, Tmax = a.Tmax, layer0 = a.layer0, b0 = a.b0, tail = a.tail;
  const uint32_t hkv_div = a.hkv_div;
  const char *k_cache = a.k_cache, *v_cache = a.v_cache, *qp = a.q;
  asm volatile("" ::"s"(P), "s"(Hkv), "s"(B), "s"(Tmax), "s"(layer0), "s"(b0), "s"(tail),
               "s"(hkv_div), "s"(k_cache), "s"(v_cache), "s"(qp));
  // Keys of this pass: 0 .. P-1 when the combine pass adds key P (always,
  // as launched), else 0 .. P.
  const int nk = P + 1 - tail;
  const int nsplit = (nk + SPLIT - 1) / SPLIT;
  if (split >= nsplit) return;
  const int l = div_magic(lh, Hkv, hkv_div);
  const int hkv = lh - l * Hkv;
  const int b = b0 + bb;
  // (layer, sequence, KV head) indices fit in 32 bits; only the row offsets
  // need 64.
  const uint32_t head = (uint32_t)(((layer0 + l) * B + b) * Hkv + hkv);
  const size_t crow0 = (size_t)head * (uint32_t)Tmax;
  const uint32_t row = (uint32_t)((l * B + b) * Hkv + hkv);  // (l, b, hq, i = 0), Hq = Hkv

  const int key0 = split * SPLIT;
  const int last = nk - 1 - key0;  // offset of the last visible key in this split
  // Uniform bases plus 32-bit per-lane byte offsets: global loads with an SGPR
  // base take one VGPR per address.
  const char *kc = k_cache + crow0 * (LPR * 16);
  const char *vc = v_cache + crow0 * (LPR * 16);

  // 1. Issue the query load and every K and V load of this split up front.
  //    Keys past the last visible one are clamped to it (a valid, written
  //    slot) so that no load sits behind a branch; their scores are masked.
  //    A paged cache first looks up the blocks (for blocks of at least NRG
  //    positions one scalar load per key load, else one load per key, all
  //    issued together), then streams the rows from their blocks.
  const u32x4 qw = reinterpret_cast<const u32x4 *>(qp)[(size_t)row * LPR + c];
  u32x4 kw[KPL], vw[KPL];
  if constexpr (PAGED) {
    size_t prow[KPL];
    if (a.pg.bs_log2 >= kLog2Nrg<NRG>) {
      // blocks of at least NRG positions: one scalar id lookup per load
      paged_rows_grouped<KPL, NRG>(a.pg, b, key0, key0 + last, rg, layer0 + l, hkv, Hkv, prow);
    } else {
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int kr = kk * NRG + rg;
        prow[kk] = paged_row(a.pg, b, key0 + (kr < last ? kr : last), layer0 + l, hkv, Hkv);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      kw[kk] = stream_load(reinterpret_cast<const u32x4 *>(k_cache) + prow[kk] * LPR + c);
      vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(v_cache) + prow[kk] * LPR + c);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KPL; ++kk) {
      const int kr = kk * NRG + rg;  // key offset within the split
      const uint32_t off = (uint32_t)((key0 + (kr < last ? kr : last)) * LPR + c) * 16u;
      kw[kk] = stream_load(reinterpret_cast<const u32x4 *>(kc + off));
      vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(vc + off));
    }
  }
  // Keep the scheduler from interleaving arithmetic (and its waits) into the
  // load burst: all loads of the split are in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);

  // 2. Scores in the log2 domain; key key0 + kk*NRG + rg is visible iff its
  //    offset is at most `last`, a compare of rg against a uniform bound.
  float qf[EV];
  unpack16<DT>(qw, qf);
  float s[KPL];
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    float kf[EV];
    unpack16<DT>(kw[kk], kf);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) dot = fmaf(qf[e], kf[e], dot);
    dot = row_allreduce<LPR>(dot);
    s[kk] = (rg <= last - kk * NRG) ? dot * a.scale_log2 : kNegInf;
  }

  // 3. Per-row-group softmax state over its KPL keys.  Row group 0 always
  //    holds key key0, which is visible, so in the merged state the max is
  //    finite.
  float m = s[0];
#pragma unroll
  for (int kk = 1; kk < KPL; ++kk) m = fmaxf(m, s[kk]);
  float lsum = 0.f, acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    float vf[EV];
    unpack16<DT>(vw[kk], vf);
    const float p = (m == kNegInf) ? 0.f : fast_exp2(s[kk] - m);
    lsum += p;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
  }

  // 4. Merge the row groups of this wave (lanes with the same c).
  {
    float M = m;
    if constexpr (LPR <= 8) M = xor_combine<8, true>(M);
    if constexpr (LPR <= 16) M = xor_combine<16, true>(M);
    M = xor_combine<32, true>(M);
    const float f = rescale(m, M);
    lsum *= f;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] *= f;
    if constexpr (LPR <= 8) {
      lsum = xor_combine<8>(lsum);
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] = xor_combine<8>(acc[e]);
    }
    if constexpr (LPR <= 16) {
      lsum = xor_combine<16>(lsum);
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] = xor_combine<16>(acc[e]);
    }
    lsum = xor_combine<32>(lsum);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = xor_combine<32>(acc[e]);
    m = M;
  }

  // 5. Merge the four waves through LDS; write this split's state (or the
  //    output, for a single split with no key left to the combine pass).
  __shared__ float sh_o[4][D];
  __shared__ float sh_m[4];
  __shared__ float sh_l[4];
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EV; ++e) sh_o[wave][c * EV + e] = acc[e];
    if (c == 0) {
      sh_m[wave] = m;
      sh_l[wave] = lsum;
    }
  }
  __syncthreads();

  if (tid < D) {
    const int d = tid;
    float M = sh_m[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh_m[w]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = rescale(sh_m[w], M);
      o = fmaf(f, sh_o[w][d], o);
      L = fmaf(f, sh_l[w], L);
    }
    if (!tail && nsplit == 1) {
      const float val = o / L;
      store_elems<DT>(a.o, (size_t)row * D + d, &val, 1);
    } else {
      const size_t ws = ws_slot(a, row, split);
      a.ws_o[ws * D + d] = o;
      if (d == 0) {
        a.ws_ml[ws * 2] = M;
        a.ws_ml[ws * 2 + 1] = L;
      }
    }
  }
}

// One element of a row in the cache dtype: raw bits, and widened to fp32.
template <int DT> struct Elem;
template <> struct Elem<KVC_F32> {
  typedef uint32_t bits;
  static __device__ __forceinline__ float widen(bits u) { return __uint_as_float(u); }
};
template <> struct Elem<KVC_BF16> {
  typedef uint16_t bits;
  static __device__ __forceinline__ float widen(bits u) { return __uint_as_float((uint32_t)u << 16); }
};

// Merge of the split-K states of query rows: o = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s with M = max_s m_s.  One wave per row, lane j holding
// elements j, j + 64, ... of it.  Grid: x = blocks of 4 rows over the Hq * N
// rows of one (layer, sequence), y = layer, z = sequence in the batch slice,
// so that a row's index needs no division.
//   Without `tail` only rows whose sequence needed more than one split are
// merged (the split kernel wrote the others).  With `tail` (one query row per
// KV head) the split states cover keys [0, P) and this pass adds key P: its
// state is (m, l, o) = (scale log2(e) q.k_P, 1, v_P), merged like any split.
// In the fused step k_P, v_P come from k_new / v_new and this pass then
// writes them to cache slot P (read by no kernel of the step, so the write
// is race-free); otherwise they are read from slot P.
template <int DT, int D, bool DEVLEN>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int EPL = D / 64;  // elements per lane
  typedef typename Elem<DT>::bits bits;
  const int lane = threadIdx.x & 63;
  // (hq, i); wave-uniform, so a row's split (max, sum) pairs are scalar loads
  const int rloc = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int bb = blockIdx.z;
  const int l = blockIdx.y;
  // Every kernel argument, fetched in one scalar round (the empty asm takes
  // them all as operands, so no load is deferred behind a branch).
  const int P = seq_hist<DEVLEN>(a, bb);
  const int Hq = a.Hq, N = a.N, tail = a.tail, split_keys = a.split_keys, B = a.B, Hkv = a.Hkv;
  const int Tmax = a.Tmax, layer0 = a.layer0, b0 = a.b0;
  const uint32_t split_div = a.split_div;
  const char *qp = a.q, *knp = a.k_new, *vnp = a.v_new;
  char *kcp = a.k_cache, *vcp = a.v_cache;
  const float *ws_o = a.ws_o, *ws_ml = a.ws_ml;
  asm volatile("" ::"s"(P), "s"(Hq), "s"(N), "s"(tail), "s"(split_keys), "s"(B), "s"(Hkv),
               "s"(Tmax), "s"(layer0), "s"(b0), "s"(split_div), "s"(qp),
               "s"(knp), "s"(vnp), "s"(kcp), "s"(vcp), "s"(ws_o), "s"(ws_ml));
  if (rloc >= Hq * N) return;
  const int nk = tail ? P : P + N;  // keys covered by split states
  const int nsplit = div_magic(nk + split_keys - 1, split_keys, split_div);
  if (!tail && nsplit <= 1) return;  // written by the split kernel
  const int b = b0 + bb;
  const long long row = ((long long)l * B + b) * (Hq * N) + rloc;

  // Cache slot P of this row's (layer, sequence, KV head); rows are
  // (l, b, hkv) in tail mode (G = N = 1), so q, k_new and v_new share the
  // row index.
  const size_t slot = (a.pg.block_table ? paged_row(a.pg, b, P, layer0 + l, rloc, Hkv)
                                         : (((size_t)(layer0 + l) * B + b) * Hkv + rloc) * Tmax + P) *
                      D;
  const bool fused = knp != nullptr;

  // Splits in chunks of CH, every load of a chunk issued before any is used
  // (indices clamped, extra splits masked), merged online across chunks.  The
  // key-P rows and the first chunk are loaded together.
  constexpr int CH = 16;
  float mv[CH], lv[CH], ov[CH][EPL];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int sp = (s0 + t < nsplit) ? s0 + t : nsplit - 1;
      const size_t ws = ws_slot(a, row, sp);
      mv[t] = ws_ml[ws * 2];
      lv[t] = ws_ml[ws * 2 + 1];
#pragma unroll
      for (int j = 0; j < EPL; ++j) ov[t][j] = ws_o[ws * D + lane + 64 * j];
    }
  };
  // Key P's rows (loaded unconditionally, from q itself when unused, so that
  // no load sits behind a branch the compiler could fill with their use).
  const bits *qb = reinterpret_cast<const bits *>(qp) + (size_t)row * D;
  const bits *kb = !tail ? qb
                   : fused ? reinterpret_cast<const bits *>(knp) + (size_t)row * D
                           : reinterpret_cast<const bits *>(kcp) + slot;
  const bits *vb = !tail ? qb
                   : fused ? reinterpret_cast<const bits *>(vnp) + (size_t)row * D
                           : reinterpret_cast<const bits *>(vcp) + slot;
  bits qn[EPL], kn[EPL], vn[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    qn[j] = qb[lane + 64 * j];
    kn[j] = kb[lane + 64 * j];
    vn[j] = vb[lane + 64 * j];
  }
  if (nsplit > 0) load_chunk(0);
  __builtin_amdgcn_sched_barrier(0);
  if (tail && fused) {
    // the append of the new row, issued before the merge arithmetic
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      reinterpret_cast<bits *>(kcp)[slot + lane + 64 * j] = kn[j];
      reinterpret_cast<bits *>(vcp)[slot + lane + 64 * j] = vn[j];
    }
  }

  float M = kNegInf, L = 0.f, o[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) o[j] = 0.f;
  if (tail) {
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) dot = fmaf(Elem<DT>::widen(qn[j]), Elem<DT>::widen(kn[j]), dot);
    dot = row_allreduce<16>(dot);
    dot = xor_combine<16>(dot);
    dot = xor_combine<32>(dot);
    M = dot * a.scale_log2;
    L = 1.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) o[j] = Elem<DT>::widen(vn[j]);
  }
  for (int s0 = 0; s0 < nsplit; s0 += CH) {
    if (s0 > 0) {
      load_chunk(s0);
      __builtin_amdgcn_sched_barrier(0);
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
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float val = o[j] * inv;
    store_elems<DT>(a.o, (size_t)row * D + lane + 64 * j, &val, 1);
  }
}

// Keys each lane group loads per split: a split covers 256 / LPR * this many
// keys (64 for fp32 D=64).  Build-time tuning constant; 4 measured best
// across the fp32, bf16 and GQA decode workloads.
#ifndef KVC_DECODE_KEYS_PER_LANE
#define KVC_DECODE_KEYS_PER_LANE 4
#endif
constexpr int kKeysPerLane = KVC_DECODE_KEYS_PER_LANE;

template <int DT, int D>
hipError_t launch_one(const DecodeArgs &a, int splits, hipStream_t s) {
  const dim3 grid((unsigned)splits, (unsigned)(a.n_layers * a.Hkv), (unsigned)a.nb);
  if (a.pg.block_table && a.hist_dev)
    hipLaunchKernelGGL((decode_kernel<DT, D, kKeysPerLane, true, true>), grid, dim3(256), 0, s, a);
  else if (a.pg.block_table)
    hipLaunchKernelGGL((decode_kernel<DT, D, kKeysPerLane, true, false>), grid, dim3(256), 0, s, a);
  else if (a.hist_dev)
    hipLaunchKernelGGL((decode_kernel<DT, D, kKeysPerLane, false, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, kKeysPerLane, false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_row_tile(int /*rows*/) { return 1; }

int decode_split_keys(int dtype, int D) {
  const int lpr = D * (dtype == KVC_BF16 ? 2 : 4) / 16;
  return (256 / lpr) * kKeysPerLane;
}

hipError_t launch_combine(const DecodeArgs &a, int dtype, int D, hipStream_t s) {
  const int rows = a.Hq * a.N;  // per (layer, sequence); one wave each
  const dim3 grid((unsigned)((rows + 3) / 4), (unsigned)a.n_layers, (unsigned)a.nb);
  if (a.hist_dev) {
    if (dtype == KVC_F32) {
      if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_F32, 64, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<KVC_F32, 128, true>), grid, dim3(256), 0, s, a);
    } else {
      if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_BF16, 64, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<KVC_BF16, 128, true>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  if (dtype == KVC_F32) {
    if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_F32, 64, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<KVC_F32, 128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((combine_kernel<KVC_BF16, 64, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<KVC_BF16, 128, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int D, int splits, hipStream_t s) {
  // The vector kernel serves one query row per KV head (G = N = 1) only.
  if (a.rows != 1 || a.N != 1 || a.group != 1) return hipErrorInvalidValue;
  if (dtype == KVC_F32) {
    if (D == 64) return launch_one<KVC_F32, 64>(a, splits, s);
    return launch_one<KVC_F32, 128>(a, splits, s);
  }
  if (D == 64) return launch_one<KVC_BF16, 64>(a, splits, s);
  return launch_one<KVC_BF16, 128>(a, splits, s);
}

}  // namespace kvc
