// kvc_decode.hip -- attention of one new query row per KV head against the
// KV cache: split-K ("flash-decode") with the merge of the splits done inside
// the same launch, and, for calls whose rows alone about fill the GPU, one
// workgroup per row streaming its whole key range (decode_row_kernel, below
// the split kernel).
//
// What it computes ([KV-4] jennyma11.github.io/infra/ch07-01.html, "Decode
// 阶段", listing 1-2; [KV-2] openai-hub.com/news/2435, "一个很容易漏掉的错误"):
// for each (layer, sequence b, KV head) the softmax of scale * q . K_j over
// keys j = 0 .. P_b, applied to V.  Decode reads every cached K/V byte once
// and does ~1 flop per byte, so it is bound by HBM bandwidth ([KV-2]
// "千倍计算量为何只换来6倍速度").  Several query rows per KV head (GQA groups,
// chunked decode) go to kvc_decode_rows.hip / kvc_decode_mfma.hip.
//
// Work split.  A workgroup (256 lanes, 4 waves) owns one (layer, sequence,
// KV head, split of SPLIT consecutive keys of [0, P)).  Inside it:
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
// The last key, P, is not in any split: it is merged as one more state
// (scale log2(e) q.k_P, 1, v_P), read from the new K/V row in the fused step
// (kvc_decode_step, which also writes that row to its cache slot) and from
// the cache otherwise, so the fused and the two-call forms do the same
// arithmetic.
//
// Merge inside the launch.  Each split workgroup writes its (max, sum, P.V)
// state to the workspace and counts itself on an arrival counter of its
// query row; the workgroup that arrives last merges every state of the row
// with key P's and writes the output (and resets the counter, so the
// workspace's counters are zero again when the kernel ends).  A device-scope
// release fence per workgroup would make this an L2 write-back on gfx950;
// instead all workgroups of a row run on one XCD and exchange the states
// through that XCD's L2: workgroups are dispatched to the XCDs round-robin
// by linear id, so the grid is one-dimensional with the row's XCD fixed by
// its position (id % 8).  A writer waits until the L2 has acknowledged its
// state stores before it counts itself, and the last one reads the states
// with L1-bypassing loads, which the L2 serves.  Each workgroup also reads
// its XCD id from the hardware and adds it to the counter; the merging
// workgroup checks that every writer of the row ran on its own XCD and
// writes NaN for the row otherwise, so a placement other than the documented
// one can only fail loudly.  The wait
// for the acknowledgement costs a round trip per workgroup, hidden while
// every workgroup is resident at once and exposed when they queue for CU
// slots, so the host takes this path only when the grid fits the chip in
// one round; otherwise (and when the XCD count does not divide 8) the merge
// is a second kernel, combine_kernel, which runs the same merge code.
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
__device__ __forceinline__ u32x4 stream_load(const u32x4 *p) { return __builtin_nontemporal_load(p); }

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

// Key P's score in the log2 domain, scale log2(e) q.k_P, from one wave whose
// lane j holds elements j, j + 64, ... of q and k_P.
template <int DT, int EPL>
__device__ __forceinline__ float key_score(const typename Elem<DT>::bits (&qn)[EPL],
                                           const typename Elem<DT>::bits (&kn)[EPL], float scale_log2) {
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) dot = fmaf(Elem<DT>::widen(qn[j]), Elem<DT>::widen(kn[j]), dot);
  dot = row_allreduce<16>(dot);
  dot = xor_combine<16>(dot);
  dot = xor_combine<32>(dot);
  return dot * scale_log2;
}

// Cache row index (in rows of D elements) of position P of this (layer,
// sequence, KV head): contiguous, or through the block table.
template <bool PAGED>
__device__ __forceinline__ size_t slot_row(const DecodeArgs &a, int b, int P, int layer, int hkv) {
  if constexpr (PAGED) return paged_row(a.pg, b, P, layer, hkv, a.Hkv);
  else return (((size_t)layer * a.B + b) * a.Hkv + hkv) * (size_t)a.Tmax + P;
}

// The split kernel.  Grid: one dimension of 8 * ceil(units / 8) * grid_splits
// workgroups.  Workgroup w runs on XCD w % 8 (round-robin dispatch); with
// j = w / 8 it takes split j % grid_splits of unit (j / grid_splits) * 8 +
// w % 8, so all splits of a unit share an XCD.  A unit is one (sequence,
// layer, KV head) = one query row (G = N = 1): u = (bb * n_layers + l) * Hkv
// + hkv.  MERGE: the last-arriving split workgroup merges (see above);
// otherwise every split only writes its state for combine_kernel.
template <int DT, int D, int KPL, bool PAGED, bool DEVLEN, bool MERGE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int EV = Dtype<DT>::kPer16B;        // elements per 16-byte vector
  constexpr int LPR = D * Dtype<DT>::kBytes / 16;  // lanes per key row
  constexpr int NRG = 256 / LPR;                 // key rows per wave-group load
  constexpr int SPLIT = NRG * KPL;               // keys per workgroup
  constexpr int EPL = D / 64;                    // output elements per lane of one wave
  typedef typename Elem<DT>::bits bits;
  static_assert(LPR * EV == D, "row layout");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = tid / LPR;
  const int c = tid % LPR;

  const int wg = blockIdx.x;
  // Every kernel argument the prologue needs, fetched in one scalar round:
  // the empty asm takes them all as operands, so none of their loads can be
  // deferred behind the early exits or the index arithmetic.
  const int units = a.units, grid_splits = a.grid_splits, n_layers = a.n_layers;
  const int Hkv = a.Hkv, B = a.B, Tmax = a.Tmax, layer0 = a.layer0, b0 = a.b0;
  const uint32_t gs_div = a.grid_splits_div, hkv_div = a.hkv_div, nl_div = a.nl_div;
  const char *k_cache = a.k_cache, *v_cache = a.v_cache, *qp = a.q;
  asm volatile("" ::"s"(units), "s"(grid_splits), "s"(n_layers), "s"(Hkv), "s"(B), "s"(Tmax),
               "s"(layer0), "s"(b0), "s"(gs_div), "s"(hkv_div), "s"(nl_div), "s"(k_cache),
               "s"(v_cache), "s"(qp));
  const int lj = wg >> 3;
  const int lu = div_magic(lj, grid_splits, gs_div);
  const int split = lj - lu * grid_splits;
  const int u = lu * 8 + (wg & 7);
  if (u >= units) return;
  const int t = div_magic(u, Hkv, hkv_div);
  const int hkv = u - t * Hkv;
  const int bb = div_magic(t, n_layers, nl_div);
  const int l = t - bb * n_layers;
  const int P = seq_hist<DEVLEN>(a, bb);
  // Split states cover keys [0, P); key P is merged by the last workgroup.
  const int nsplit = (P + SPLIT - 1) / SPLIT;
  if (split >= (nsplit > 0 ? nsplit : 1)) return;
  if (!MERGE && nsplit == 0) return;
  const int b = b0 + bb;
  // (layer, sequence, KV head) indices fit in 32 bits; only the row offsets
  // need 64.
  const uint32_t head = (uint32_t)(((layer0 + l) * B + b) * Hkv + hkv);
  const size_t crow0 = (size_t)head * (uint32_t)Tmax;
  const uint32_t row = (uint32_t)((l * B + b) * Hkv + hkv);  // (l, b, hq, i = 0), Hq = Hkv

  float Mw = kNegInf, Lw = 0.f, ow[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) ow[j] = 0.f;
  const int key0 = split * SPLIT;
  const int last = P - 1 - key0;  // offset of the last key of this split
  // 1. Issue the query load and every K and V load of this split up front.
  //    Keys past the last one are clamped to it (a valid, written slot) so
  //    that no load sits behind a branch; their scores are masked.  A paged
  //    cache first looks up the blocks (for blocks of at least NRG positions
  //    one scalar load per key load, else one load per key, all issued
  //    together), then streams the rows from their blocks.
  u32x4 qw, kw[KPL], vw[KPL];
  if (nsplit > 0) {
    // Uniform bases plus 32-bit per-lane byte offsets (the host bounds a
    // head's rows below 4 GiB): global loads with an SGPR base take one VGPR
    // per address.
    const char *kc = k_cache + crow0 * (LPR * 16);
    const char *vc = v_cache + crow0 * (LPR * 16);
    qw = reinterpret_cast<const u32x4 *>(qp)[(size_t)row * LPR + c];
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
        if constexpr (KPL < 8) vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(v_cache) + prow[kk] * LPR + c);
      }
      if constexpr (KPL >= 8) {
        __builtin_amdgcn_sched_barrier(0);  // K ahead of V (see below)
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(v_cache) + prow[kk] * LPR + c);
      }
    } else {
      // With eight keys per lane group every K load goes out ahead of every
      // V load: the scores and the softmax, which need only K, then run while
      // V is still arriving, and only the P.V products and the merges are
      // left after the last byte (measured: -0.15 to -0.2 us on the 12-layer
      // step at T=1024).  With four, K and V alternate.
      uint32_t off[KPL];
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int kr = kk * NRG + rg;  // key offset within the split
        off[kk] = (uint32_t)((key0 + (kr < last ? kr : last)) * LPR + c) * 16u;
        kw[kk] = stream_load(reinterpret_cast<const u32x4 *>(kc + off[kk]));
        if constexpr (KPL < 8) vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(vc + off[kk]));
      }
      if constexpr (KPL >= 8) {
        __builtin_amdgcn_sched_barrier(0);  // the compiler would interleave them again
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(vc + off[kk]));
      }
    }
  }
  // Key P's rows for the merge (lane j holds elements j + 64 e), behind the
  // burst in every wave (no branch, so nothing waits for them before the
  // merge): q, and k_P / v_P from the new rows (fused step) or from cache
  // slot P.
  bits qn[EPL], kn[EPL], vn[EPL];
  size_t slot = 0;
  if constexpr (MERGE) {
    slot = slot_row<PAGED>(a, b, P, layer0 + l, hkv) * D;
    const bits *qb = reinterpret_cast<const bits *>(qp) + (size_t)row * D;
    const bits *kb = a.k_new ? reinterpret_cast<const bits *>(a.k_new) + (size_t)row * D
                             : reinterpret_cast<const bits *>(k_cache) + slot;
    const bits *vb = a.v_new ? reinterpret_cast<const bits *>(a.v_new) + (size_t)row * D
                             : reinterpret_cast<const bits *>(v_cache) + slot;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      qn[j] = qb[lane + 64 * j];
      kn[j] = kb[lane + 64 * j];
      vn[j] = vb[lane + 64 * j];
    }
  }
  // Keep the scheduler from interleaving arithmetic (and its waits) into the
  // load burst: all loads of the split are in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);

  if (nsplit > 0) {

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

    // 5. Merge the four waves through LDS into wave 0 (lane j: elements
    //    j + 64 e) and write this split's state.
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
    if (wave != 0) return;
    Mw = sh_m[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mw = fmaxf(Mw, sh_m[w]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = rescale(sh_m[w], Mw);
#pragma unroll
      for (int j = 0; j < EPL; ++j) ow[j] = fmaf(f, sh_o[w][lane + 64 * j], ow[j]);
      Lw = fmaf(f, sh_l[w], Lw);
    }
    const size_t ws = (size_t)split * (size_t)a.ws_rows + row;
#pragma unroll
    for (int j = 0; j < EPL; ++j) a.ws_o[ws * D + lane + 64 * j] = ow[j];
    if (lane == 0)
      *reinterpret_cast<uint64_t *>(a.ws_ml + ws * 2) =
          (uint64_t)__float_as_uint(Mw) | ((uint64_t)__float_as_uint(Lw) << 32);
  }
  if constexpr (MERGE) {
    if (wave != 0) return;
    bool misplaced = false;
    if (nsplit > 1) {
      // Count this split once the L2 holds its state; the last to arrive
      // merges (and checks that every state went through its L2).
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      uint32_t last = 0, mis = 0;
      if (lane == 0) {
        bool m = false;
        last = arrive_last(a.counters + row, nsplit, m);
        mis = m;
      }
      if (!__builtin_amdgcn_readfirstlane(last)) return;
      asm volatile("" ::: "memory");
      misplaced = __builtin_amdgcn_readfirstlane(mis) != 0;
    } else if (nsplit == 1) {
      // the merge reads back this workgroup's own state: wait until the L2
      // holds it, or the read may return the previous call's
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // The merge: key P's state first, then every split's (this one's
    // included, read back), then the normalisation.
    float M = key_score<DT, EPL>(qn, kn, a.scale_log2);
    float L = 1.f, o[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) o[j] = Elem<DT>::widen(vn[j]);
    merge_states<D>(a.ws_o, a.ws_ml, a.ws_rows, row, nsplit, lane, M, L, o);
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const float val = misplaced ? __builtin_nanf("") : o[j] * inv;
      store_elems<DT>(a.o, (size_t)row * D + lane + 64 * j, &val, 1);
    }
    if (a.k_new) {
      // the append of the new row (no workgroup of this launch reads slot P)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        reinterpret_cast<bits *>(a.k_cache)[slot + lane + 64 * j] = kn[j];
        reinterpret_cast<bits *>(a.v_cache)[slot + lane + 64 * j] = vn[j];
      }
    }
    if (nsplit > 1 && lane == 0) reset_counter(a.counters + row);
  }
}

// Block ids of one sequence the paged row kernel stages in LDS (8 KB).
constexpr int kRowMaxBlocks = 2048;

// One workgroup per query row, for calls whose rows alone fill the chip
// (about one per CU).  The workgroup streams the whole key range [0, P) of
// its (layer, sequence, KV head) in chunks of CH = NRG * KPL keys, with the
// next chunk's K and V loads in flight while the current chunk is reduced
// (two register buffers; chunks past the end are clamped to key P - 1 and
// reduce to nothing, so no load sits behind a branch).  Rows are laid out
// as in decode_kernel's split: a key row is LPR lanes wide, one 16-byte
// vector per lane, so a wave's load reads 1 KB of consecutive rows (two
// vectors per lane, each load then reading half rows at the row stride,
// measured slower despite a third less vector work).  Each row group carries its online-softmax
// state across the chunks (rescaled by 2^(m_old - m_new) when its running
// max grows); at the end the states merge across the wave with cross-lane
// exchanges and across the waves through LDS, then with key P's state as in
// the split form.  Nothing goes through the workspace: the merge is an LDS
// round trip instead of a state store, its acknowledgement, an arrival
// atomic and the merging workgroup's loads through the L2.  Streaming from
// one workgroup per row leaves the CUs beyond the row count idle, which the
// host plan weighs against that merge.
//   PAGED: the row's block ids are staged in LDS once (at most kRowMaxBlocks
// of them; the host sends longer tables to the split kernel), so a chunk's
// loads wait only for LDS reads, not for block-table loads from memory.
template <int DT, int D, int KPL, int NT, bool PAGED, bool DEVLEN>
__global__ __launch_bounds__(NT) void decode_row_kernel(DecodeArgs a) {
  constexpr int EV = Dtype<DT>::kPer16B;
  constexpr int LPR = D * Dtype<DT>::kBytes / 16;  // lanes per row
  constexpr int NW = NT / 64;                      // waves
  constexpr int NRG = NT / LPR;                    // rows per load
  constexpr int CH = NRG * KPL;                    // keys per chunk
  constexpr int EPL = D / 64;
  typedef typename Elem<DT>::bits bits;
  static_assert(LPR * EV == D && LPR >= 8, "row layout");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = tid / LPR;
  const int c = tid % LPR;
  const int u = blockIdx.x;
  const int units = a.units, n_layers = a.n_layers, Hkv = a.Hkv, B = a.B, Tmax = a.Tmax;
  const int layer0 = a.layer0, b0 = a.b0;
  const uint32_t hkv_div = a.hkv_div, nl_div = a.nl_div;
  const char *k_cache = a.k_cache, *v_cache = a.v_cache, *qp = a.q;
  const float scale_log2 = a.scale_log2;
  asm volatile("" ::"s"(units), "s"(n_layers), "s"(Hkv), "s"(B), "s"(Tmax), "s"(layer0), "s"(b0),
               "s"(hkv_div), "s"(nl_div), "s"(k_cache), "s"(v_cache), "s"(qp), "s"(scale_log2));
  if (u >= units) return;
  const int t = div_magic(u, Hkv, hkv_div);
  const int hkv = u - t * Hkv;
  const int bb = div_magic(t, n_layers, nl_div);
  const int l = t - bb * n_layers;
  const int P = seq_hist<DEVLEN>(a, bb);
  const int b = b0 + bb;
  const uint32_t head = (uint32_t)(((layer0 + l) * B + b) * Hkv + hkv);
  const size_t crow0 = (size_t)head * (uint32_t)Tmax;
  const uint32_t row = (uint32_t)((l * B + b) * Hkv + hkv);
  const int nch = (P + CH - 1) / CH;
  const char *kc = k_cache + crow0 * (LPR * 16);
  const char *vc = v_cache + crow0 * (LPR * 16);

  __shared__ int32_t sh_blk[PAGED ? kRowMaxBlocks : 1];
  if constexpr (PAGED) {
    const int bsl = a.pg.bs_log2;
    const int nblk = (P + (1 << bsl) - 1) >> bsl;
    const int32_t *tbl = a.pg.block_table + (size_t)b * a.pg.max_blocks;
    for (int i = tid; i < nblk; i += NT) {
      const int blk = tbl[i];
      sh_blk[i] = blk < 0 ? 0 : (blk >= a.pg.num_blocks ? a.pg.num_blocks - 1 : blk);
    }
    __syncthreads();
  }

  // Chunk ch's K loads, then its V loads (positions past P - 1 clamped to it).
  auto load_chunk = [&](int ch, u32x4 (&kw)[KPL], u32x4 (&vw)[KPL]) {
    const int key0 = ch * CH;
    if constexpr (PAGED) {
      const int bsl = a.pg.bs_log2;
      size_t prow[KPL];
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int pos0 = key0 + kk * NRG + rg;
        const int pos = pos0 < P - 1 ? pos0 : P - 1;
        prow[kk] = ((((size_t)(layer0 + l) * a.pg.num_blocks + sh_blk[pos >> bsl]) * Hkv + hkv) << bsl) +
                   (size_t)(pos & ((1 << bsl) - 1));
      }
      const u32x4 *kb = reinterpret_cast<const u32x4 *>(k_cache);
      const u32x4 *vb = reinterpret_cast<const u32x4 *>(v_cache);
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) kw[kk] = stream_load(kb + prow[kk] * LPR + c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) vw[kk] = stream_load(vb + prow[kk] * LPR + c);
    } else {
      uint32_t off[KPL];
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const int pos = key0 + kk * NRG + rg;
        off[kk] = (uint32_t)((pos < P - 1 ? pos : P - 1) * LPR + c) * 16u;
        kw[kk] = stream_load(reinterpret_cast<const u32x4 *>(kc + off[kk]));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) vw[kk] = stream_load(reinterpret_cast<const u32x4 *>(vc + off[kk]));
    }
  };

  // Key P's rows (lane j holds elements j + 64 e): q, and k_P / v_P from the
  // new rows (fused step) or from cache slot P.
  const size_t slot = slot_row<PAGED>(a, b, P, layer0 + l, hkv) * D;
  bits qn[EPL], kn[EPL], vn[EPL];
  {
    const bits *qb = reinterpret_cast<const bits *>(qp) + (size_t)row * D;
    const bits *kb = a.k_new ? reinterpret_cast<const bits *>(a.k_new) + (size_t)row * D
                             : reinterpret_cast<const bits *>(k_cache) + slot;
    const bits *vb = a.v_new ? reinterpret_cast<const bits *>(a.v_new) + (size_t)row * D
                             : reinterpret_cast<const bits *>(v_cache) + slot;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      qn[j] = qb[lane + 64 * j];
      kn[j] = kb[lane + 64 * j];
      vn[j] = vb[lane + 64 * j];
    }
  }

  float m = kNegInf, lsum = 0.f, acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
  if (nch > 0) {
    const u32x4 qw = reinterpret_cast<const u32x4 *>(qp)[(size_t)row * LPR + c];
    u32x4 kA[KPL], vA[KPL], kB[KPL], vB[KPL];
    load_chunk(0, kA, vA);
    // q pre-scaled: scores come out in the log2 domain
    float qf[EV];
    unpack16<DT>(qw, qf);
#pragma unroll
    for (int e = 0; e < EV; ++e) qf[e] *= scale_log2;
    // Fold chunk ch into the row group's state.
    auto reduce_chunk = [&](int ch, const u32x4 (&kw)[KPL], const u32x4 (&vw)[KPL]) {
      const int last = P - 1 - ch * CH;  // offset of the last visible key
      float s[KPL];
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        float kf[EV];
        unpack16<DT>(kw[kk], kf);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) dot = fmaf(qf[e], kf[e], dot);
        dot = row_allreduce<LPR>(dot);
        s[kk] = (rg <= last - kk * NRG) ? dot : kNegInf;
      }
      float mn = m;
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) mn = fmaxf(mn, s[kk]);
      const float f = rescale(m, mn);
      lsum *= f;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] *= f;
#pragma unroll
      for (int kk = 0; kk < KPL; ++kk) {
        const float p = (mn == kNegInf) ? 0.f : fast_exp2(s[kk] - mn);
        lsum += p;
        float vf[EV];
        unpack16<DT>(vw[kk], vf);
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
      }
      m = mn;
    };
    // Two chunks per trip with no branch inside: a chunk past the end (odd
    // nch) reduces to a no-op (every score masked), and the last trip's
    // prefetch reads key P - 1 again.
    for (int ch = 0; ch < nch; ch += 2) {
      load_chunk(ch + 1, kB, vB);
      __builtin_amdgcn_sched_barrier(0);
      reduce_chunk(ch, kA, vA);
      load_chunk(ch + 2, kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      reduce_chunk(ch + 1, kB, vB);
    }
  }

  // Merge the row groups of each wave (lanes with the same c) ...
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
  // ... and the waves through LDS into wave 0 (lane j: elements j + 64 e).
  __shared__ float sh_o[NW][D];
  __shared__ float sh_m[NW];
  __shared__ float sh_l[NW];
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EV; ++e) sh_o[wave][c * EV + e] = acc[e];
    if (c == 0) {
      sh_m[wave] = m;
      sh_l[wave] = lsum;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float Mw = sh_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mw = fmaxf(Mw, sh_m[w]);
  float Lw = 0.f, ow[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) ow[j] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float f = rescale(sh_m[w], Mw);
#pragma unroll
    for (int j = 0; j < EPL; ++j) ow[j] = fmaf(f, sh_o[w][lane + 64 * j], ow[j]);
    Lw = fmaf(f, sh_l[w], Lw);
  }
  // Key P's state (M, 1, v_P) merged with the keys before it.
  float M = key_score<DT, EPL>(qn, kn, scale_log2);
  const float Mc = fmaxf(M, Mw);
  const float fp = rescale(M, Mc), fw = rescale(Mw, Mc);
  const float L = fmaf(fw, Lw, fp);
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float val = fmaf(fw, ow[j], fp * Elem<DT>::widen(vn[j])) * inv;
    store_elems<DT>(a.o, (size_t)row * D + lane + 64 * j, &val, 1);
  }
  if (a.k_new) {
    // the append of the new row (no workgroup of this launch reads slot P)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      reinterpret_cast<bits *>(a.k_cache)[slot + lane + 64 * j] = kn[j];
      reinterpret_cast<bits *>(a.v_cache)[slot + lane + 64 * j] = vn[j];
    }
  }
}

// Merge of the split-K states of query rows as a second launch.  One wave
// per row, lane j holding elements j, j + 64, ... of it.  Grid: x = blocks
// of 4 rows over the Hq * N rows of one (layer, sequence), y = layer, z =
// sequence in the batch slice, so that a row's index needs no division.
//   Without `tail` (several rows per KV head) only rows whose sequence needed
// more than one split are merged (the split kernel wrote the others).  With
// `tail` (one query row per KV head) the split states cover keys [0, P) and
// this pass adds key P first, as the fused kernel's merge does: from k_new /
// v_new in the fused step, which it then writes to cache slot P (read by no
// kernel of the step, so the write is race-free), else from the cache.
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
  if (tail && fused) {
    // the append of the new row
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
    M = key_score<DT, EPL>(qn, kn, a.scale_log2);
    L = 1.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) o[j] = Elem<DT>::widen(vn[j]);
  }
  merge_states<D>(ws_o, ws_ml, a.ws_rows, row, nsplit, lane, M, L, o);
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float val = o[j] * inv;
    store_elems<DT>(a.o, (size_t)row * D + lane + 64 * j, &val, 1);
  }
}

template <int DT, int D, int KPL, bool MERGE>
hipError_t launch_kpl(const DecodeArgs &a, unsigned grid, hipStream_t s) {
  if (a.pg.block_table && a.hist_dev)
    hipLaunchKernelGGL((decode_kernel<DT, D, KPL, true, true, MERGE>), dim3(grid), dim3(256), 0, s, a);
  else if (a.pg.block_table)
    hipLaunchKernelGGL((decode_kernel<DT, D, KPL, true, false, MERGE>), dim3(grid), dim3(256), 0, s, a);
  else if (a.hist_dev)
    hipLaunchKernelGGL((decode_kernel<DT, D, KPL, false, true, MERGE>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, KPL, false, false, MERGE>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D, bool MERGE>
hipError_t launch_dt(const DecodeArgs &a, int kpl, unsigned grid, hipStream_t s) {
  switch (kpl) {
    case 4: return launch_kpl<DT, D, 4, MERGE>(a, grid, s);
    case 8: return launch_kpl<DT, D, 8, MERGE>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// Two waves per row, 8 keys per lane group and chunk (measured on the
// 12-layer fp32 step at T=1024: 14.3 us against 14.8 with four waves, 19.4
// with one, 17.3 with eight; 4 or 16 keys per lane group slower).
constexpr int kRowThreads = 128;
constexpr int kRowKpl = 8;

template <int DT, int D, bool PAGED>
hipError_t launch_row_pg(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.units);
  if (a.hist_dev)
    hipLaunchKernelGGL((decode_row_kernel<DT, D, kRowKpl, kRowThreads, PAGED, true>), grid, dim3(kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_row_kernel<DT, D, kRowKpl, kRowThreads, PAGED, false>), grid, dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_row_dt(const DecodeArgs &a, hipStream_t s) {
  if (!a.pg.block_table) return launch_row_pg<DT, D, false>(a, s);
  if (a.pg.max_blocks > kRowMaxBlocks) return hipErrorInvalidValue;
  return launch_row_pg<DT, D, true>(a, s);
}

}  // namespace

int decode_rows_per_load(int dtype, int D) {
  const int lpr = D * (dtype == KVC_BF16 ? 2 : 4) / 16;
  return 256 / lpr;
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

hipError_t launch_decode(const DecodeArgs &a, int dtype, int D, int kpl, bool merge, hipStream_t s) {
  // The vector kernel serves one query row per KV head (G = N = 1) only.
  if (a.rows != 1 || a.N != 1 || a.group != 1 || a.grid_splits < 1) return hipErrorInvalidValue;
  const unsigned grid = 8u * (unsigned)((a.units + 7) / 8) * (unsigned)a.grid_splits;
  if (dtype == KVC_F32) {
    if (D == 64) return merge ? launch_dt<KVC_F32, 64, true>(a, kpl, grid, s)
                              : launch_dt<KVC_F32, 64, false>(a, kpl, grid, s);
    return merge ? launch_dt<KVC_F32, 128, true>(a, kpl, grid, s)
                 : launch_dt<KVC_F32, 128, false>(a, kpl, grid, s);
  }
  if (D == 64) return merge ? launch_dt<KVC_BF16, 64, true>(a, kpl, grid, s)
                            : launch_dt<KVC_BF16, 64, false>(a, kpl, grid, s);
  return merge ? launch_dt<KVC_BF16, 128, true>(a, kpl, grid, s)
               : launch_dt<KVC_BF16, 128, false>(a, kpl, grid, s);
}

hipError_t launch_decode_row(const DecodeArgs &a, int dtype, int D, hipStream_t s) {
  if (a.rows != 1 || a.N != 1 || a.group != 1 || a.units < 1) return hipErrorInvalidValue;
  if (dtype == KVC_F32) return D == 64 ? launch_row_dt<KVC_F32, 64>(a, s) : launch_row_dt<KVC_F32, 128>(a, s);
  return D == 64 ? launch_row_dt<KVC_BF16, 64>(a, s) : launch_row_dt<KVC_BF16, 128>(a, s);
}

int decode_row_max_blocks() { return kRowMaxBlocks; }

}  // namespace kvc
