// kvc_prefill.hip -- causal self-attention over a whole prompt on the matrix
// cores, writing the prompt's K/V rows into the cache on the way.
//
// What it computes ([KV-4] jennyma11.github.io/infra/ch07-01.html, "Prefill
// 阶段"; [KV-1] gitcode.csdn.net/69e62cef0a2f6a37c5a11c4f.html, "KV Cache
// 原理"): every prompt row i attends to rows 0..i; the K/V of all S rows land
// in cache rows [0, S).  Unlike decode this is a dense contraction (two
// S x S x D products per head), so it runs on MFMA.
//
// The same kernel serves kvc_attn_prefill_varlen ([KV-4] "Prefill 阶段":
// prompts packed along the token axis, each with its own cached prefix):
// sequence b brings S_b new tokens on top of P_b cached positions, new token
// i sits at position P_b + i and attends to positions 0 .. P_b + i; keys
// below P_b come from the cache, the others from the new K/V rows.  Rows of
// q / o / k / v are addressed through strides, so the padded layout of
// kvc_attn_prefill and the packed token-major one share the code; without
// history (every P_b = 0) a template switch drops the cache reads.
//
// Tiling.  A workgroup of 4 waves owns one (layer, sequence, query head) and a
// tile of BM = 128 new tokens (32 per wave); it walks key tiles of BN = 64
// positions up to the diagonal, staging each K/V tile in LDS once for all four
// waves.  Per wave and key tile:
//   S^T = K_tile . Q^T   (keys x queries; 32x32 MFMA blocks, Q held in
//                          registers for the whole kernel)
//   online softmax per query: each lane owns one query column, so the running
//   max / sum need a single exchange between the two half-waves
//   O^T += V^T . P^T     (P^T is taken straight from the S^T accumulators)
// Computing the transposed products keeps the softmax probabilities in the
// registers that feed the second MFMA.  Their key order inside a 16-key MFMA
// step follows the accumulator layout ({0-3, 8-11} in the low half-wave,
// {4-7, 12-15} in the high); the bf16 V tile stays in LDS as loaded (keys x
// D) and the gfx950 transpose load (ds_read_b64_tr_b16) hands each lane one
// d of four keys, two loads giving exactly that order -- no transposition
// work in the staging.
//   bf16: v_mfma_f32_32x32x16_bf16, P rounded to bf16 for the PV product
//         (and for the row sum), fp32 accumulation.
//   fp32: v_mfma_f32_32x32x2_f32, everything in fp32 (no reduced precision).
// Key split (fp32 at D = 64 on small grids): the workgroup owns 64 new tokens
// instead, two row groups of 32, and the two waves of a row group take the
// two 32-key halves of every tile, each with its own online-softmax state;
// at the end one hands its (max, sum, output) to the other through LDS,
// which rescales both to the larger max and adds them.  That halves the
// matrix work on a workgroup's longest chain for the same tile staging.
// Tiles above the diagonal are never loaded; a wave skips key tiles that lie
// entirely above its own 32 rows.  Grid order puts the longest (last) query
// tiles of every sequence first, and with a (layer, head) count that is a
// multiple of 8 all tiles of one head land on the same XCD and share its L2.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int BN = 64;   // keys per tile

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (low half = lo), round to nearest even, in
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int DT, int D> struct Smem;
template <int D> struct Smem<KVC_BF16, D> {
  static constexpr int kKStride = D + 8;    // bf16 elements per K row (16-B multiple)
  // V rows as loaded (keys x D).  The PV operand is read through the gfx950
  // transpose load (ds_read_b64_tr_b16): a 16-lane group reads four rows of
  // 32 bytes and each lane receives one d of the four keys.  A row stride of
  // D + 16 elements puts the four rows 8 banks apart, so a group's read is
  // conflict-free.
  static constexpr int kVStride = D + 16;
  alignas(16) uint16_t k[BN * kKStride];
  alignas(16) uint16_t v[BN * kVStride];
};
template <int D> struct Smem<KVC_F32, D> {
  static constexpr int kKStride = D + 4;
  static constexpr int kVStride = D;
  alignas(16) float k[BN * kKStride];
  alignas(16) float v[BN * kVStride];
};

template <int DT, int D, int KS, bool HIST, bool PAGED>
__device__ __forceinline__ void prefill_tile(const PrefillArgs &a) {
  static_assert(KS == 1 || KS == 2, "key split");
  constexpr int RG = 4 / KS;                   // query row groups of 32 rows
  constexpr int BM = 32 * RG;                  // query rows per workgroup
  constexpr int KBW = BN / 32 / KS;            // 32-key blocks per wave and tile
  constexpr int EB = Dtype<DT>::kBytes;
  constexpr int EV = Dtype<DT>::kPer16B;
  constexpr int RB = D * EB;                   // bytes per row
  constexpr int LPR = RB / 16;                 // 16-byte vectors per row
  constexpr int TILE_VECS = BN * LPR;          // 16-byte vectors per K (or V) tile
  constexpr int VPT = TILE_VECS / 256;         // per thread
  constexpr int DB = D / 32;                   // 32-wide d blocks of O^T
  static_assert(TILE_VECS % 256 == 0, "tile load split");
  __shared__ Smem<DT, D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int rg = wave % RG;        // query row group
  const int kh = wave / RG;        // key block of every tile: keys kb0 .. kb0 + 32 KBW - 1
  const int kb0 = 32 * KBW * kh;
  const int h = lane >> 5;     // half-wave
  const int col = lane & 31;   // MFMA column / row within a 32 block
  // Transpose-load address of this lane (bf16 V operand): in its 16-lane
  // group, lane 4 j + p names row 4 h + j, elements 4 p .. 4 p + 3 of the
  // group's 16 d (16 for the second group of a half-wave).
  const int v_tr_off = (4 * h + ((lane & 15) >> 2)) * ((DT == KVC_BF16) ? D + 16 : 0) +
                       (lane & 16) + 4 * (lane & 3);

  // Grid: x = (layer, query head); y = tile rank, so that every sequence's
  // longest (last) query tiles come first; z = sequence in the slice, read
  // straight from the grid so that its length and offsets load in the first
  // scalar round.
  const int head = blockIdx.x;
  const int rank = blockIdx.y;
  const int bb = blockIdx.z;
  // Every kernel argument the prologue needs, fetched in one scalar round
  // (the empty asm takes them all as operands, so none of their loads is
  // deferred behind the early exit or the index arithmetic).
  const int S = a.len[bb];   // new tokens of this sequence
  const int P = HIST ? a.hist[bb] : 0;  // positions already cached
  const uint32_t q_row0 = a.q_row0[bb], kv_row0 = a.kv_row0[bb];
  const int Hq = a.Hq, group = a.group, Bn = a.B, Hkv = a.Hkv, Tmax = a.Tmax;
  const int layer0 = a.layer0, b0 = a.b0;
  const int64_t q_sl = a.q_sl, kv_sl = a.kv_sl;
  const int q_sh = a.q_sh, q_si = a.q_si, kv_sh = a.kv_sh, kv_si = a.kv_si;
  const char *qp = a.q, *kp_in = a.k, *vp_in = a.v;
  char *kcp = a.k_cache, *vcp = a.v_cache;
  asm volatile("" ::"s"(S), "s"(P), "s"(q_row0), "s"(kv_row0), "s"(Hq), "s"(group), "s"(Bn),
               "s"(Hkv), "s"(Tmax), "s"(layer0), "s"(b0), "s"(q_sl), "s"(kv_sl), "s"(q_sh),
               "s"(q_si), "s"(kv_sh), "s"(kv_si), "s"(qp), "s"(kp_in), "s"(vp_in), "s"(kcp),
               "s"(vcp));
  const int qt = (S + BM - 1) / BM - 1 - rank;
  if (qt < 0) return;
  // Issue priority: a query tile with at most half the key tiles of the
  // sequence's last one outranks the longer ones it shares a CU with.  The
  // arbiter otherwise favours the oldest waves, so all workgroups resident
  // on a CU finish together and the short tiles still queued run last, a few
  // per CU; with the short ones first, their slots turn over early.  Short
  // sequences (under four query tiles) gain nothing and keep the default.
  // Measured: causal bf16 S=1024 45.5 -> 43 us.
  if (S > 3 * BM && 2 * ((P + qt * BM + BM + BN - 1) / BN) <= (P + S + BN - 1) / BN)
    __builtin_amdgcn_s_setprio(2);
  const int hq = head % Hq;
  const int l = head / Hq;
  const int b = b0 + bb;
  const int hkv = hq / group;
  const bool writer = (hq % group) == 0;
  const int q0 = qt * BM;
  const int qrow = q0 + rg * 32 + col;              // this lane's new token
  const int wave_last = P + q0 + rg * 32 + 31;      // last position the wave's rows see
  const int q_end = (q0 + BM < S) ? q0 + BM : S;
  const int kv_end = P + q_end;                     // positions this tile needs

  // New token i of this sequence: q / o at qbase + i * q_stride, its k / v
  // at kin / vin + i * kv_stride.  Cached position j at kcache / vcache + j * RB.
  const size_t q_off = ((size_t)l * q_sl + (size_t)hq * q_sh + q_row0) * RB;
  const char *qbase = qp + q_off;
  const size_t q_stride = (size_t)q_si * RB;
  const size_t kv_in = ((size_t)l * kv_sl + (size_t)hkv * kv_sh + kv_row0) * RB;
  const char *kin = kp_in + kv_in;
  const char *vin = vp_in + kv_in;
  const size_t kv_stride = (size_t)kv_si * RB;
  const size_t crow0 = (((size_t)(layer0 + l) * Bn + b) * Hkv + hkv) * (size_t)Tmax;
  char *kcache = kcp + crow0 * RB;
  char *vcache = vcp + crow0 * RB;

  // Q fragments, resident for the whole kernel.
  //   bf16: qv[ds] = Q[qrow][16 ds + 8 h .. +7]        (B operand of 32x32x16)
  //   fp32: qv[j]  = Q[qrow][8 j + 4 h .. +3]           (4 B operands of 32x32x2)
  //   Rows past the sequence read its last row (valid, finite); their
  //   outputs are never written.
  constexpr int QV = (DT == KVC_BF16) ? D / 16 : D / 8;
  u32x4 qv[QV];
  const char *qrow_p = qbase + (size_t)(qrow < S ? qrow : S - 1) * q_stride;
  const uint32_t q_keep = a.q_keep, q_flip = a.q_flip;
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const int d0 = (DT == KVC_BF16) ? 16 * j + 8 * h : 8 * j + 4 * h;
    // the sign of the score scale (a zero scale zeroes q)
    qv[j] = (*reinterpret_cast<const u32x4 *>(qrow_p + d0 * EB) & q_keep) ^ q_flip;
  }

  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;

  const int n_kt = (kv_end + BN - 1) / BN;
  // Tiles every wave needs: the first key of every wave's block is at most
  // the position of the first row.  At most two more follow, which some
  // waves skip.
  const int first_last = P + q0 + 31 - 32 * KBW * (KS - 1);
  const int n_all_raw = first_last >= 0 ? first_last / BN + 1 : 0;
  const int n_all = n_all_raw < n_kt ? n_all_raw : n_kt;

  // Tile staging.  Each thread moves VPT 16-byte vectors of K and of V per
  // tile, from pairs of adjacent keys (rows 2p and 2p+1) at the same column
  // c; K and V land in LDS row-major, one 16-byte store per vector.
  // Tile kt+1 is loaded into registers while tile kt is computed.  Positions
  // past kv_end are clamped to its last one (always valid): their scores are
  // masked, so no load needs a branch.  Positions below P come from the
  // cache, the others from the new rows.
  auto tile_row = [&](int it) { return 2 * (tid / LPR + (it >> 1) * (256 / LPR)) + (it & 1); };
  // Rows of one wave for one pair of vectors (it = 2 g, 2 g + 1): a
  // kGroup-aligned run of kGroup = 128 / LPR consecutive rows.
  constexpr int kGroup = 128 / LPR;
  constexpr int kGroupLog2 = kGroup == 4 ? 2 : kGroup == 8 ? 3 : 4;
  static_assert(VPT % 2 == 0 && (kGroup == 4 || kGroup == 8 || kGroup == 16), "row groups");
  const int c = tid % LPR;
  u32x4 kreg[VPT], vreg[VPT];
  // Byte offset of this thread's rows inside a tile of new rows (loop
  // invariant, so the common tile costs no per-lane multiply).
  size_t in_off[VPT];
#pragma unroll
  for (int it = 0; it < VPT; ++it) in_off[it] = (size_t)tile_row(it) * kv_stride + c * 16;
  // Cached position `key` of this (layer, sequence, KV head): contiguous
  // rows, or its slot through the block table.
  auto cache_ptr = [&](char *contig, char *pool, int key) -> char * {
    if constexpr (PAGED)
      return pool + paged_row(a.pg, b, key, layer0 + l, hkv, Hkv) * RB;
    else
      return contig + (size_t)key * RB;
  };
  auto load_tile = [&](int kt) {
    const int tk0 = kt * BN;
    if (HIST && !PAGED && tk0 + BN <= P) {
      // the whole tile is cached rows of a contiguous cache
#pragma unroll
      for (int it = 0; it < VPT; ++it) {
        const size_t off = (size_t)(tk0 + tile_row(it)) * RB + c * 16;
        kreg[it] = *reinterpret_cast<const u32x4 *>(kcache + off);
        vreg[it] = *reinterpret_cast<const u32x4 *>(vcache + off);
      }
    } else if (HIST && PAGED && tk0 + BN <= P && a.pg.bs_log2 >= kGroupLog2) {
      // The whole tile is cached rows of a paged pool whose blocks hold at
      // least G = 128 / LPR positions: the G rows a wave loads with each
      // pair of vectors are G-aligned, so they lie in one block and its id
      // is the same in all the wave's lanes -- one scalar load per pair.
      const int32_t *tbl = a.pg.block_table + (size_t)b * a.pg.max_blocks;
      int blk[VPT / 2];
#pragma unroll
      for (int g = 0; g < VPT / 2; ++g) {
        const int r0 = __builtin_amdgcn_readfirstlane(tile_row(2 * g) & ~(kGroup - 1));
        blk[g] = uniform_load(tbl + ((tk0 + r0) >> a.pg.bs_log2));
      }
      __builtin_amdgcn_sched_barrier(0);
      const int nb = a.pg.num_blocks, bmask = (1 << a.pg.bs_log2) - 1;
#pragma unroll
      for (int it = 0; it < VPT; ++it) {
        const int key = tk0 + tile_row(it);
        const int bk = blk[it >> 1] < 0 ? 0 : (blk[it >> 1] >= nb ? nb - 1 : blk[it >> 1]);
        const size_t prow = ((((size_t)(layer0 + l) * nb + bk) * Hkv + hkv) << a.pg.bs_log2) +
                            (size_t)(key & bmask);
        kreg[it] = *reinterpret_cast<const u32x4 *>(kcp + prow * RB + c * 16);
        vreg[it] = *reinterpret_cast<const u32x4 *>(vcp + prow * RB + c * 16);
      }
    } else if (tk0 + BN <= kv_end && (!HIST || tk0 >= P)) {
      // the whole tile is new rows, none past kv_end
      const size_t base = (size_t)(tk0 - P) * kv_stride;
#pragma unroll
      for (int it = 0; it < VPT; ++it) {
        kreg[it] = *reinterpret_cast<const u32x4 *>(kin + base + in_off[it]);
        vreg[it] = *reinterpret_cast<const u32x4 *>(vin + base + in_off[it]);
      }
    } else {
#pragma unroll
      for (int it = 0; it < VPT; ++it) {
        const int key0 = tk0 + tile_row(it);
        const int key = key0 < kv_end ? key0 : kv_end - 1;
        const char *kp, *vp;
        if (HIST && key < P) {
          kp = cache_ptr(kcache, kcp, key);
          vp = cache_ptr(vcache, vcp, key);
        } else {
          kp = kin + (size_t)(key - P) * kv_stride;
          vp = vin + (size_t)(key - P) * kv_stride;
        }
        kreg[it] = *reinterpret_cast<const u32x4 *>(kp + c * 16);
        vreg[it] = *reinterpret_cast<const u32x4 *>(vp + c * 16);
      }
    }
  };
  load_tile(0);

  // Stage tile kt in LDS (and in the cache when it is ours to write), then
  // start loading tile kt + 1.
  // The new rows of this query tile's tokens, positions [P + q0, kv_end),
  // are this workgroup's to write to the cache (the first query head of a
  // group writes them).
  auto stage = [&](int kt) {
    const int key0 = kt * BN;
    const bool store_cache = writer && key0 + BN > P + q0;
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int it = 0; it < VPT; ++it) {
      const int row = tile_row(it);
      const int key = key0 + row;
      if (store_cache && key >= P + q0 && key < kv_end) {
        // streaming stores: nothing in this call reads these rows back
        __builtin_nontemporal_store(kreg[it], reinterpret_cast<u32x4 *>(cache_ptr(kcache, kcp, key) + c * 16));
        __builtin_nontemporal_store(vreg[it], reinterpret_cast<u32x4 *>(cache_ptr(vcache, vcp, key) + c * 16));
      }
      *reinterpret_cast<u32x4 *>(&sm.k[row * Smem<DT, D>::kKStride + c * EV]) = kreg[it];
      *reinterpret_cast<u32x4 *>(&sm.v[row * Smem<DT, D>::kVStride + c * EV]) = vreg[it];
    }
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);
  };

  auto compute = [&](int kt) {
    const int key0 = kt * BN;
    // S^T blocks: acc_s[kb][i] = score of key key0 + kb0 + 32 kb + 8 (i/4) +
    // 4 h + i%4 for query qrow.
    // The KBW accumulator chains are interleaved so that consecutive MFMAs are
    // independent.
    f32x16 acc_s[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) acc_s[kb] = f32x16{};
    if constexpr (DT == KVC_BF16) {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const u32x4 kf = *reinterpret_cast<const u32x4 *>(
              &sm.k[(kb0 + 32 * kb + col) * Smem<DT, D>::kKStride + 16 * ds + 8 * h]);
          acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qv[ds]), acc_s[kb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 qf = __builtin_bit_cast(f32x4, qv[j]);
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const f32x4 kf = *reinterpret_cast<const f32x4 *>(
              &sm.k[(kb0 + 32 * kb + col) * Smem<DT, D>::kKStride + 8 * j + 4 * h]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[r], qf[r], acc_s[kb], 0, 0, 0);
        }
      }
    }

    // Causal mask, only on tiles that reach past the position of the wave's
    // first row or past kv_end (a wave-uniform branch).  Key key0 + 32 kb +
    // 8 (i/4) + 4 h + i%4 is visible iff it is <= P + qrow and < kv_end,
    // i.e. iff the compile-time offset 32 kb + 8 (i/4) + i%4 is <= lim.
    if ((key0 + kb0 + 32 * KBW - 1 > P + q0 + rg * 32) || (key0 + kb0 + 32 * KBW > kv_end)) {
      const int lim = (P + qrow < kv_end - 1 ? P + qrow : kv_end - 1) - key0 - kb0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) acc_s[kb][i] = kNegInf;
      }
    }
    // Online softmax for this lane's query, in log2 units: the raw scores are
    // maximised first (sc is positive -- the scale's sign sits on q -- so
    // scaling commutes with max and a masked -inf stays -inf) and the scale
    // is folded into the exponent, p = 2^(s sc - m), one FMA per score.
    const float sc = a.scale_log2;
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, acc_s[kb][i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * sc;
    // Lazy rescale: the running max only moves when this tile raises it by
    // more than 8 (log2 domain), so probabilities stay <= 2^8 and the output
    // rescale is skipped whenever no lane of the wave needs it.  Subtracting
    // any constant leaves the softmax unchanged.
    const bool grow = mt > m_run + 8.f;  // also true on the first tile
    const float m_new = grow ? mt : m_run;
    // Under the key split a query can have seen no visible key yet in its
    // wave's half (its max still -inf); subtracting 0 instead keeps its
    // weights 0 rather than 2^(-inf + inf).  Without the split the first tile
    // holds key 0, which every query sees.
    const float m_sub = (KS == 2 && m_new == kNegInf) ? 0.f : m_new;
    if (__any(grow)) {
      const float alpha = fast_exp2(m_run - m_sub);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(acc_s[kb][i], sc, -m_sub));
        acc_s[kb][i] = p;
        if constexpr (DT != KVC_BF16) psum += p;  // bf16: summed below, as rounded
      }
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      if constexpr (DT == KVC_BF16) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pw;
          // The row sum adds the same bf16-rounded p that the PV product
          // uses, two per v_dot2 against (1, 1): half the adds, and the
          // normalised weights sum to one.  (The packed word goes through a
          // scalar first: a bit_cast of the vector element itself made the
          // compiler feed element 0 to every dot2.)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t pk = pack_bf16x2(acc_s[kb][8 * t + 2 * j], acc_s[kb][8 * t + 2 * j + 1]);
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                   __builtin_bit_cast(bf16x2, 0x3f803f80u), psum, false);
            pw[j] = pk;
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            // keys 32 kb + 16 t + {0-3, 8-11} (low half-wave) or {4-7, 12-15}
            // (high), the order of pw; this lane's d = 32 db + col
            const uint16_t *vb = &sm.v[(kb0 + 32 * kb + 16 * t) * Smem<DT, D>::kVStride + 32 * db + v_tr_off];
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)vb);
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)(vb + 8 * Smem<DT, D>::kVStride));
            const v8i16 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pw), acc_o[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int vrow = kb0 + 32 * kb + 8 * (s >> 2) + 4 * h + (s & 3);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float vf = sm.v[vrow * Smem<DT, D>::kVStride + 32 * db + col];
            acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, acc_s[kb][s], acc_o[db], 0, 0, 0);
          }
        }
      }
    }
    l_run += psum;
  };

  // Every wave computes the first n_all tiles; the at most two after them
  // (first key past the position of the tile's first row, within 96 of it)
  // are skipped by the waves whose rows all lie before them.  The skip tests
  // sit outside the loop: inside it the compiler copies the accumulators on
  // every iteration.
  for (int kt = 0; kt < n_all; ++kt) {
    stage(kt);
    compute(kt);
  }
  if (n_all < n_kt) {
    stage(n_all);
    if (n_all * BN + kb0 <= wave_last) compute(n_all);
  }
  if (n_all + 1 < n_kt) {
    stage(n_all + 1);
    if ((n_all + 1) * BN + kb0 <= wave_last) compute(n_all + 1);
  }

  if constexpr (KS == 2) {
    // The two waves of a row group hold online-softmax states over disjoint
    // keys, each relative to its own running max: wave kh = 1 hands its
    // state over through LDS (register j of every lane, lanes contiguous)
    // and wave kh = 0 rescales both to the larger max and adds them.
    constexpr int NO = DB * 16;
    float *st = reinterpret_cast<float *>(&sm) + rg * (NO + 2) * 64;
    static_assert(RG * (NO + 2) * 64 * 4 <= (int)sizeof(Smem<DT, D>), "state hand-over fits");
    __syncthreads();  // every wave is done with the last tile's K / V
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[(16 * db + i) * 64 + lane] = acc_o[db][i];
      st[NO * 64 + lane] = m_run;
      st[(NO + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (kh == 0) {
      const float m1 = st[NO * 64 + lane], l1 = st[(NO + 1) * 64 + lane];
      const float m = fmaxf(m_run, m1);
      const float f0 = fast_exp2(m_run - m), f1 = fast_exp2(m1 - m);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] = acc_o[db][i] * f0 + st[(16 * db + i) * 64 + lane] * f1;
      l_run = l_run * f0 + l1 * f1;
    }
  }

  // Normalise and write O.  The wave's 32 x D outputs go through its own
  // slice of the (now free) K/V staging area, so that every global store is
  // a whole 16-byte piece of a row and one wave instruction writes whole rows
  // (lane (col, h) holds d = 32 db + 8 g + 4 h + 0..3 of row col).  The
  // stores are streaming: written straight through instead of filling the L2
  // with lines the call never reads, which otherwise all had to be written
  // back when the kernel ends (bf16 S=1024: 43-44 -> 37-39 us).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  constexpr int ORB = D * EB + (DT == KVC_BF16 ? 16 : 8);  // LDS row pitch (bytes)
  static_assert(4 * 32 * ORB <= (int)sizeof(Smem<DT, D>), "output staging fits");
  constexpr int R16 = D * EB / 16;  // 16-byte pieces per row
  const float inv = 1.f / l_tot;
  char *ow = reinterpret_cast<char *>(&sm) + rg * 32 * ORB;
  __syncthreads();  // every wave is done with the last tile's K / V (and the hand-over)
  if (kh != 0) return;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * h;
      const float o0 = acc_o[db][4 * g] * inv, o1 = acc_o[db][4 * g + 1] * inv;
      const float o2 = acc_o[db][4 * g + 2] * inv, o3 = acc_o[db][4 * g + 3] * inv;
      if constexpr (DT == KVC_BF16)
        *reinterpret_cast<u32x2 *>(ow + col * ORB + d0 * EB) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      else
        *reinterpret_cast<f32x4 *>(ow + col * ORB + d0 * EB) = f32x4{o0, o1, o2, o3};
    }
  }
  __builtin_amdgcn_wave_barrier();  // the slice is this wave's alone
#pragma unroll
  for (int it = 0; it < 32 * R16 / 64; ++it) {
    const int idx = lane + 64 * it;
    const int r = idx / R16, ch = idx % R16;
    const u32x4 val = *reinterpret_cast<const u32x4 *>(ow + r * ORB + ch * 16);
    const int tok = q0 + rg * 32 + r;
    if (tok < S)
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(a.o + q_off + (size_t)tok * q_stride + ch * 16));
  }
}

// Register budgets: at D = 64, three workgroups per CU for bf16 and two for
// fp32; D = 128 keeps one, since capping it would spill.  KS: key split (2
// only for fp32 at D = 64, see prefill_key_split).  HIST: some sequence has
// cached positions before its new tokens; PAGED: the cache is a paged pool.
template <int DT, int KS, bool HIST, bool PAGED>
__global__ __launch_bounds__(256, DT == KVC_BF16 ? 3 : 2) void prefill_kernel_d64(PrefillArgs a) {
  prefill_tile<DT, 64, KS, HIST, PAGED>(a);
}
template <int DT, bool HIST, bool PAGED>
__global__ __launch_bounds__(256) void prefill_kernel_d128(PrefillArgs a) {
  prefill_tile<DT, 128, 1, HIST, PAGED>(a);
}

template <int DT, bool HIST, bool PAGED>
void launch_dt(const PrefillArgs &a, int D, int ks, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_layers * a.Hq), (unsigned)a.q_tiles, (unsigned)a.nb);
  if (D == 128)
    hipLaunchKernelGGL((prefill_kernel_d128<DT, HIST, PAGED>), grid, dim3(256), 0, s, a);
  else if constexpr (DT == KVC_F32)
    if (ks == 2)
      hipLaunchKernelGGL((prefill_kernel_d64<DT, 2, HIST, PAGED>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel_d64<DT, 1, HIST, PAGED>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel_d64<DT, 1, HIST, PAGED>), grid, dim3(256), 0, s, a);
}

template <int DT>
void launch_flags(const PrefillArgs &a, int D, bool history, int ks, hipStream_t s) {
  const bool paged = a.pg.block_table != nullptr;
  if (paged) {
    if (history) launch_dt<DT, true, true>(a, D, ks, s);
    else launch_dt<DT, false, true>(a, D, ks, s);
  } else {
    if (history) launch_dt<DT, true, false>(a, D, ks, s);
    else launch_dt<DT, false, false>(a, D, ks, s);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int D, bool history, int ks, hipStream_t s) {
  if (a.q_tiles <= 0 || a.nb <= 0) return hipSuccess;
  if (ks != 1 && !(ks == 2 && dtype == KVC_F32 && D == 64)) return hipErrorInvalidValue;
  if (dtype == KVC_F32) launch_flags<KVC_F32>(a, D, history, ks, s);
  else launch_flags<KVC_BF16>(a, D, history, ks, s);
  return hipGetLastError();
}

// Key split for a call whose one-split grid has `workgroups` workgroups on a
// device of `cus` compute units.  fp32 at D = 64 is bound by the matrix
// cores, so two waves per row group, each taking half of every key tile,
// halve a workgroup's longest chain; that pays while the grid is small
// (fewer than two workgroups per CU: short prompts, single layers), and
// costs the doubled tile staging on larger grids.  Measured (12 layers,
// H=12, cold): fp32 S=256 35.5 -> 25.3 us; S=1024 200 -> 204 us (kept at 1);
// bf16 S=256 10.2 -> 10.8 us (kept at 1).
int prefill_key_split(int dtype, int D, long long workgroups, int cus) {
  return (dtype == KVC_F32 && D == 64 && workgroups < 2LL * cus) ? 2 : 1;
}

int prefill_query_tile(int ks) { return 32 * 4 / ks; }

}  // namespace kvc
