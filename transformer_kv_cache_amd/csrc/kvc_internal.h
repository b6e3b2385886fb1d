// kvc_internal.h -- shared definitions of the HIP kernels and their host
// launchers inside libkvcache.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvcache.h"

namespace kvc {

// Sequences carried per launch in the kernel-argument block.  Larger batches
// are split into several launches over batch slices.
constexpr int kMaxBatchPerLaunch = 64;

// 16-byte vector moved by one lane per global load or store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Dtype;
template <> struct Dtype<KVC_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;  // elements per 16-byte vector
};
template <> struct Dtype<KVC_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};

// Widen a 16-byte vector into fp32 values (bf16 widening is exact).
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4 &w, float *out);
template <>
__device__ __forceinline__ void unpack16<KVC_F32>(const u32x4 &w, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
}
template <>
__device__ __forceinline__ void unpack16<KVC_BF16>(const u32x4 &w, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Store n consecutive fp32 values as the output element type.
template <int DT>
__device__ __forceinline__ void store_elems(void *base, size_t index, const float *v, int n);
template <>
__device__ __forceinline__ void store_elems<KVC_F32>(void *base, size_t index, const float *v, int n) {
  float *p = reinterpret_cast<float *>(base) + index;
  for (int i = 0; i < n; ++i) p[i] = v[i];
}
template <>
__device__ __forceinline__ void store_elems<KVC_BF16>(void *base, size_t index, const float *v, int n) {
  uint16_t *p = reinterpret_cast<uint16_t *>(base) + index;
  for (int i = 0; i < n; ++i) p[i] = (uint16_t)f32_to_bf16_rne(v[i]);
}

// ---- launch descriptors (passed by value as kernel arguments) -------------

// Paged cache geometry: K and V are pools [L][num_blocks][Hkv][block_size][D]
// and position t of sequence b is row t % block_size of block
// block_table[b][t / block_size].  block_table == nullptr for the contiguous
// [L][B][Hkv][Tmax][D] cache.
struct PagedGeom {
  const int32_t *block_table;  // device, [B][max_blocks]
  int32_t max_blocks, num_blocks, bs_log2;
};

// Row index (in rows of D elements) of position t of sequence b, KV head h,
// layer `layer` of a paged pool.  Block ids outside [0, num_blocks) are
// clamped, so a bad table can give wrong results but never reads or writes
// outside the pools.
__device__ __forceinline__ size_t paged_row(const PagedGeom &p, int b, int t, int layer, int h,
                                            int Hkv) {
  int blk = p.block_table[(size_t)b * p.max_blocks + (t >> p.bs_log2)];
  blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
  return ((((size_t)layer * p.num_blocks + blk) * Hkv + h) << p.bs_log2) +
         (size_t)(t & ((1 << p.bs_log2) - 1));
}

// A load whose address is the same in every lane, through the constant
// address space so that it becomes a scalar load.
__device__ __forceinline__ int uniform_load(const int32_t *p) {
  return *(const __attribute__((address_space(4))) int32_t *)(p);
}

// Pool rows of KPL groups of NRG consecutive positions of sequence b: group
// kk holds positions first + kk * NRG + lane_off for lane_off in [0, NRG),
// clamped to last_pos.  Call only when the block size is at least NRG and
// `first` is a multiple of NRG: then every group lies in one block, so its
// id is the same in all lanes and the KPL ids are fetched as scalar loads,
// all in flight together, instead of one vector load per lane and key.
// Block ids are clamped into the pool as in paged_row.
template <int KPL, int NRG>
__device__ __forceinline__ void paged_rows_grouped(const PagedGeom &p, int b, int first, int last_pos,
                                                   int lane_off, int layer, int h, int Hkv,
                                                   size_t (&prow)[KPL]) {
  const int32_t *tbl = p.block_table + (size_t)b * p.max_blocks;
  int blk[KPL];
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    const int g0 = first + kk * NRG;
    blk[kk] = uniform_load(tbl + ((g0 < last_pos ? g0 : last_pos) >> p.bs_log2));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KPL; ++kk) {
    const int pos0 = first + kk * NRG + lane_off;
    const int pos = pos0 < last_pos ? pos0 : last_pos;
    const int bk = blk[kk] < 0 ? 0 : (blk[kk] >= p.num_blocks ? p.num_blocks - 1 : blk[kk]);
    prow[kk] = ((((size_t)layer * p.num_blocks + bk) * Hkv + h) << p.bs_log2) +
               (size_t)(pos & ((1 << p.bs_log2) - 1));
  }
}

struct AppendArgs {
  char *k_cache, *v_cache;
  const char *k_new, *v_new;
  int32_t B, Hkv, Tmax;
  int32_t layer0, n_layers, N;
  int32_t b0, nb;       // batch slice [b0, b0+nb) of this launch
  int32_t row_vec16;    // 16-byte vectors per row (D * elem / 16)
  PagedGeom pg;         // paged cache, else block_table == nullptr
  int32_t hist[kMaxBatchPerLaunch];
};

struct DecodeArgs {
  char *k_cache, *v_cache;    // written only by the fused step (new rows)
  const char *k_new, *v_new;  // fused step: the N new rows, [n_layers,B,Hkv,N,D]
  const char *q;
  char *o;
  float *ws_o;       // [max_splits][ws_rows][D] unnormalised partial outputs
  float *ws_ml;      // [max_splits][ws_rows][2] partial (max, sum), log2 domain
  int64_t ws_rows;   // query rows of the call: n_layers * B * Hq * N
  int32_t B, Hkv, Hq, Tmax, N;
  int32_t layer0, n_layers;
  int32_t group;       // Hq / Hkv
  int32_t rows;        // G * N query rows per (layer, sequence, KV head)
  int32_t row_tiles;   // ceil(rows / row tile)
  int32_t max_splits;  // workspace stride in splits
  int32_t split_keys;  // keys per split of the launched kernel
  int32_t b0, nb;
  float scale_log2;    // scale * log2(e)
  uint32_t hkv_div;    // div_magic multiplier for Hkv
  uint32_t split_div;  // div_magic multiplier for split_keys
  int32_t tail;        // 1 (vector kernel): the split states cover keys
                       // [0, P) and the combine adds key P
  // Vector kernel: one-dimensional grid of 8 * ceil(units / 8) * grid_splits
  // workgroups (units = n_layers * nb * Hkv query rows), and the per-row
  // arrival counters of the in-launch merge (zero before and after a call).
  uint64_t *counters;
  int32_t units, grid_splits;
  uint32_t grid_splits_div;  // div_magic multiplier for grid_splits
  uint32_t nl_div;           // div_magic multiplier for n_layers
  PagedGeom pg;        // paged cache, else block_table == nullptr
  // Device lengths (kvc_decode_step_dl): hist_dev[b0 + bb] clamped into
  // [0, hist_max] replaces hist[bb]; null for host lengths.
  const int32_t *hist_dev;
  int32_t hist_max;
  int32_t hist[kMaxBatchPerLaunch];
};

// Workspace slot of query row `row` (index into the call's
// [n_layers, B, Hq, N] rows) and split `split`, split-major: the rows a
// workgroup writes for one split are contiguous, and the next (layer, head)
// unit's rows for the same split follow them.
__device__ __forceinline__ size_t ws_slot(const DecodeArgs &a, long long row, int split) {
  return (size_t)split * (size_t)a.ws_rows + (size_t)row;
}

// Cached positions of sequence bb of the launch slice: the host value from
// the kernel arguments, or with DEVLEN the device array, clamped so that a
// wrong value can give wrong results but no access outside the cache.
template <bool DEVLEN>
__device__ __forceinline__ int seq_hist(const DecodeArgs &a, int bb) {
  if constexpr (DEVLEN) {
    const int v = a.hist_dev[a.b0 + bb];
    return v < 0 ? 0 : (v > a.hist_max ? a.hist_max : v);
  } else {
    return a.hist[bb];
  }
}

// floor(2^32 / d) capped at 2^32 - 1: the multiplier div_magic uses for d.
inline uint32_t magic_for(int d) {
  const unsigned long long m = (1ull << 32) / (unsigned long long)d;
  return m > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)m;
}

// floor(n / d) for 0 <= n < 2^31 and d >= 1, with m = magic_for(d).  m falls
// short of 2^32 / d by less than one, so n m / 2^32 lies in (n/d - 1, n/d]:
// umulhi(n, m) is floor(n / d) or one less, and one compare fixes it.
__device__ __forceinline__ int div_magic(int n, int d, uint32_t m) {
  int q = (int)__umulhi((uint32_t)n, m);
  if (n - q * d >= d) ++q;
  return q;
}

// Prefill of S_b new tokens per sequence on top of P_b cached positions,
// for a batch slice [b0, b0 + nb).  q / o and the new k / v rows are
// addressed through strides, in rows of D elements:
//   row(l, sequence, h, i) = l * sl + h * sh + row0[sequence] + i * si
// which covers both the padded [n_layers, B, H, S, D] layout and the packed
// token-major [n_layers, T, H, D] one.
struct PrefillArgs {
  char *k_cache, *v_cache;
  const char *q, *k, *v;
  char *o;
  int32_t B, Hkv, Hq, Tmax;
  int32_t layer0, n_layers, group;
  int32_t b0, nb;
  int32_t q_tiles;      // most query tiles of one sequence in the slice
  // |scale| * log2(e) (log2(e) when scale is 0).  The kernel takes the max of
  // the raw scores and folds this positive factor into the exponent; the
  // sign of the scale is moved onto q instead: each 32-bit word of q is
  // replaced by (word & q_keep) ^ q_flip -- the sign bits flipped for a
  // negative scale, q zeroed for a zero one (exact in both cases).
  float scale_log2;
  uint32_t q_keep, q_flip;
  int64_t q_sl, kv_sl;
  int32_t q_sh, q_si, kv_sh, kv_si;
  int32_t hist[kMaxBatchPerLaunch];     // P_b
  int32_t len[kMaxBatchPerLaunch];      // S_b
  uint32_t q_row0[kMaxBatchPerLaunch];  // row0 of q / o
  uint32_t kv_row0[kMaxBatchPerLaunch]; // row0 of k / v
  PagedGeom pg;         // paged cache, else block_table == nullptr
};

// Dense layer of a decode step: y = act(LN?(x) W + bias) + res, fp32, for at
// most kMaxLinearRows rows (kvc_linear_f32).
constexpr int kMaxLinearRows = 8;
constexpr int kMaxLinearInputs = 12288;  // M * K floats staged in LDS (48 KiB)
struct LinearArgs {
  const float *x;      // [M][K]
  const float *wt;     // [N][K]
  const float *bias;   // [N] or null
  const float *ln_g;   // [K] or null (no layer norm)
  const float *ln_b;   // [K] (with ln_g)
  const float *res;    // [M][N] or null
  float *y;            // [M][N]
  int32_t M, K, N;
  int32_t act;         // 0: none, 1: GELU (tanh form)
  float ln_eps;
  int32_t a_heads;     // > 0: x is head-major [H][M][K/H]
  int32_t y_qkv_heads; // > 0: y is [3][H][M][N/(3H)]
};

// Dense layer of a prompt on the matrix cores (kvc_gemm_f32):
// y = act(a wt^T + bias) + res.  a is [M][K] row-major, or head-major
// [a_heads][M][K / a_heads]; wt is [N][K]; y is [M][N] row-major, or with
// y_qkv_heads = H the attention layout [3][H][M][N / (3 H)].  res is
// [M][N] row-major.
struct GemmArgs {
  const float *a, *wt, *bias, *res;
  float *y;
  int32_t M, K, N;
  int32_t act;          // 0: none, 1: GELU (tanh form)
  int32_t a_heads;      // 0: row-major a
  int32_t y_qkv_heads;  // 0: row-major y
  // Split of K over `splits` workgroups per output tile (1: none).  Each
  // writes its partial tile to part[split][tile][64 x 64]; the last one to
  // arrive on the tile's counter (ctr[tile], zero before the call and left
  // zero) sums them in split order and applies the epilogue.
  int32_t splits;
  int32_t tiles_m, tiles_n;
  float *part;
  uint64_t *ctr;
};

// K split of a kvc_gemm_f32 call (1 when the output tiles alone fill the
// chip) and the workspace it needs (0 without a split): kGemmCounterBytes of
// arrival counters (one per tile; splits only happen below 256 tiles), then
// the partial tiles.
constexpr size_t kGemmCounterBytes = 256 * sizeof(uint64_t);
int gemm_splits(int M, int K, int N);
size_t gemm_workspace_bytes(int M, int K, int N, int splits);

// Row-wise layer norm (kvc_layernorm_f32): y = (x - mean) / sqrt(var + eps)
// * g + b over the K features of each of M rows.
struct LayerNormArgs {
  const float *x, *g, *b;
  float *y;
  int32_t M, K;
  float eps;
};

// Token + position embedding (kvc_embed_f32).
struct EmbedArgs {
  const float *wte, *wpe;
  const int64_t *ids;
  const int32_t *pos;  // device start position, or null (then pos0)
  float *y;
  int32_t V, T, d, N, pos0;
};

// Greedy token choice (kvc_argmax_f32).
struct ArgmaxArgs {
  const float *x;
  int64_t *index;
  int64_t *seq, *seq_pos;  // token history and its device counter, or null
  int64_t cap;
  int32_t n;
};

// Host launchers (one translation unit each).  They assume validated
// arguments and return the launch status.
hipError_t launch_linear(const LinearArgs &a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);
hipError_t launch_layernorm(const LayerNormArgs &p, hipStream_t s);
hipError_t launch_embed(const EmbedArgs &e, hipStream_t s);
hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t s);
hipError_t launch_lengths_add(int32_t *hist, int B, int n, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, int dtype, int D, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int D, int kpl, bool merge, hipStream_t s);
// One workgroup per query row (G = N = 1, grid = a.units): the whole key
// range and the merge with key P in one workgroup, no workspace state.
hipError_t launch_decode_row(const DecodeArgs &a, int dtype, int D, hipStream_t s);
// Longest block table (blocks per sequence) launch_decode_row takes.
int decode_row_max_blocks();
hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int D, int splits,
                              bool fused_append, hipStream_t s);
hipError_t launch_decode_rows(const DecodeArgs &a, int dtype, int D, int splits,
                              bool fused_append, hipStream_t s);
// decode_rows_kernel's rows with one workgroup per (layer, sequence, KV
// head) over the whole key range, writing o directly (grid x = n_layers *
// Hkv, z = nb); paged caches with at most decode_rows_loop_max_blocks
// blocks per sequence.
hipError_t launch_decode_rows_loop(const DecodeArgs &a, int dtype, int D, bool fused, hipStream_t s);
int decode_rows_loop_max_blocks();
hipError_t launch_combine(const DecodeArgs &a, int dtype, int D, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int D, bool history, int ks, hipStream_t s);
// Key split (1 or 2) of a prefill call whose grid at key split 1 has
// `workgroups` workgroups, on `cus` compute units; query rows per workgroup
// at key split ks.
int prefill_key_split(int dtype, int D, long long workgroups, int cus);
int prefill_query_tile(int ks);

// Geometry shared by kvc_decode_workspace_bytes and the decode launchers.
// One query row per KV head runs on the vector kernel; a few rows with
// 256-byte key rows (GQA groups, short chunks) on the multi-row vector
// kernel; other multi-row calls on the matrix-core kernel in tiles of 16 rows.
// Single-row kernel: a split covers decode_rows_per_load * kpl keys, kpl 4
// or 8 chosen per call.
int decode_rows_per_load(int dtype, int D);
int decode_mfma_split_keys(int dtype, int D);
// Multi-row vector kernel: 2 <= rows <= 8, fp32 with D = 64 (256-byte key
// rows) or bf16 with D = 128 or 64 (256- or 128-byte rows); all rows in one
// tile.
bool decode_rows_fits(int dtype, int D, int rows);
int decode_rows_split_keys(int dtype, int D);
constexpr int kMfmaRowTile = 16;

}  // namespace kvc
