/*
 * kvcache.h -- C ABI of libkvcache.so: attention over a per-layer KV cache on
 * an AMD Instinct MI355X (gfx950).
 *
 * Three operations make up the hot path of autoregressive GPT-2-style
 * generation with a KV cache:
 *
 *   kvc_append        write the new K/V rows of a step into the cache
 *   kvc_attn_decode   N >= 1 new query rows against the P+N cached keys
 *   kvc_attn_prefill  causal self-attention over a whole prompt, which also
 *                     writes the prompt's K/V into the cache
 *
 * Pages defining the operations (cited by address and section title):
 *   [KV-1] gitcode.csdn.net/69e62cef0a2f6a37c5a11c4f.html
 *          "KV Cache 原理", "Prefill/Decode 双图", "Decode Shape 示例"
 *   [KV-2] openai-hub.com/news/2435 "GPT-2缓存实测：千倍计算只快6倍"
 *          "正确性先于性能", "一个很容易漏掉的错误", "GPT-2缓存要占多少显存"
 *   [KV-4] jennyma11.github.io/infra/ch07-01.html "7.1 自回归生成过程"
 *          "Prefill 阶段", "Decode 阶段" (listing 1-2)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory.  Every tensor argument is a DEVICE pointer to contiguous,
 *    row-major memory owned by the caller (for example a torch tensor on
 *    the GPU), 16-byte aligned.  hist_len is a HOST pointer.  The library
 *    allocates no memory and keeps no pointer after a call returns.
 *  - Streams.  `stream` is a hipStream_t passed as void* (NULL = the legacy
 *    default stream).  All work is enqueued on it; no call synchronises the
 *    host with the device.
 *  - Cache.  One K and one V tensor per model, each [L, B, Hkv, Tmax, D]:
 *    layer l's slice is the pages' per-layer [batch, heads, sequence,
 *    head_dim] tensor, with the sequence axis preallocated to Tmax rows
 *    ([KV-1] "Decode Shape 示例"; [KV-2] "一个很容易漏掉的错误").
 *  - Step tensors.  Queries, new K/V rows and outputs of a call that covers
 *    layers [layer0, layer0 + n_layers) are [n_layers, B, H, N, D] with
 *    H = Hq for queries and outputs and H = Hkv for new K/V rows.  All of
 *    them share the cache's element type.
 *  - Element types.  KVC_F32 (IEEE binary32) or KVC_BF16 (bfloat16: the high
 *    16 bits of a binary32).  Arithmetic is fp32 in both cases; bf16 outputs
 *    are rounded to nearest-even.
 *  - Positions.  hist_len[b] = P_b is the number of tokens of sequence b
 *    already in the cache.  Calls read it and never change it; after a step
 *    the caller adds N.
 *  - Head dims.  D is 64 or 128.  Hq must be a multiple of Hkv; query head
 *    hq uses KV head hq / (Hq / Hkv) (contiguous groups: GQA / MQA, [KV-2]
 *    "GPT-2缓存要占多少显存"; Hq == Hkv is plain multi-head attention).
 *  - Errors.  Every argument is checked before anything is enqueued.  On a
 *    non-zero status nothing has been enqueued, no memory has been written,
 *    and kvc_last_error() describes the problem.  KVC_E_HIP reports a failed
 *    kernel launch; work enqueued before it by the same call may have run.
 *    No exception crosses the ABI and there is no CPU fallback.
 *  - Empty work.  N = 0, S = 0, B = 0 or n_layers = 0 are valid no-ops.
 *  - Concurrency.  Calls on different streams may run concurrently unless
 *    they write the same cache rows or share a decode workspace.
 */
#ifndef KVCACHE_H
#define KVCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 13

typedef enum {
  KVC_OK = 0,
  KVC_E_NULL = -1,        /* a required pointer is NULL */
  KVC_E_SHAPE = -2,       /* a size is negative, inconsistent or out of range */
  KVC_E_DTYPE = -3,       /* unknown element type */
  KVC_E_CAPACITY = -4,    /* hist_len[b] + N (or S) exceeds Tmax */
  KVC_E_WORKSPACE = -5,   /* decode workspace missing or too small */
  KVC_E_UNSUPPORTED = -6, /* a valid shape the library has no kernel for */
  KVC_E_HIP = -7          /* the HIP runtime refused a launch */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* A caller-owned cache: k and v are device pointers to [L,B,Hkv,Tmax,D]. */
typedef struct {
  void *k;
  void *v;
  int32_t L, B, Hkv, Tmax, D;
  int32_t dtype; /* kvc_dtype */
} kvc_cache;

/*
 * Bytes of one model's cache (K and V together):
 *   2 x L x Hkv x D x Tmax x B x element size.
 * [KV-2] "GPT-2缓存要占多少显存", the cache-size formula; for GPT-2 Small in
 * fp32 (L = 12, Hkv = 12, D = 64, B = 1) this is 73,728 bytes per token.
 * Returns 0 for negative sizes or an unknown dtype.
 */
uint64_t kvc_cache_bytes(int64_t L, int64_t B, int64_t Hkv, int64_t Tmax,
                         int64_t D, int32_t dtype);

/*
 * kv_append: for layers l in [layer0, layer0+n_layers), every b < B, every
 * KV head h and i < N, copy row k_new[l-layer0][b][h][i][:] to
 * cache.k[l][b][h][hist_len[b] + i][:], and the same for v.  Nothing else in
 * the cache changes; the copy is bit-exact.
 * [KV-1] "KV Cache 原理" (each round's new K/V join the cache) and
 * "Decode Shape 示例" (the join is along the sequence axis); [KV-4] "Decode
 * 阶段" (a real implementation writes into slots in place rather than
 * concatenating).
 *   k_new, v_new : device, [n_layers, B, Hkv, N, D], cache dtype
 *   hist_len     : host int32[B]; requires hist_len[b] + N <= Tmax
 *                  (KVC_E_CAPACITY otherwise, nothing written)
 */
kvc_status kvc_append(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                      const void *k_new, const void *v_new, int32_t N,
                      const int32_t *hist_len, void *stream);

/*
 * Workspace bytes kvc_attn_decode needs for this geometry: the partial
 * softmax states (max, sum and unnormalised output row) of the split-K
 * passes and, for one query row per KV head, one 8-byte arrival counter per
 * query row (the last split of a row to finish merges the row inside the
 * same launch).  It depends only on the cache geometry, n_layers, Hq and N,
 * never on the lengths, so one workspace serves every step.  Returns 0 on
 * invalid sizes.
 */
size_t kvc_decode_workspace_bytes(const kvc_cache *cache, int32_t n_layers,
                                  int32_t Hq, int32_t N);

/*
 * attn_decode: for layers l in [layer0, layer0+n_layers), sequences b, query
 * heads hq and new rows i < N, with P = hist_len[b], G = Hq / Hkv and
 * h = hq / G:
 *   s_j   = scale * <q[l][b][hq][i], K[l][b][h][j]>   for j = 0 .. P + i
 *   o[l][b][hq][i] = sum_j softmax(s)_j * V[l][b][h][j]
 * i.e. the causal mask is offset by the history length and new row i sees
 * P + i + 1 keys ([KV-2] "一个很容易漏掉的错误"; the score, softmax and
 * weighted sum are [KV-4] "Decode 阶段", listing 1-2, with scale = 1/sqrt(D)
 * there).  The K/V rows of the N new tokens must already be in the cache at
 * positions [P, P+N) (call kvc_append first with the same hist_len).
 *   q, o       : device, [n_layers, B, Hq, N, D], cache dtype
 *   scale      : finite score scale, normally 1/sqrt(D); any finite value
 *                is accepted (0 gives equal weights over the visible keys, a
 *                negative one the scores' negation).  Every decode and
 *                prefill entry point takes it the same way; an infinite or
 *                NaN scale is KVC_E_SHAPE.
 *   workspace  : device, >= kvc_decode_workspace_bytes(...) bytes, 256-byte
 *                aligned, caller-owned.  Zero-fill it once before its first
 *                use: with one query row per KV head its first bytes are
 *                arrival counters that must be zero when a call starts, and
 *                every call that returns KVC_OK leaves them zero again when
 *                its kernels end; the rest is scratch.  A call of another
 *                geometry (cache shape, n_layers, B, Hq or N) may use those
 *                bytes as scratch, so give each geometry its own workspace
 *                (or zero-fill it again when switching).  Calls enqueued one
 *                after another on a stream may share one.  Two calls in
 *                flight at the same time must not share a workspace.
 */
kvc_status kvc_attn_decode(const kvc_cache *cache, int32_t layer0,
                           int32_t n_layers, const void *q, int32_t Hq,
                           int32_t N, const int32_t *hist_len, float scale,
                           void *o, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * One whole decode step in one call: kvc_append of k_new / v_new at
 * positions [hist_len[b], hist_len[b] + N) followed by kvc_attn_decode with
 * the same hist_len, with identical results (cache bytes bit for bit,
 * outputs as kvc_attn_decode computes them).  The new rows are read once,
 * straight from k_new / v_new, and written into their slots by the decode
 * kernels themselves, so the step needs no separate append launch.  This is the
 * decode graph's "one token + cache in, output + updated cache out" ([KV-1]
 * "Prefill/Decode 双图"; [KV-2] "一个很容易漏掉的错误": append on the sequence
 * axis, then attend with the offset mask).
 *   q, o         : device, [n_layers, B, Hq, N, D]
 *   k_new, v_new : device, [n_layers, B, Hkv, N, D]
 *   other arguments, errors and workspace rules as kvc_attn_decode; on
 *   KVC_E_CAPACITY nothing is written.
 */
kvc_status kvc_decode_step(const kvc_cache *cache, int32_t layer0,
                           int32_t n_layers, const void *q, const void *k_new,
                           const void *v_new, int32_t Hq, int32_t N,
                           const int32_t *hist_len, float scale, void *o,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kvc_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split states and arrival counters
 * live in a 16 MiB scratch array inside the library, one per GPU, held from
 * library load until the process ends; the call itself allocates nothing.
 * Calls whose states need more than that scratch (the decode workspace of
 * kvc_decode_workspace_bytes beyond 16 MiB - 64 KiB of states, or more than
 * 8192 query rows) return KVC_E_WORKSPACE before enqueuing anything.  Every
 * call on a GPU shares its scratch: calls that may overlap on one GPU (other
 * streams, or graphs replayed concurrently) race and must not use this entry
 * point.  Arguments, results and other errors as kvc_decode_step.
 */
kvc_status kvc_decode_step_noalloc(const kvc_cache *cache, int32_t layer0,
                                   int32_t n_layers, const void *q,
                                   const void *k_new, const void *v_new,
                                   int32_t Hq, int32_t N,
                                   const int32_t *hist_len, float scale,
                                   void *o, void *stream);

/* kvc_decode_step with the sequence lengths in device memory, for a step that
 * is captured once in a HIP graph and replayed every token ([KV-4]
 * jennyma11.github.io/infra/ch07-01.html, "Decode 阶段": decode steps are
 * short, fixed-shape kernels whose launch cost graphs remove; [KV-2]
 * "实验到底测了什么" lists graphs beside paged attention in serving systems);
 * each replay sees the lengths as they are on the device then.
 *   hist_len_dev : device, int32 [B], 4-byte aligned; P_b = hist_len_dev[b]
 *                  is read by the kernels, never by the host.
 *   hist_max     : bound on every P_b; the launch is sized for it and the
 *                  kernels clamp P_b into [0, hist_max] (a wrong length gives
 *                  wrong results, never an access outside the cache).
 *                  KVC_E_CAPACITY if hist_max + N > Tmax, KVC_E_SHAPE if < 0.
 * Contiguous cache only; other arguments and errors as kvc_decode_step. */
kvc_status kvc_decode_step_dl(const kvc_cache *cache, int32_t layer0,
                              int32_t n_layers, const void *q,
                              const void *k_new, const void *v_new, int32_t Hq,
                              int32_t N, const int32_t *hist_len_dev,
                              int32_t hist_max, float scale, void *o,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* hist_len_dev[b] += n for b < B, enqueued on `stream`: the length update
 * that follows a captured kvc_decode_step_dl ([KV-4] "Decode 阶段": each step
 * grows every sequence by its new tokens).  B = 0 or n = 0 is a no-op;
 * KVC_E_NULL for a NULL array, KVC_E_SHAPE for B < 0 or misalignment. */
kvc_status kvc_lengths_add(int32_t *hist_len_dev, int32_t B, int32_t n,
                           void *stream);

/*
 * The two phases of kvc_attn_decode / kvc_decode_step as separate calls, for
 * callers that want to place other work between them (or time them apart).
 * Both take the arguments of kvc_decode_step; with k_new and v_new both NULL
 * they are the phases of kvc_attn_decode (rows [P, P+N) already appended),
 * with both given the phases of kvc_decode_step.  Call kvc_decode_combine
 * with the same arguments as kvc_decode_split, on the same stream, before
 * anything else uses the workspace; together they compute the one-call
 * form's result.  Calls whose (layer, sequence, KV head) units about fill
 * the GPU (from half a unit per compute unit to two) and that have at most
 * 8 query rows per KV head run the one-call form as one workgroup per unit
 * over its whole key range, which sums the same terms in another order, so
 * there the two forms agree to fp32 rounding rather than bit for bit.
 *
 * kvc_decode_split runs the split-K pass: each (layer, sequence, KV head,
 * split of the keys) computes the softmax state (max, sum, unnormalised
 * output) of its keys, into `workspace`, or straight into `o` for query rows
 * whose keys fit one split when nothing is left to merge.
 * kvc_decode_combine merges the states of every remaining query row and
 * writes its output: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with
 * M = max_s m_s (the rescaling that makes split softmax states additive; the
 * result is the same softmax-weighted sum [KV-4] "Decode 阶段" defines).
 * Which phase writes the new K/V rows into the cache in the k_new form is an
 * implementation detail: after both phases they are in their slots.
 * Arguments, errors and workspace rules as kvc_attn_decode / kvc_decode_step;
 * passing only one of k_new / v_new is KVC_E_NULL.
 */
kvc_status kvc_decode_split(const kvc_cache *cache, int32_t layer0,
                            int32_t n_layers, const void *q, const void *k_new,
                            const void *v_new, int32_t Hq, int32_t N,
                            const int32_t *hist_len, float scale, void *o,
                            void *workspace, size_t workspace_bytes,
                            void *stream);
kvc_status kvc_decode_combine(const kvc_cache *cache, int32_t layer0,
                              int32_t n_layers, const void *q,
                              const void *k_new, const void *v_new,
                              int32_t Hq, int32_t N, const int32_t *hist_len,
                              float scale, void *o, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * attn_prefill: causal self-attention over an S-token prompt that starts an
 * empty cache.  Writes k[..][i] and v[..][i] to cache rows [0, S) of every
 * sequence (as kvc_append with hist_len = 0 and N = S would) and computes,
 * for every prompt row i,
 *   o[l][b][hq][i] = sum_{j <= i} softmax_j(scale * <q_i, k_j>) * v_j
 * with the contiguous GQA grouping above.  Equal to kvc_append +
 * kvc_attn_decode with P = 0 and N = S, computed with matrix-core tiles.
 * [KV-1] "KV Cache 原理" (the first round runs the whole prompt and yields
 * each layer's K/V) and "Prefill/Decode 双图"; [KV-4] "Prefill 阶段" (all
 * prompt positions in parallel under a causal mask).
 *   q, o : device, [n_layers, B, Hq, S, D];  k, v : device, [n_layers, B,
 *   Hkv, S, D]; all in the cache dtype.  Requires S <= Tmax.  Prior cache
 *   contents at rows >= S are left unchanged.
 */
kvc_status kvc_attn_prefill(const kvc_cache *cache, int32_t layer0,
                            int32_t n_layers, const void *q, const void *k,
                            const void *v, int32_t Hq, int32_t S, float scale,
                            void *o, void *stream);

/*
 * attn_prefill_varlen: a batch of prompts packed along the token axis, each
 * with its own cached prefix, in one call.  [KV-4] "Prefill 阶段": the packed
 * batch ([total_tokens, hidden] with cu_seqlens marking where each sequence
 * starts) lets one launch cover the whole batch; long prompts are prefilled
 * in chunks, and a prompt whose prefix is already cached prefills only the
 * increment.  Sequence b brings S_b = cu_seqlens[b+1] - cu_seqlens[b] new
 * tokens on top of P_b = hist_len[b] cached positions: their K/V are written
 * to cache positions [P_b, P_b + S_b) and new token i attends to positions
 * 0 .. P_b + i ([KV-2] "一个很容易漏掉的错误": the causal mask offset by the
 * history).  Same result as kvc_append + kvc_attn_decode per sequence with
 * N = S_b.
 *   q, o       : device, [n_layers, T, Hq, D], token-major (token
 *                cu_seqlens[b] + i is new token i of sequence b), T =
 *                cu_seqlens[B]
 *   k, v       : device, [n_layers, T, Hkv, D]
 *   cu_seqlens : host int32 [B + 1], cu_seqlens[0] = 0, non-decreasing
 *                (S_b = 0 is allowed: that sequence is left alone)
 *   hist_len   : host int32 [B], P_b >= 0; P_b + S_b > Tmax is
 *                KVC_E_CAPACITY and nothing is written
 * Other rules as kvc_attn_prefill.  Computed on the matrix cores like it.
 */
kvc_status kvc_attn_prefill_varlen(const kvc_cache *cache, int32_t layer0,
                                   int32_t n_layers, const void *q,
                                   const void *k, const void *v, int32_t Hq,
                                   const int32_t *cu_seqlens,
                                   const int32_t *hist_len, float scale,
                                   void *o, void *stream);

/*
 * ---- paged cache ---------------------------------------------------------
 * The cache as pools of fixed-size blocks shared by all sequences, each
 * sequence owning a list of blocks (its block table).  [KV-2]
 * "显存测量最容易被分配器误导" (production engines manage the cache in pages or
 * blocks instead of concatenating) and [KV-4] "Decode 阶段" (the note after
 * listing 1-2: real implementations write each step's K/V in place, slot by
 * slot, with PagedAttention).  The pages give no layout; this one is:
 *   k, v        : device, [L, num_blocks, Hkv, block_size, D] each, the
 *                 cache dtype; a block holds block_size consecutive positions
 *                 of every KV head of one layer
 *   block_table : device int32 [B, max_blocks], caller-owned; position t of
 *                 sequence b lives in row t % block_size of block
 *                 block_table[b][t / block_size]
 * block_size is a power of two in [1, 1024]; D in {64, 128}.  Sequences may
 * share blocks (a common prefix); a call must not write a block that another
 * sequence still reads.  The library cannot check the table's contents
 * without a device sync: block ids outside [0, num_blocks) are clamped into
 * the pools (wrong results, never an access outside them).  Everything else
 * -- argument checks before any enqueue, hist_len on the host, no
 * allocation, caller workspace, stream -- is as for the contiguous cache,
 * with capacity max_blocks * block_size positions per sequence.
 */
typedef struct {
  void *k, *v;          /* device pools [L, num_blocks, Hkv, block_size, D] */
  int32_t L, num_blocks, Hkv, block_size, D;
  int32_t dtype;        /* kvc_dtype */
} kvc_paged_cache;

/* 2 x L x num_blocks x Hkv x block_size x D x element size; 0 on bad input. */
uint64_t kvc_paged_cache_bytes(int64_t L, int64_t num_blocks, int64_t Hkv,
                               int64_t block_size, int64_t D, int32_t dtype);

/* kvc_append into a paged cache: row i of k_new / v_new ([n_layers, B, Hkv,
 * N, D]) goes to position hist_len[b] + i, i.e. its slot in the block the
 * table names.  Positions past max_blocks * block_size: KVC_E_CAPACITY. */
kvc_status kvc_paged_append(const kvc_paged_cache *cache, int32_t layer0,
                            int32_t n_layers, const void *k_new,
                            const void *v_new, int32_t B, int32_t N,
                            const int32_t *hist_len,
                            const int32_t *block_table, int32_t max_blocks,
                            void *stream);

/* Workspace bytes for the paged decode calls with these arguments. */
size_t kvc_paged_decode_workspace_bytes(const kvc_paged_cache *cache,
                                        int32_t n_layers, int32_t B, int32_t Hq,
                                        int32_t N, int32_t max_blocks);

/* kvc_attn_decode over a paged cache: keys 0 .. hist_len[b] + i of sequence
 * b, read through its block table; q, o [n_layers, B, Hq, N, D]. */
kvc_status kvc_paged_attn_decode(const kvc_paged_cache *cache, int32_t layer0,
                                 int32_t n_layers, const void *q, int32_t Hq,
                                 int32_t B, int32_t N, const int32_t *hist_len,
                                 const int32_t *block_table, int32_t max_blocks,
                                 float scale, void *o, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* kvc_decode_step over a paged cache: kvc_paged_append followed by
 * kvc_paged_attn_decode, with the same results, in the same launches as
 * kvc_decode_step. */
kvc_status kvc_paged_decode_step(const kvc_paged_cache *cache, int32_t layer0,
                                 int32_t n_layers, const void *q,
                                 const void *k_new, const void *v_new,
                                 int32_t Hq, int32_t B, int32_t N,
                                 const int32_t *hist_len,
                                 const int32_t *block_table, int32_t max_blocks,
                                 float scale, void *o, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* kvc_paged_decode_step with the lengths in device memory: hist_len_dev and
 * hist_max as for kvc_decode_step_dl (capacity: hist_max + N within
 * max_blocks * block_size), so that a captured graph of the paged step stays
 * valid as the sequences grow; the block table is read on the device as
 * before, so its entries may change between replays too. */
kvc_status kvc_paged_decode_step_dl(const kvc_paged_cache *cache, int32_t layer0,
                                    int32_t n_layers, const void *q,
                                    const void *k_new, const void *v_new,
                                    int32_t Hq, int32_t B, int32_t N,
                                    const int32_t *hist_len_dev, int32_t hist_max,
                                    const int32_t *block_table, int32_t max_blocks,
                                    float scale, void *o, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* kvc_attn_prefill_varlen into a paged cache: cached positions below
 * hist_len[b] are read through sequence b's block table and the new tokens'
 * K/V are written to their slots.  B sequences (cu_seqlens [B + 1],
 * hist_len [B] on the host; block_table [B, max_blocks] on the device);
 * capacity max_blocks * block_size positions per sequence. */
kvc_status kvc_paged_attn_prefill_varlen(const kvc_paged_cache *cache,
                                         int32_t layer0, int32_t n_layers,
                                         const void *q, const void *k,
                                         const void *v, int32_t Hq, int32_t B,
                                         const int32_t *cu_seqlens,
                                         const int32_t *hist_len,
                                         const int32_t *block_table,
                                         int32_t max_blocks, float scale,
                                         void *o, void *stream);

/* ---- dense layer of a cached decode step ---------------------------------
 *
 * [KV-2] openai-hub.com/news/2435, "千倍计算量为何只换来6倍速度": with the cache,
 * a decode step computes the projections and the MLP of the new tokens only,
 * so each weight matrix is read once for a handful of rows.  This is that
 * step of the GPT-2 block the same page measures (pre-norm, GELU, residual):
 *
 *   y[m][n] = act( sum_k xh[m][k] wt[n][k] + bias[n] ) + res[m][n]
 *   xh[m] = (x[m] - mean) / sqrt(var + ln_eps) * ln_g + ln_b  when ln_g is
 *           given (mean and biased variance over the K features of row m),
 *           else x[m];  act = 0: identity, 1: GELU, tanh form
 *           0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
 *
 * All fp32, device pointers: x [M, K] row-major, or head-major [H, M, K/H]
 * with a_heads = H > 0 (the attention output as the decode call writes it;
 * K/H a multiple of 4; not with the layer norm); wt [N, K], the weight
 * transposed (output feature n's K input weights contiguous, packed once per
 * model, as kvc_gemm_f32 takes it); bias [N] or NULL; ln_g / ln_b [K] (both
 * or neither); res [M, N] or NULL; y [M, N], or with y_qkv_heads = H > 0 the
 * attention layout [3, H, M, N/(3H)] (q, k, v of the decode call; N/(3H) a
 * multiple of 4; no residual).  1 <= M <= 8, M * K <= 12288, K a multiple
 * of 4; x, wt, res and y 16-byte aligned.  y may be the same buffer as res
 * (in-place residual update) but must not overlap x.  The caller owns every
 * buffer; nothing is allocated.
 * Errors: KVC_E_NULL (x, wt or y missing, or only one of ln_g / ln_b),
 * KVC_E_SHAPE (sizes, layouts, alignment, act, ln_eps, overlaps),
 * KVC_E_UNSUPPORTED (more rows or inputs than that -- prompt-sized inputs go
 * to kvc_gemm_f32 -- or a layout with the norm / residual), KVC_E_HIP
 * (launch failure). */
kvc_status kvc_linear_f32(const float *x, int32_t a_heads, int32_t M, int32_t K,
                          const float *wt, int32_t N, const float *bias,
                          const float *ln_g, const float *ln_b, float ln_eps,
                          int32_t act, const float *res, float *y,
                          int32_t y_qkv_heads, void *stream);

/* ---- dense layers of a prompt ---------------------------------------------
 *
 * [KV-2] openai-hub.com/news/2435, "千倍计算量为何只换来6倍速度": without the
 * cache every step runs the projections and the MLP for every position of
 * the context again (products of the context length by the model width, on
 * the matrix cores here); with it only a prompt's first pass does.  The
 * GPT-2 block of that section: pre-norm, GELU, residual.
 *
 * gemm_f32: y[m][n] = act( sum_k a[m][k] wt[n][k] + bias[n] ) + res[m][n],
 * fp32 throughout (matrix-core fp32 products, no reduced precision),
 * act = 0: identity, 1: GELU, tanh form (as kvc_linear_f32).
 *   a  : device [M, K] row-major, or with a_heads = H > 0 head-major
 *        [H, M, K/H] (the attention output as the prefill writes it); K/H
 *        a multiple of 64.
 *   wt : device [N, K]: the weight transposed (output feature n's K input
 *        weights contiguous, a linear layer's usual layout), packed once
 *        per model.  bias [N] or NULL.  res [M, N] row-major or NULL; it
 *        may be y itself (in-place residual update).
 *   y  : device [M, N] row-major, or with y_qkv_heads = H > 0 the attention
 *        layout [3, H, M, N/(3H)] (q, k, v for kvc_attn_prefill /
 *        kvc_decode_step without a permute); N/(3H) a multiple of 4, and no
 *        res then.
 *   workspace : optional device scratch of at least
 *        kvc_gemm_workspace_bytes(M, K, N) bytes, 256-byte aligned,
 *        zero-filled once before its first use (every call leaves its
 *        counters zero again); calls sharing one must not overlap.  With it,
 *        a product whose 64 x 64 output tiles are too few to fill the chip
 *        splits K over several workgroups per tile, the last of which sums
 *        the partial tiles in a fixed order (the result does not depend on
 *        timing).  NULL (or a size of 0 from the query): no split.
 *   K a positive multiple of 64, N >= 1, M >= 0 (0: no-op); a, wt, res, y
 *   16-byte aligned, y not overlapping a.  Errors: KVC_E_NULL, KVC_E_SHAPE
 *   (sizes, layouts, alignment, overlap), KVC_E_UNSUPPORTED (too large for
 *   one launch, a residual with the attention layout), KVC_E_WORKSPACE (a
 *   workspace smaller than the query's answer), KVC_E_HIP. */
kvc_status kvc_gemm_f32(const float *a, int32_t a_heads, int32_t M, int32_t K,
                        const float *wt, int32_t N, const float *bias,
                        int32_t act, const float *res, float *y,
                        int32_t y_qkv_heads, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Workspace bytes kvc_gemm_f32 uses for an M x K x N product on the current
 * device (0: it would not split K; also 0 for invalid sizes). */
size_t kvc_gemm_workspace_bytes(int32_t M, int32_t K, int32_t N);

/* layernorm_f32: y[m] = (x[m] - mean) / sqrt(var + eps) * g + b over the K
 * features of each row (biased variance), the GPT-2 block's pre-norm.
 * x, y device [M, K] (y may be x), g, b [K]; K a multiple of 4 up to 4096;
 * all 16-byte aligned; eps finite and >= 0.  Errors as kvc_gemm_f32. */
kvc_status kvc_layernorm_f32(const float *x, int32_t M, int32_t K,
                             const float *g, const float *b, float eps,
                             float *y, void *stream);

/* Input layer of the GPT-2 block ([KV-2] openai-hub.com/news/2435, "实验到底测了
 * 什么": GPT-2 Small, learned token and position embeddings): row i of y is
 * the embedding of token ids[i] plus that of its position p0 + i,
 *
 *   y[i][k] = wte[ids[i]][k] + wpe[p0 + i][k],   i < N, k < d,
 *
 * with p0 = pos[0] when pos (a device int32) is given -- a length that
 * advances on the device, as kvc_lengths_add keeps it -- else pos0.  All
 * device pointers: wte [V, d] and wpe [T, d] fp32 row-major, ids int64 [N],
 * y [N, d]; d a multiple of 4, wte / wpe / y 16-byte aligned, y overlapping
 * neither table.  The ids and a device position are read by the kernel, so
 * they are not checked here: a row whose id lies outside [0, V) or whose
 * position lies outside [0, T) is written as NaN.  Errors: KVC_E_NULL,
 * KVC_E_SHAPE (sizes, alignment, overlap, pos0 + N > T without pos),
 * KVC_E_HIP.  N = 0 is a no-op. */
kvc_status kvc_embed_f32(const float *wte, int32_t V, const float *wpe, int32_t T,
                         int32_t d, const int64_t *ids, int32_t N, int32_t pos0,
                         const int32_t *pos, float *y, void *stream);

/* Greedy choice of the next token ([KV-2] openai-hub.com/news/2435, "实验到底测
 * 了什么": greedy decoding, batch 1): index[0] = the first i in [0, n) at
 * which x[i] is largest, a NaN counting as larger than every number (so the
 * first NaN wins).  With seq given, the same launch then advances the device
 * counter *seq_pos by one and, if its new value p lies in [0, seq_capacity),
 * stores the index at seq[p]: the token history of a graph-captured
 * generation loop, which then needs no other kernel per token.  All device
 * pointers: x fp32 [n], 16-byte aligned; index int64 [1]; seq int64
 * [seq_capacity] and seq_pos int64 [1], both given or both NULL.  Errors:
 * KVC_E_NULL (x, index, or one of seq / seq_pos without the other),
 * KVC_E_SHAPE (n < 1 or n >= 2^31, x misaligned, seq_capacity < 1 with seq),
 * KVC_E_HIP. */
kvc_status kvc_argmax_f32(const float *x, int64_t n, int64_t *index, int64_t *seq,
                          int64_t *seq_pos, int64_t seq_capacity, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *kvc_last_error(void);

/* KVC_ABI_VERSION of the loaded library. */
int32_t kvc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVCACHE_H */
