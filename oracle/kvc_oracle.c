/*
 * kvc_oracle.c -- plain CPU oracle for attention over a per-layer KV cache.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load this library.  It shares no
 * source, header, table or build flag with the HIP library; the two meet only
 * at the byte level, on inputs made by the seeded generators.
 *
 * Everything here is the plain definition written out: loops in the obvious
 * order, every product and sum in double precision, no blocking, no fusion,
 * no reordering beyond what the definition states.  Keys are visited in
 * ascending position, so two calls that see the same keys give bit-identical
 * results.
 *
 * Pages followed (cited by address and section title):
 *   [KV-1] gitcode.csdn.net/69e62cef0a2f6a37c5a11c4f.html  (miniONNXRuntime GPT-2)
 *          sections "KV Cache 原理", "Decode Shape 示例"
 *   [KV-2] openai-hub.com/news/2435 "GPT-2缓存实测：千倍计算只快6倍"
 *          sections "一个很容易漏掉的错误", "GPT-2缓存要占多少显存"
 *   [KV-4] jennyma11.github.io/infra/ch07-01.html "7.1 自回归生成过程"
 *          section "Decode 阶段", code listing 1-2
 *
 * Layout (the pages' [batch, heads, sequence, head_dim] per layer, stacked
 * over layers): cache K and V are each [L, B, Hkv, Tmax, D], row-major,
 * contiguous.  New rows and queries are [n_layers, B, H, N, D].
 *
 * Element types: 0 = IEEE fp32, 1 = bfloat16 (the high 16 bits of an fp32).
 * Inputs are decoded exactly into double; results are returned in double and
 * any rounding to an output type is left to the caller.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_E_ARG (-1)
#define ORACLE_E_CAPACITY (-4)

static size_t elem_size(int dtype) { return dtype == 1 ? 2u : 4u; }

/* Exact decode of one stored element into double. */
static double load_elem(const void *base, size_t index, int dtype) {
  if (dtype == 1) {
    uint16_t hi;
    memcpy(&hi, (const char *)base + index * 2u, 2u);
    uint32_t bits = (uint32_t)hi << 16;
    float f;
    memcpy(&f, &bits, 4u);
    return (double)f;
  }
  float f;
  memcpy(&f, (const char *)base + index * 4u, 4u);
  return (double)f;
}

/* Flat element index of cache[l][b][h][t][0]. */
static size_t cache_row(int l, int b, int h, int t, int B, int Hkv, int Tmax,
                        int D) {
  return ((((size_t)l * B + b) * Hkv + h) * (size_t)Tmax + (size_t)t) *
         (size_t)D;
}

/* Flat element index of x[l][b][h][i][0] for an [n_layers, B, H, N, D] array. */
static size_t step_row(int l, int b, int h, int i, int B, int H, int N,
                       int D) {
  return ((((size_t)l * B + b) * H + h) * (size_t)N + (size_t)i) * (size_t)D;
}

/*
 * Bytes held by one model's cache: 2 (K and V) x layers x KV heads x head dim
 * x tokens x batch x bytes per element.  [KV-2] "GPT-2缓存要占多少显存", the
 * cache-size formula.
 */
uint64_t oracle_cache_bytes(int64_t layers, int64_t batch, int64_t kv_heads,
                            int64_t tokens, int64_t head_dim,
                            int64_t elem_bytes) {
  return (uint64_t)(2 * layers * kv_heads * head_dim * tokens * batch *
                    elem_bytes);
}

/*
 * Write the N new K/V rows of layers [layer0, layer0+n_layers) at sequence
 * positions [P_b, P_b+N) of each batch entry b, where P_b = hist_len[b].
 * Nothing else in the cache changes.  The rows are copied byte for byte.
 *
 * [KV-1] "KV Cache 原理" (new K/V are appended to the cache for the next
 * round) and "Decode Shape 示例" (the append is along the sequence axis,
 * [1,H,T,D] + [1,H,1,D] -> [1,H,T+1,D]); [KV-2] "一个很容易漏掉的错误"
 * (prefill fills the cache, each decode step concatenates the new rows on the
 * sequence dimension before attention).  A preallocated cache replaces the
 * concatenation by a write into slots P_b..P_b+N-1, which leaves the same
 * bytes at the same positions.
 *
 * Returns ORACLE_E_CAPACITY and writes nothing if any P_b + N > Tmax.
 */
int oracle_append(void *k_cache, void *v_cache, int L, int B, int Hkv,
                  int Tmax, int D, int dtype, int layer0, int n_layers,
                  const void *k_new, const void *v_new, int N,
                  const int32_t *hist_len) {
  if (L < 0 || B < 0 || Hkv < 0 || Tmax < 0 || D < 0 || N < 0 ||
      layer0 < 0 || n_layers < 0 || layer0 + n_layers > L)
    return ORACLE_E_ARG;
  for (int b = 0; b < B; ++b) {
    if (hist_len[b] < 0) return ORACLE_E_ARG;
    if ((int64_t)hist_len[b] + N > Tmax) return ORACLE_E_CAPACITY;
  }
  const size_t es = elem_size(dtype);
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hkv; ++h)
        for (int i = 0; i < N; ++i) {
          size_t dst = cache_row(layer0 + l, b, h, hist_len[b] + i, B, Hkv,
                                 Tmax, D);
          size_t src = step_row(l, b, h, i, B, Hkv, N, D);
          memcpy((char *)k_cache + dst * es, (const char *)k_new + src * es,
                 (size_t)D * es);
          memcpy((char *)v_cache + dst * es, (const char *)v_new + src * es,
                 (size_t)D * es);
        }
  return ORACLE_OK;
}

/*
 * Attention of N new query rows against the cache, after their K/V rows have
 * been appended.  For layer l, batch b, query head hq and new row i:
 *
 *   n      = P_b + i + 1            visible keys, positions 0 .. P_b+i
 *   hkv    = floor(hq / (Hq/Hkv))   KV head shared by a contiguous group
 *   s_j    = scale * sum_d q[d] * K[hkv][j][d]            (j < n)
 *   m      = max_j s_j
 *   w_j    = exp(s_j - m)
 *   out[d] = (sum_j w_j * V[hkv][j][d]) / (sum_j w_j)
 *
 * [KV-4] "Decode 阶段", listing 1-2: scores are q times the transposed key
 * cache divided by sqrt(D), then softmax, then times the value cache.
 * [KV-2] "一个很容易漏掉的错误": with P cached tokens and N new ones, new row
 * i may attend to P+i+1 keys (causal mask offset by the history length).
 * [KV-2] "GPT-2缓存要占多少显存" and listing 1-2's H_q / H_kv: several query
 * heads share fewer KV heads.  The pages do not fix which ones; the reading
 * taken is contiguous groups (query heads g*G .. g*G+G-1 share KV head g,
 * G = Hq/Hkv).  Subtracting m leaves the softmax unchanged and keeps exp finite.
 *
 * q is [n_layers, B, Hq, N, D] in `dtype`; out is [n_layers, B, Hq, N, D]
 * double.  Returns ORACLE_E_ARG on bad shapes, ORACLE_E_CAPACITY if any
 * P_b + N > Tmax; out is then untouched.
 */
/*
 * One query row against the n visible keys 0 .. n-1 of cache head
 * (layer, b, hkv): the definition above, written once and used by every
 * attention function here.  q_row and out_row point at the row's D
 * elements; s and acc are scratch of n and D doubles.
 */
static void attend_row(const void *q, size_t q_row, const void *k_cache,
                       const void *v_cache, int layer, int b, int hkv, int B,
                       int Hkv, int Tmax, int D, int dtype, int n,
                       double scale, double *s, double *acc, double *out_row) {
  for (int j = 0; j < n; ++j) {
    const size_t krow = cache_row(layer, b, hkv, j, B, Hkv, Tmax, D);
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += load_elem(q, q_row + d, dtype) * load_elem(k_cache, krow + d, dtype);
    s[j] = scale * dot;
  }
  double m = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (s[j] > m) m = s[j];
  double denom = 0.0;
  for (int d = 0; d < D; ++d) acc[d] = 0.0;
  for (int j = 0; j < n; ++j) {
    const double w = exp(s[j] - m);
    const size_t vrow = cache_row(layer, b, hkv, j, B, Hkv, Tmax, D);
    denom += w;
    for (int d = 0; d < D; ++d) acc[d] += w * load_elem(v_cache, vrow + d, dtype);
  }
  for (int d = 0; d < D; ++d) out_row[d] = acc[d] / denom;
}

int oracle_attention(const void *q, const void *k_cache, const void *v_cache,
                     int L, int B, int Hkv, int Tmax, int D, int dtype,
                     int layer0, int n_layers, int Hq, int N,
                     const int32_t *hist_len, double scale, double *out) {
  if (L < 0 || B < 0 || Hkv <= 0 || Tmax < 0 || D <= 0 || N < 0 ||
      Hq <= 0 || Hq % Hkv != 0 || layer0 < 0 || n_layers < 0 ||
      layer0 + n_layers > L)
    return ORACLE_E_ARG;
  for (int b = 0; b < B; ++b) {
    if (hist_len[b] < 0) return ORACLE_E_ARG;
    if ((int64_t)hist_len[b] + N > Tmax) return ORACLE_E_CAPACITY;
  }
  const int group = Hq / Hkv;
  const long units = (long)n_layers * B * Hq;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (long u = 0; u < units; ++u) {
    const int hq = (int)(u % Hq);
    const int b = (int)((u / Hq) % B);
    const int l = (int)(u / ((long)Hq * B));
    const int hkv = hq / group;
    double *s = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
      free(s);
      free(acc);
      failed = 1;
      continue;
    }
    for (int i = 0; i < N; ++i) {
      const int n = hist_len[b] + i + 1;
      const size_t qrow = step_row(l, b, hq, i, B, Hq, N, D);
      attend_row(q, qrow, k_cache, v_cache, layer0 + l, b, hkv, B, Hkv, Tmax, D,
                 dtype, n, scale, s, acc, out + qrow);
    }
    free(s);
    free(acc);
  }
  return failed ? ORACLE_E_ARG : ORACLE_OK;
}

/*
 * Prefill of a whole prompt of S tokens into an empty cache: the prompt's K/V
 * rows go to positions [0, S) and every prompt row attends causally to
 * itself and the rows before it.  This is exactly append with P_b = 0 and
 * N = S followed by attention with the same P_b and N.
 * [KV-1] "KV Cache 原理" (the first round runs the whole prompt and yields
 * each layer's K/V); [KV-4] "Prefill 阶段" (all prompt positions in parallel
 * under a causal mask, K/V written into the cache).
 */
int oracle_prefill(void *k_cache, void *v_cache, int L, int B, int Hkv,
                   int Tmax, int D, int dtype, int layer0, int n_layers,
                   const void *q, const void *k, const void *v, int Hq, int S,
                   double scale, double *out) {
  if (B < 0) return ORACLE_E_ARG;
  int32_t *zeros = (int32_t *)calloc((size_t)(B > 0 ? B : 1), sizeof(int32_t));
  if (!zeros) return ORACLE_E_ARG;
  int rc = oracle_append(k_cache, v_cache, L, B, Hkv, Tmax, D, dtype, layer0,
                         n_layers, k, v, S, zeros);
  if (rc == ORACLE_OK)
    rc = oracle_attention(q, k_cache, v_cache, L, B, Hkv, Tmax, D, dtype,
                          layer0, n_layers, Hq, S, zeros, scale, out);
  free(zeros);
  return rc;
}

/*
 * Packed variable-length prefill with history.  [KV-4] "Prefill 阶段": a
 * batch of prompts is packed along the token axis ([total_tokens, hidden],
 * cu_seqlens marking where each sequence starts) so one launch covers the
 * whole batch; a long prompt is prefilled in chunks, and a prompt whose
 * prefix is already cached only prefills the increment.  So sequence b
 * brings S_b = cu_seqlens[b+1] - cu_seqlens[b] new tokens on top of P_b =
 * hist_len[b] cached ones: they are appended at positions [P_b, P_b + S_b)
 * and new token i attends to positions 0 .. P_b + i ([KV-2]
 * "一个很容易漏掉的错误": the causal mask offset by the history length).
 * That is exactly append then attention as above, one sequence at a time.
 *
 * Packed tensors are token-major per layer, as the page's packed batch:
 * q and out [n_layers, T, Hq, D], k and v [n_layers, T, Hkv, D], T =
 * cu_seqlens[B]; token cu_seqlens[b] + i is new token i of sequence b.
 * Returns ORACLE_E_CAPACITY if any P_b + S_b > Tmax, ORACLE_E_ARG on bad
 * shapes (cu_seqlens not non-decreasing from 0); nothing is written then.
 */
int oracle_prefill_varlen(void *k_cache, void *v_cache, int L, int B, int Hkv,
                          int Tmax, int D, int dtype, int layer0,
                          int n_layers, const void *q, const void *k,
                          const void *v, int Hq, const int32_t *cu_seqlens,
                          const int32_t *hist_len, double scale, double *out) {
  if (L < 0 || B < 0 || Hkv <= 0 || Tmax < 0 || D <= 0 || Hq <= 0 ||
      Hq % Hkv != 0 || layer0 < 0 || n_layers < 0 || layer0 + n_layers > L ||
      cu_seqlens[0] != 0)
    return ORACLE_E_ARG;
  for (int b = 0; b < B; ++b) {
    if (hist_len[b] < 0 || cu_seqlens[b + 1] < cu_seqlens[b]) return ORACLE_E_ARG;
    if ((int64_t)hist_len[b] + (cu_seqlens[b + 1] - cu_seqlens[b]) > Tmax)
      return ORACLE_E_CAPACITY;
  }
  const int T = cu_seqlens[B];
  const size_t es = elem_size(dtype);
  /* append: token cu[b] + i of head h to cache position P_b + i */
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hkv; ++h)
        for (int i = 0; i < cu_seqlens[b + 1] - cu_seqlens[b]; ++i) {
          const int pos = hist_len[b] + i;
          const size_t src = (((size_t)l * T + cu_seqlens[b] + i) * Hkv + h) * (size_t)D;
          const size_t dst = cache_row(layer0 + l, b, h, pos, B, Hkv, Tmax, D);
          memcpy((char *)k_cache + dst * es, (const char *)k + src * es, (size_t)D * es);
          memcpy((char *)v_cache + dst * es, (const char *)v + src * es, (size_t)D * es);
        }
  /* attention: new token i of sequence b sees P_b + i + 1 keys */
  const int group = Hq / Hkv;
  const long units = (long)n_layers * B * Hq;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (long u = 0; u < units; ++u) {
    const int hq = (int)(u % Hq);
    const int b = (int)((u / Hq) % B);
    const int l = (int)(u / ((long)Hq * B));
    double *s = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
      free(s);
      free(acc);
      failed = 1;
      continue;
    }
    for (int i = 0; i < cu_seqlens[b + 1] - cu_seqlens[b]; ++i) {
      const size_t qrow = (((size_t)l * T + cu_seqlens[b] + i) * Hq + hq) * (size_t)D;
      attend_row(q, qrow, k_cache, v_cache, layer0 + l, b, hq / group, B, Hkv,
                 Tmax, D, dtype, hist_len[b] + i + 1, scale, s, acc, out + qrow);
    }
    free(s);
    free(acc);
  }
  return failed ? ORACLE_E_ARG : ORACLE_OK;
}

/*
 * Paged cache.  [KV-2] "显存测量最容易被分配器误导" (production engines
 * preallocate and manage the cache in pages or blocks instead of
 * concatenating) and [KV-4] "Decode 阶段" (the note after listing 1-2: real
 * implementations write each step's K/V in place, slot by slot, with
 * PagedAttention).  The pages give no layout; the reading taken is the usual
 * one for such a cache:
 *   * K and V are each a pool [L, num_blocks, Hkv, block_size, D]: a block
 *     holds block_size consecutive positions of every KV head of one layer;
 *   * block_table[b][j] (int32 [B, max_blocks]) names the block that holds
 *     positions j*block_size .. j*block_size + block_size - 1 of sequence b;
 *   * position t of sequence b is row t % block_size of block
 *     block_table[b][t / block_size].
 * Attention over a paged cache is the attention above over the sequence's
 * rows in position order; which physical block holds them changes nothing.
 */

/* Flat element index of pool[l][blk][h][r][0]. */
static size_t paged_row(int l, int blk, int h, int r, int num_blocks, int Hkv,
                        int block_size, int D) {
  return ((((size_t)l * num_blocks + blk) * Hkv + h) * (size_t)block_size +
          (size_t)r) *
         (size_t)D;
}

/* Checks shared by the paged functions: positions [0, hist_len[b] + N) must
 * fit the table row, and every block id they use must name a block. */
static int paged_check(int L, int num_blocks, int Hkv, int block_size, int D,
                       int layer0, int n_layers, int B, int N,
                       const int32_t *hist_len, const int32_t *block_table,
                       int max_blocks, const int32_t *cu_seqlens) {
  if (L < 0 || num_blocks < 0 || Hkv <= 0 || block_size <= 0 || D <= 0 ||
      B < 0 || N < 0 || max_blocks < 0 || layer0 < 0 || n_layers < 0 ||
      layer0 + n_layers > L)
    return ORACLE_E_ARG;
  for (int b = 0; b < B; ++b) {
    if (hist_len[b] < 0) return ORACLE_E_ARG;
    /* N new rows each, or sequence b's share of a packed batch */
    const int n_new = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : N;
    if (n_new < 0) return ORACLE_E_ARG;
    const int64_t end = (int64_t)hist_len[b] + n_new;
    if (end > (int64_t)max_blocks * block_size) return ORACLE_E_CAPACITY;
    for (int64_t j = 0; j * block_size < end; ++j) {
      const int32_t blk = block_table[(size_t)b * max_blocks + j];
      if (blk < 0 || blk >= num_blocks) return ORACLE_E_ARG;
    }
  }
  return ORACLE_OK;
}

/*
 * Write the N new K/V rows of layers [layer0, layer0+n_layers) at positions
 * [P_b, P_b+N) of each sequence b, each into its slot: row (P_b+i) %
 * block_size of block block_table[b][(P_b+i) / block_size].  Nothing else in
 * the pools changes; rows are copied byte for byte.  Returns
 * ORACLE_E_CAPACITY (P_b + N beyond the table row) or ORACLE_E_ARG (a block
 * id out of range) and writes nothing.
 */
int oracle_paged_append(void *k_pool, void *v_pool, int L, int num_blocks,
                        int Hkv, int block_size, int D, int dtype, int layer0,
                        int n_layers, const void *k_new, const void *v_new,
                        int B, int N, const int32_t *hist_len,
                        const int32_t *block_table, int max_blocks) {
  int rc = paged_check(L, num_blocks, Hkv, block_size, D, layer0, n_layers, B,
                       N, hist_len, block_table, max_blocks, NULL);
  if (rc != ORACLE_OK) return rc;
  const size_t es = elem_size(dtype);
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hkv; ++h)
        for (int i = 0; i < N; ++i) {
          const int t = hist_len[b] + i;
          const int blk = block_table[(size_t)b * max_blocks + t / block_size];
          const size_t dst = paged_row(layer0 + l, blk, h, t % block_size,
                                       num_blocks, Hkv, block_size, D);
          const size_t src = step_row(l, b, h, i, B, Hkv, N, D);
          memcpy((char *)k_pool + dst * es, (const char *)k_new + src * es,
                 (size_t)D * es);
          memcpy((char *)v_pool + dst * es, (const char *)v_new + src * es,
                 (size_t)D * es);
        }
  return ORACLE_OK;
}

/*
 * Attention over a paged cache: gather each sequence's rows 0 ..
 * hist_len[b]+N-1 in position order into a contiguous [n_layers, B, Hkv,
 * Tlog, D] copy (Tlog = max_blocks * block_size), then oracle_attention on
 * it -- the same definition, keys visited in the same order.
 */
int oracle_paged_attention(const void *q, const void *k_pool,
                           const void *v_pool, int L, int num_blocks, int Hkv,
                           int block_size, int D, int dtype, int layer0,
                           int n_layers, int Hq, int B, int N,
                           const int32_t *hist_len, const int32_t *block_table,
                           int max_blocks, double scale, double *out) {
  int rc = paged_check(L, num_blocks, Hkv, block_size, D, layer0, n_layers, B,
                       N, hist_len, block_table, max_blocks, NULL);
  if (rc != ORACLE_OK) return rc;
  if (Hq <= 0 || Hq % Hkv != 0) return ORACLE_E_ARG;
  const int Tlog = max_blocks * block_size;
  const size_t es = elem_size(dtype);
  const size_t n = (size_t)n_layers * B * Hkv * (size_t)Tlog * D;
  char *kc = (char *)calloc(n > 0 ? n : 1, es);
  char *vc = (char *)calloc(n > 0 ? n : 1, es);
  if (!kc || !vc) {
    free(kc);
    free(vc);
    return ORACLE_E_ARG;
  }
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hkv; ++h)
        for (int pos = 0; pos < hist_len[b] + N; ++pos) {
          const int blk = block_table[(size_t)b * max_blocks + pos / block_size];
          const size_t src = paged_row(layer0 + l, blk, h, pos % block_size,
                                       num_blocks, Hkv, block_size, D);
          const size_t dst = cache_row(l, b, h, pos, B, Hkv, Tlog, D);
          memcpy(kc + dst * es, (const char *)k_pool + src * es, (size_t)D * es);
          memcpy(vc + dst * es, (const char *)v_pool + src * es, (size_t)D * es);
        }
  rc = oracle_attention(q, kc, vc, n_layers, B, Hkv, Tlog, D, dtype, 0,
                        n_layers, Hq, N, hist_len, scale, out);
  free(kc);
  free(vc);
  return rc;
}

/*
 * Packed variable-length prefill into a paged cache: gather each sequence's
 * cached positions [0, P_b) in order into a contiguous copy, run
 * oracle_prefill_varlen on it, and write the new rows, positions [P_b, P_b +
 * S_b), back to their slots.  Same definition; only where rows live differs.
 */
int oracle_paged_prefill_varlen(void *k_pool, void *v_pool, int L,
                                int num_blocks, int Hkv, int block_size, int D,
                                int dtype, int layer0, int n_layers,
                                const void *q, const void *k, const void *v,
                                int Hq, int B, const int32_t *cu_seqlens,
                                const int32_t *hist_len,
                                const int32_t *block_table, int max_blocks,
                                double scale, double *out) {
  if (B < 0 || cu_seqlens[0] != 0) return ORACLE_E_ARG;
  int rc = paged_check(L, num_blocks, Hkv, block_size, D, layer0, n_layers, B,
                       0, hist_len, block_table, max_blocks, cu_seqlens);
  if (rc != ORACLE_OK) return rc;
  const int Tlog = max_blocks * block_size;
  const size_t es = elem_size(dtype);
  const size_t n = (size_t)n_layers * B * Hkv * (size_t)Tlog * D;
  char *kc = (char *)calloc(n > 0 ? n : 1, es);
  char *vc = (char *)calloc(n > 0 ? n : 1, es);
  if (!kc || !vc) {
    free(kc);
    free(vc);
    return ORACLE_E_ARG;
  }
  for (int l = 0; l < n_layers; ++l)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hkv; ++h)
        for (int cpos = 0; cpos < hist_len[b]; ++cpos) {
          const int blk = block_table[(size_t)b * max_blocks + cpos / block_size];
          const size_t src = paged_row(layer0 + l, blk, h, cpos % block_size,
                                       num_blocks, Hkv, block_size, D);
          const size_t dst = cache_row(l, b, h, cpos, B, Hkv, Tlog, D);
          memcpy(kc + dst * es, (const char *)k_pool + src * es, (size_t)D * es);
          memcpy(vc + dst * es, (const char *)v_pool + src * es, (size_t)D * es);
        }
  rc = oracle_prefill_varlen(kc, vc, n_layers, B, Hkv, Tlog, D, dtype, 0,
                             n_layers, q, k, v, Hq, cu_seqlens, hist_len,
                             scale, out);
  if (rc == ORACLE_OK)
    for (int l = 0; l < n_layers; ++l)
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
          for (int npos = hist_len[b]; npos < hist_len[b] + cu_seqlens[b + 1] - cu_seqlens[b]; ++npos) {
            const int blk = block_table[(size_t)b * max_blocks + npos / block_size];
            const size_t dst = paged_row(layer0 + l, blk, h, npos % block_size,
                                         num_blocks, Hkv, block_size, D);
            const size_t src = cache_row(l, b, h, npos, B, Hkv, Tlog, D);
            memcpy((char *)k_pool + dst * es, kc + src * es, (size_t)D * es);
            memcpy((char *)v_pool + dst * es, vc + src * es, (size_t)D * es);
          }
  free(kc);
  free(vc);
  return rc;
}

/* Thread control for the timed CPU baseline (independent (l, b, hq) units). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
