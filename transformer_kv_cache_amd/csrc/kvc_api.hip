// kvc_api.hip -- the C ABI of libkvcache.so (declared in include/kvcache.h):
// argument validation, launch geometry and the kernel launches.  Every check
// runs before the first enqueue, so a rejected call leaves device memory
// untouched and never touches the HIP runtime.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kvc_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kvc_status fail(kvc_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

kvc_status ok() {
  g_last_error[0] = '\0';
  return KVC_OK;
}

int elem_bytes(int32_t dtype) { return dtype == KVC_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by every entry point: the cache descriptor and layer range.
kvc_status check_cache(const kvc_cache *c, int32_t layer0, int32_t n_layers, const char *fn) {
  if (!c) return fail(KVC_E_NULL, "%s: cache descriptor is NULL", fn);
  if (c->dtype != KVC_F32 && c->dtype != KVC_BF16)
    return fail(KVC_E_DTYPE, "%s: unknown dtype %d", fn, (int)c->dtype);
  if (c->L < 0 || c->B < 0 || c->Hkv <= 0 || c->Tmax < 0 || c->D <= 0)
    return fail(KVC_E_SHAPE, "%s: bad cache geometry L=%d B=%d Hkv=%d Tmax=%d D=%d", fn, c->L, c->B,
                c->Hkv, c->Tmax, c->D);
  if (c->D != 64 && c->D != 128)
    return fail(KVC_E_UNSUPPORTED, "%s: head dim D=%d (supported: 64, 128)", fn, c->D);
  if (layer0 < 0 || n_layers < 0 || (int64_t)layer0 + n_layers > c->L)
    return fail(KVC_E_SHAPE, "%s: layers [%d, %d+%d) outside [0, %d)", fn, layer0, layer0, n_layers,
                c->L);
  // the decode kernels address a head's rows with 32-bit byte offsets
  if ((int64_t)c->Tmax * c->D * elem_bytes(c->dtype) >= (int64_t)1 << 32)
    return fail(KVC_E_UNSUPPORTED, "%s: Tmax = %d rows of %d bytes exceed 4 GiB per head", fn, c->Tmax,
                c->D * elem_bytes(c->dtype));
  return KVC_OK;
}

kvc_status check_cache_pointers(const kvc_cache *c, const char *fn) {
  if (!c->k || !c->v) return fail(KVC_E_NULL, "%s: cache k or v pointer is NULL", fn);
  if (!aligned16(c->k) || !aligned16(c->v))
    return fail(KVC_E_SHAPE, "%s: cache pointers must be 16-byte aligned", fn);
  return KVC_OK;
}

kvc_status check_hist(const kvc_cache *c, const int32_t *hist_len, int32_t N, const char *fn) {
  if (c->B > 0 && !hist_len) return fail(KVC_E_NULL, "%s: hist_len is NULL", fn);
  for (int b = 0; b < c->B; ++b) {
    if (hist_len[b] < 0) return fail(KVC_E_SHAPE, "%s: hist_len[%d] = %d < 0", fn, b, hist_len[b]);
    if ((int64_t)hist_len[b] + N > c->Tmax)
      return fail(KVC_E_CAPACITY, "%s: hist_len[%d] + N = %d + %d exceeds Tmax = %d", fn, b,
                  hist_len[b], N, c->Tmax);
  }
  return KVC_OK;
}

kvc_status hip_status(hipError_t e, const char *fn) {
  if (e != hipSuccess) return fail(KVC_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// Split kernel of a decode call: one query row per KV head (vector kernel),
// a few rows with 256-byte key rows (multi-row vector kernel), else the
// matrix-core kernel in tiles of 16 rows.
enum class DecodeKernel { kVector, kRows, kMfma };

struct DecodeGeometry {
  DecodeKernel kernel;
  bool mfma;  // several query rows per KV head (rows or matrix-core kernel)
  int rows, row_tile, row_tiles;
  int split_keys;  // keys per split (single-row kernel: its smallest split)
  int max_splits;  // workspace stride in splits (for the smallest split)
  size_t ws_o_bytes, ws_ml_bytes, ctr_bytes, total;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

DecodeGeometry decode_geometry(const kvc_cache *c, int32_t n_layers, int32_t Hq, int32_t N) {
  DecodeGeometry g{};
  const int G = Hq / c->Hkv;
  g.rows = G * N;
  g.mfma = g.rows > 1;
  g.kernel = !g.mfma ? DecodeKernel::kVector
             : kvc::decode_rows_fits(c->dtype, c->D, g.rows) ? DecodeKernel::kRows
                                                              : DecodeKernel::kMfma;
  g.row_tile = g.kernel == DecodeKernel::kVector ? 1
               : g.kernel == DecodeKernel::kRows ? g.rows
                                                 : kvc::kMfmaRowTile;
  g.row_tiles = (g.rows + g.row_tile - 1) / g.row_tile;
  // (the single-row kernel's splits hold at least 4 keys per lane group)
  g.split_keys = g.kernel == DecodeKernel::kVector ? kvc::decode_rows_per_load(c->dtype, c->D) * 4
                 : g.kernel == DecodeKernel::kRows ? kvc::decode_rows_split_keys(c->dtype, c->D)
                                                   : kvc::decode_mfma_split_keys(c->dtype, c->D);
  g.max_splits = (c->Tmax + g.split_keys - 1) / g.split_keys;
  if (g.max_splits < 1) g.max_splits = 1;
  const size_t qrows = (size_t)n_layers * c->B * Hq * N;
  g.ws_o_bytes = round_up(qrows * g.max_splits * c->D * sizeof(float), 256);
  g.ws_ml_bytes = round_up(qrows * g.max_splits * 2 * sizeof(float), 256);
  // arrival counters of the single-row kernel's in-launch merge
  g.ctr_bytes = g.kernel == DecodeKernel::kVector ? round_up(qrows * sizeof(uint64_t), 256) : 0;
  g.total = g.ws_o_bytes + g.ws_ml_bytes + g.ctr_bytes;
  return g;
}

// Single-row kernel: keys per lane group (kpl; a split holds rows_per_load
// * kpl keys) and whether the merge runs inside the launch.  Measured
// (12-layer fp32 step at T=1024, and the same as 12 one-layer calls):
// in-launch merge with kpl 8 -- 16.2 us and 74 us per step -- beats kpl 4
// (17.1 / 78) and smaller splits by far (kpl 1: 43 / 185 us: every split
// of a row counts itself on one counter, so many splits serialise there),
// and the two-launch form at any kpl (best: kpl 4, 16.5 / 78 us).  The
// in-launch merge holds every split workgroup until the L2 has taken its
// state, which is hidden only while all of them are resident at once (about
// six per CU at kpl 8); larger grids merge in a second launch, with kpl 4.
constexpr long long kMaxMergeWorkgroups = 1280;

struct VectorPlan {
  int kpl;
  bool merge_in_launch;
};

VectorPlan plan_vector(int units, int max_keys, int rows_per_load, bool merge_supported) {
  const long long split8 = (long long)rows_per_load * 8;
  const long long splits8 = (max_keys + split8 - 1) / split8;
  const long long grid8 = 8LL * ((units + 7) / 8) * (splits8 > 0 ? splits8 : 1);
  if (merge_supported && grid8 <= kMaxMergeWorkgroups) return {8, true};
  return {4, false};
}

// XCDs of the current device (the attribute is read once per device): the
// in-launch merge needs every split of a row on one XCD, which the
// round-robin dispatch gives when the count divides 8.
bool merge_in_launch_supported() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 supported, 2 not (calls may come from any thread)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c) return c == 1;
  }
  int n = 0;
  const bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess &&
                  n >= 1 && n <= 8 && (8 % n) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok;
}

// Compute units of the current device (read once per device; 0 if the
// runtime does not say, which makes every prefill take key split 1).
int device_cus() {
  static std::atomic<int> cache[64];  // 0 unknown, else CUs + 1
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c) return c - 1;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
  if (dev < 64) cache[dev].store(n + 1, std::memory_order_relaxed);
  return n;
}

// Single-row calls whose rows alone about fill the chip (from one workgroup
// per two CUs to two per CU) run one workgroup per row (decode_row_kernel):
// no split states, arrival counters or merge through the L2.  Measured on
// the 12-layer fp32 step at T=1024 (144 rows on 256 CUs): see the kernel's
// notes.  Fewer rows leave most CUs idle (a one-layer call has 12), more
// queue behind one another, and the split grid serves both.
constexpr long long kRowKernelMaxPerCu = 2;

bool row_kernel_fits(int units) {
  const long long cus = device_cus();
  return cus > 0 && 2LL * units >= cus && units <= kRowKernelMaxPerCu * cus;
}

// Key split of a prefill call: from its grid at key split 1 (the first batch
// slice's), see kvc::prefill_key_split.
int prefill_ks(const kvc_cache *cache, int32_t n_layers, int32_t Hq, int max_len) {
  const long long nb = cache->B < kvc::kMaxBatchPerLaunch ? cache->B : kvc::kMaxBatchPerLaunch;
  const long long wg1 = (long long)n_layers * Hq * ((max_len + 127) / 128) * nb;
  return kvc::prefill_key_split(cache->dtype, cache->D, wg1, device_cus());
}

// Shared by kvc_append and kvc_paged_append (pg.block_table set: `cache` is
// the logical view of the pools, Tmax = max_blocks * block_size).
kvc_status append_impl(const char *fn, const kvc_cache *cache, const kvc::PagedGeom &pg,
                       int32_t layer0, int32_t n_layers, const void *k_new, const void *v_new,
                       int32_t N, const int32_t *hist_len, void *stream) {
  kvc_status st = check_cache(cache, layer0, n_layers, fn);
  if (st != KVC_OK) return st;
  if (N < 0) return fail(KVC_E_SHAPE, "%s: N = %d < 0", fn, N);
  if ((st = check_hist(cache, hist_len, N, fn)) != KVC_OK) return st;
  if (N == 0 || n_layers == 0 || cache->B == 0) return ok();
  if ((st = check_cache_pointers(cache, fn)) != KVC_OK) return st;
  if (!k_new || !v_new) return fail(KVC_E_NULL, "%s: k_new or v_new is NULL", fn);
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KVC_E_SHAPE, "%s: k_new / v_new must be 16-byte aligned", fn);

  kvc::AppendArgs a{};
  a.k_cache = (char *)cache->k;
  a.v_cache = (char *)cache->v;
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.B = cache->B;
  a.Hkv = cache->Hkv;
  a.Tmax = cache->Tmax;
  a.layer0 = layer0;
  a.n_layers = n_layers;
  a.N = N;
  a.row_vec16 = cache->D * elem_bytes(cache->dtype) / 16;
  a.pg = pg;
  for (int b0 = 0; b0 < cache->B; b0 += kvc::kMaxBatchPerLaunch) {
    a.b0 = b0;
    a.nb = cache->B - b0 < kvc::kMaxBatchPerLaunch ? cache->B - b0 : kvc::kMaxBatchPerLaunch;
    for (int i = 0; i < a.nb; ++i) a.hist[i] = hist_len[b0 + i];
    hipError_t e = kvc::launch_append(a, cache->dtype, cache->D, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

// A paged cache descriptor checked and turned into the logical view the
// shared implementations take: B sequences of max_blocks * block_size
// positions each, plus the block-table geometry.
kvc_status paged_view(const kvc_paged_cache *pc, int32_t B, const int32_t *block_table,
                      int32_t max_blocks, const char *fn, kvc_cache *view, kvc::PagedGeom *pg) {
  if (!pc) return fail(KVC_E_NULL, "%s: cache descriptor is NULL", fn);
  if (pc->num_blocks <= 0 || pc->block_size <= 0 || (pc->block_size & (pc->block_size - 1)) ||
      pc->block_size > 1024)
    return fail(KVC_E_SHAPE, "%s: num_blocks = %d must be > 0 and block_size = %d a power of two "
                "in [1, 1024]", fn, pc->num_blocks, pc->block_size);
  if (B < 0 || max_blocks < 0 || (int64_t)max_blocks * pc->block_size > 2147483647LL)
    return fail(KVC_E_SHAPE, "%s: B = %d, max_blocks = %d", fn, B, max_blocks);
  if (B > 0 && max_blocks > 0 && (!block_table || ((uintptr_t)block_table & 3u)))
    return fail(KVC_E_NULL, "%s: block_table is NULL or misaligned", fn);
  *view = kvc_cache{pc->k, pc->v, pc->L, B, pc->Hkv, max_blocks * pc->block_size, pc->D, pc->dtype};
  int log2 = 0;
  while ((1 << log2) < pc->block_size) ++log2;
  *pg = kvc::PagedGeom{block_table, max_blocks, pc->num_blocks, log2};
  return KVC_OK;
}

// Fields of a prefill launch shared by the padded and the packed entry
// points (validated arguments).
kvc::PrefillArgs prefill_args(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                              const void *q, const void *k, const void *v, int32_t Hq, float scale,
                              void *o) {
  kvc::PrefillArgs a{};
  a.k_cache = (char *)cache->k;
  a.v_cache = (char *)cache->v;
  a.q = (const char *)q;
  a.k = (const char *)k;
  a.v = (const char *)v;
  a.o = (char *)o;
  a.B = cache->B;
  a.Hkv = cache->Hkv;
  a.Hq = Hq;
  a.Tmax = cache->Tmax;
  a.layer0 = layer0;
  a.n_layers = n_layers;
  a.group = Hq / cache->Hkv;
  // The prefill kernel needs a positive exponent factor (see PrefillArgs):
  // a negative scale flips the sign of q, a zero one zeroes q.
  a.scale_log2 = (scale == 0.f ? 1.f : std::fabs(scale)) * 1.4426950408889634f;
  a.q_keep = scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_flip = scale < 0.f ? (cache->dtype == KVC_BF16 ? 0x80008000u : 0x80000000u) : 0u;
  return a;
}

void set_slice(kvc::PrefillArgs *a, int b0, int B) {
  a->b0 = b0;
  a->nb = B - b0 < kvc::kMaxBatchPerLaunch ? B - b0 : kvc::kMaxBatchPerLaunch;
}

// Shared by kvc_attn_prefill_varlen and kvc_paged_attn_prefill_varlen
// (pg.block_table set: `cache` is the logical view of the pools).
kvc_status varlen_impl(const char *fn, const kvc_cache *cache, const kvc::PagedGeom &pg,
                       int32_t layer0, int32_t n_layers, const void *q, const void *k,
                       const void *v, int32_t Hq, const int32_t *cu_seqlens,
                       const int32_t *hist_len, float scale, void *o, void *stream) {
  kvc_status st = check_cache(cache, layer0, n_layers, fn);
  if (st != KVC_OK) return st;
  if (Hq <= 0 || Hq % cache->Hkv != 0)
    return fail(KVC_E_SHAPE, "%s: Hq = %d is not a positive multiple of Hkv = %d", fn, Hq, cache->Hkv);
  if (!std::isfinite(scale)) return fail(KVC_E_SHAPE, "%s: scale is not finite", fn);
  if (!cu_seqlens) return fail(KVC_E_NULL, "%s: cu_seqlens is NULL", fn);
  if (cu_seqlens[0] != 0) return fail(KVC_E_SHAPE, "%s: cu_seqlens[0] = %d, not 0", fn, cu_seqlens[0]);
  for (int b = 0; b < cache->B; ++b)
    if (cu_seqlens[b + 1] < cu_seqlens[b])
      return fail(KVC_E_SHAPE, "%s: cu_seqlens decreases at %d", fn, b + 1);
  const int64_t T = cu_seqlens[cache->B];
  std::vector<int32_t> lens(cache->B);
  for (int b = 0; b < cache->B; ++b) lens[b] = cu_seqlens[b + 1] - cu_seqlens[b];
  // capacity: hist_len[b] + S_b <= Tmax, checked per sequence
  if (cache->B > 0 && !hist_len) return fail(KVC_E_NULL, "%s: hist_len is NULL", fn);
  for (int b = 0; b < cache->B; ++b) {
    if (hist_len[b] < 0) return fail(KVC_E_SHAPE, "%s: hist_len[%d] = %d < 0", fn, b, hist_len[b]);
    if ((int64_t)hist_len[b] + lens[b] > cache->Tmax)
      return fail(KVC_E_CAPACITY, "%s: hist_len[%d] + S_%d = %d + %d exceeds Tmax = %d", fn, b, b,
                  hist_len[b], lens[b], cache->Tmax);
  }
  if (T == 0 || n_layers == 0 || cache->B == 0) return ok();
  if ((st = check_cache_pointers(cache, fn)) != KVC_OK) return st;
  if (!q || !k || !v || !o) return fail(KVC_E_NULL, "%s: q, k, v or o is NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(KVC_E_SHAPE, "%s: q / k / v / o must be 16-byte aligned", fn);
  int max_len = 0;
  for (int b = 0; b < cache->B; ++b) max_len = lens[b] > max_len ? lens[b] : max_len;
  const int ks = prefill_ks(cache, n_layers, Hq, max_len);
  const int bm = kvc::prefill_query_tile(ks);
  const int64_t tiles = (max_len + bm - 1) / bm;
  if (tiles > 65535 || T * Hq >= 4294967296LL)
    return fail(KVC_E_UNSUPPORTED, "%s: too many query tiles or tokens for one launch", fn);

  // Packed token-major layout [n_layers, T, H, D].
  kvc::PrefillArgs a = prefill_args(cache, layer0, n_layers, q, k, v, Hq, scale, o);
  a.pg = pg;
  a.q_sl = T * Hq;
  a.q_sh = 1;
  a.q_si = Hq;
  a.kv_sl = T * cache->Hkv;
  a.kv_sh = 1;
  a.kv_si = cache->Hkv;
  for (int b0 = 0; b0 < cache->B; b0 += kvc::kMaxBatchPerLaunch) {
    set_slice(&a, b0, cache->B);
    int slice_len = 0;
    bool history = false;
    for (int i = 0; i < a.nb; ++i) {
      const int b = b0 + i;
      a.hist[i] = hist_len[b];
      a.len[i] = lens[b];
      a.q_row0[i] = (uint32_t)((int64_t)cu_seqlens[b] * Hq);
      a.kv_row0[i] = (uint32_t)((int64_t)cu_seqlens[b] * cache->Hkv);
      if (lens[b] > slice_len) slice_len = lens[b];
      if (hist_len[b] > 0 && lens[b] > 0) history = true;
    }
    a.q_tiles = (slice_len + bm - 1) / bm;
    hipError_t e = kvc::launch_prefill(a, cache->dtype, cache->D, history, ks, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

}  // namespace

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char *kvc_last_error(void) { return g_last_error; }

uint64_t kvc_cache_bytes(int64_t L, int64_t B, int64_t Hkv, int64_t Tmax, int64_t D, int32_t dtype) {
  if (L < 0 || B < 0 || Hkv < 0 || Tmax < 0 || D < 0) return 0;
  if (dtype != KVC_F32 && dtype != KVC_BF16) return 0;
  return (uint64_t)2 * L * Hkv * D * Tmax * B * elem_bytes(dtype);
}

kvc_status kvc_append(const kvc_cache *cache, int32_t layer0, int32_t n_layers, const void *k_new,
                      const void *v_new, int32_t N, const int32_t *hist_len, void *stream) {
  return append_impl("kvc_append", cache, kvc::PagedGeom{}, layer0, n_layers, k_new, v_new, N,
                     hist_len, stream);
}

size_t kvc_decode_workspace_bytes(const kvc_cache *cache, int32_t n_layers, int32_t Hq, int32_t N) {
  if (!cache || cache->Hkv <= 0 || cache->B < 0 || cache->Tmax < 0 || n_layers < 0 || Hq <= 0 ||
      N < 0 || Hq % cache->Hkv != 0 || (cache->D != 64 && cache->D != 128) ||
      (cache->dtype != KVC_F32 && cache->dtype != KVC_BF16))
    return 0;
  return decode_geometry(cache, n_layers, Hq, N).total;
}

}  // extern "C"

namespace {

enum Phases { kSplit = 1, kCombine = 2, kBoth = 3 };

// Scratch of kvc_decode_step_noalloc: 16 MiB per device (the split states of
// the 12-layer batched decode workloads fit), held from library load until
// the process ends.  The first 64 KiB are arrival counters (one per query
// row, 8192 rows), zero at load and left zero by every call; the states
// follow.  Host code uses the address hipGetSymbolAddress gives for the
// current device, never the array's name.
constexpr size_t kScratchCounterBytes = 64 * 1024;
constexpr size_t kScratchStateBytes = 16 * 1024 * 1024 - kScratchCounterBytes;
static __device__ __align__(256) unsigned char scratch[kScratchCounterBytes + kScratchStateBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];

// This device's copy of `scratch`, looked up on the first call per device
// (with that device current).
kvc_status scratch_for_current_device(const char *fn, void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVC_E_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(KVC_E_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVC_E_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KVC_OK;
}

// Shared by kvc_attn_decode, kvc_decode_step (fused: k_new / v_new given),
// kvc_decode_split and kvc_decode_combine.
kvc_status decode_impl(const char *fn, int phases, const kvc_cache *cache,
                       const kvc::PagedGeom &pg, int32_t layer0, int32_t n_layers, const void *q,
                       const void *k_new, const void *v_new, bool fused, int32_t Hq, int32_t N,
                       const int32_t *hist_len, float scale, void *o, void *workspace,
                       size_t workspace_bytes, void *stream, bool device_lengths = false,
                       const int32_t *hist_dev = nullptr, int32_t hist_max = 0,
                       bool in_scratch = false) {
  kvc_status st = check_cache(cache, layer0, n_layers, fn);
  if (st != KVC_OK) return st;
  if (N < 0) return fail(KVC_E_SHAPE, "%s: N = %d < 0", fn, N);
  if (Hq <= 0 || Hq % cache->Hkv != 0)
    return fail(KVC_E_SHAPE, "%s: Hq = %d is not a positive multiple of Hkv = %d", fn, Hq, cache->Hkv);
  if (!std::isfinite(scale)) return fail(KVC_E_SHAPE, "%s: scale is not finite", fn);
  if (device_lengths) {
    // lengths stay on the device: only their bound is checked here
    if (!hist_dev && N > 0 && n_layers > 0 && cache->B > 0)
      return fail(KVC_E_NULL, "%s: hist_len is NULL", fn);
    if (((uintptr_t)hist_dev & 3u) != 0)
      return fail(KVC_E_SHAPE, "%s: hist_len must be 4-byte aligned", fn);
    if (hist_max < 0) return fail(KVC_E_SHAPE, "%s: hist_max = %d < 0", fn, hist_max);
    if ((int64_t)hist_max + N > cache->Tmax)
      return fail(KVC_E_CAPACITY, "%s: hist_max + N = %d + %d exceeds Tmax = %d", fn, hist_max, N,
                  cache->Tmax);
  } else if ((st = check_hist(cache, hist_len, N, fn)) != KVC_OK) {
    return st;
  }
  if (N == 0 || n_layers == 0 || cache->B == 0) return ok();
  if ((st = check_cache_pointers(cache, fn)) != KVC_OK) return st;
  if (!q || !o) return fail(KVC_E_NULL, "%s: q or o is NULL", fn);
  if (!aligned16(q) || !aligned16(o))
    return fail(KVC_E_SHAPE, "%s: q / o must be 16-byte aligned", fn);
  if (fused) {
    if (!k_new || !v_new) return fail(KVC_E_NULL, "%s: k_new or v_new is NULL", fn);
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(KVC_E_SHAPE, "%s: k_new / v_new must be 16-byte aligned", fn);
  }
  const DecodeGeometry g = decode_geometry(cache, n_layers, Hq, N);
  if ((long long)n_layers * cache->Hkv * g.row_tiles > 65535)
    return fail(KVC_E_UNSUPPORTED, "%s: %d layers x %d KV heads x %d row tiles exceed one launch", fn,
                n_layers, cache->Hkv, g.row_tiles);
  // the single-row kernel's one-dimensional grid
  if (g.kernel == DecodeKernel::kVector &&
      8LL * ((n_layers * (long long)(cache->B < kvc::kMaxBatchPerLaunch ? cache->B : kvc::kMaxBatchPerLaunch) *
              cache->Hkv + 7) / 8) * g.max_splits > 2147483647LL)
    return fail(KVC_E_UNSUPPORTED, "%s: %d layers x %d KV heads x %d key splits exceed one launch", fn,
                n_layers, cache->Hkv, g.max_splits);
  // the multi-row vector kernel puts the splits on the grid's y axis
  if (g.kernel == DecodeKernel::kRows && g.max_splits > 65535)
    return fail(KVC_E_UNSUPPORTED, "%s: Tmax = %d gives %d key splits, more than one launch holds", fn,
                cache->Tmax, g.max_splits);
  // Workspace layout: [arrival counters][partial outputs][partial (max,
  // sum)].  The allocation-free entry point keeps its counters in a fixed
  // region of the library's scratch that no call writes states into, so
  // calls of any geometry leave them zero for the next one.
  size_t state_off = g.ctr_bytes;
  if (in_scratch) {
    if (g.ctr_bytes > kScratchCounterBytes || g.ws_o_bytes + g.ws_ml_bytes > kScratchStateBytes)
      return fail(KVC_E_WORKSPACE, "%s: this call needs %zu bytes of scratch (%zu of counters), more "
                  "than the %zu (%zu) the allocation-free entry point holds; use kvc_decode_step "
                  "with a workspace", fn, g.ws_o_bytes + g.ws_ml_bytes, g.ctr_bytes,
                  (size_t)kScratchStateBytes, (size_t)kScratchCounterBytes);
    state_off = kScratchCounterBytes;
    // every check has passed: only now touch the runtime
    if ((st = scratch_for_current_device(fn, &workspace)) != KVC_OK) return st;
  } else {
    if (!workspace) return fail(KVC_E_WORKSPACE, "%s: workspace is NULL", fn);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(KVC_E_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    if (workspace_bytes < g.total)
      return fail(KVC_E_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, g.total);
  }

  kvc::DecodeArgs a{};
  a.k_cache = (char *)cache->k;
  a.v_cache = (char *)cache->v;
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.q = (const char *)q;
  a.o = (char *)o;
  a.ws_o = (float *)((char *)workspace + state_off);
  a.ws_ml = (float *)((char *)workspace + state_off + g.ws_o_bytes);
  a.B = cache->B;
  a.Hkv = cache->Hkv;
  a.Hq = Hq;
  a.Tmax = cache->Tmax;
  a.N = N;
  a.layer0 = layer0;
  a.n_layers = n_layers;
  a.group = Hq / cache->Hkv;
  a.rows = g.rows;
  a.row_tiles = g.row_tiles;
  a.max_splits = g.max_splits;
  a.ws_rows = (int64_t)n_layers * cache->B * Hq * N;
  a.split_keys = g.split_keys;  // the single-row kernel picks its own per launch
  a.scale_log2 = scale * 1.4426950408889634f;
  a.hkv_div = kvc::magic_for(cache->Hkv);
  a.split_div = kvc::magic_for(g.split_keys);
  // Vector kernel: the split pass covers keys [0, P) and the combine pass
  // adds key P (from k_new / v_new in the fused step, which it then writes to
  // the cache, else from the cache), so both forms do the same arithmetic.
  a.tail = g.mfma ? 0 : 1;
  a.pg = pg;
  a.hist_dev = hist_dev;
  a.hist_max = hist_max;
  a.counters = g.ctr_bytes ? (uint64_t *)workspace : nullptr;
  a.nl_div = kvc::magic_for(n_layers);
  const bool vec = g.kernel == DecodeKernel::kVector;
  for (int b0 = 0; b0 < cache->B; b0 += kvc::kMaxBatchPerLaunch) {
    a.b0 = b0;
    a.nb = cache->B - b0 < kvc::kMaxBatchPerLaunch ? cache->B - b0 : kvc::kMaxBatchPerLaunch;
    int max_keys = 0;  // keys the split pass covers, longest sequence
    if (hist_dev) {
      // sized for the bound; workgroups past a sequence's own length exit
      max_keys = hist_max + (a.tail ? 0 : N);
    } else {
      for (int i = 0; i < a.nb; ++i) {
        a.hist[i] = hist_len[b0 + i];
        const int keys = hist_len[b0 + i] + (a.tail ? 0 : N);
        if (keys > max_keys) max_keys = keys;
      }
    }
    hipError_t e = hipSuccess;
    if (vec) {
      // Single-row kernel: split size for this call, then one launch with
      // the merge inside it, or the split pass and the combine pass.
      a.units = n_layers * a.nb * cache->Hkv;
      const int rpl = kvc::decode_rows_per_load(cache->dtype, cache->D);
      // the same plan for the one-call and the two-phase entry points, so
      // that their outputs are bit-identical
      const VectorPlan plan = plan_vector(a.units, max_keys, rpl, merge_in_launch_supported());
      const int kpl = plan.kpl;
      a.split_keys = rpl * kpl;
      a.split_div = kvc::magic_for(a.split_keys);
      const int splits = (max_keys + a.split_keys - 1) / a.split_keys;
      // a launch always covers every row: with no cached key (P = 0) the
      // merge alone gives the output (v_P)
      a.grid_splits = splits > 0 ? splits : 1;
      a.grid_splits_div = kvc::magic_for(a.grid_splits);
      // (a paged cache: block tables it can stage in LDS)
      const bool row_kernel = phases == kBoth && row_kernel_fits(a.units) &&
                              (!pg.block_table || pg.max_blocks <= kvc::decode_row_max_blocks());
      if (row_kernel) {
        e = kvc::launch_decode_row(a, cache->dtype, cache->D, (hipStream_t)stream);
      } else if (phases == kBoth && plan.merge_in_launch) {
        e = kvc::launch_decode(a, cache->dtype, cache->D, kpl, true, (hipStream_t)stream);
      } else {
        if ((phases & kSplit) && splits > 0)
          e = kvc::launch_decode(a, cache->dtype, cache->D, kpl, false, (hipStream_t)stream);
        if (e == hipSuccess && (phases & kCombine))
          e = kvc::launch_combine(a, cache->dtype, cache->D, (hipStream_t)stream);
      }
    } else {
      // Several rows per KV head: split pass, then the combine pass (an
      // in-launch merge measured no faster here: these grids exceed one
      // resident round, so each split's wait for its state stores queues the
      // next workgroups).
      const int splits = (max_keys + g.split_keys - 1) / g.split_keys;
      // One workgroup per (layer, sequence, KV head) over the whole key range
      // when those alone about fill the chip, as for one row per KV head.
      const int heads = n_layers * a.nb * cache->Hkv;
      if (phases == kBoth && g.kernel == DecodeKernel::kRows && row_kernel_fits(heads) &&
          (!pg.block_table || pg.max_blocks <= kvc::decode_rows_loop_max_blocks())) {
        e = kvc::launch_decode_rows_loop(a, cache->dtype, cache->D, fused, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, fn);
        continue;
      }
      if ((phases & kSplit) && splits > 0)
        e = g.kernel == DecodeKernel::kRows
                ? kvc::launch_decode_rows(a, cache->dtype, cache->D, splits, fused, (hipStream_t)stream)
                : kvc::launch_decode_mfma(a, cache->dtype, cache->D, splits, fused, (hipStream_t)stream);
      if (e == hipSuccess && (phases & kCombine) && splits > 1)
        e = kvc::launch_combine(a, cache->dtype, cache->D, (hipStream_t)stream);
    }
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

}  // namespace

extern "C" {

kvc_status kvc_attn_decode(const kvc_cache *cache, int32_t layer0, int32_t n_layers, const void *q,
                           int32_t Hq, int32_t N, const int32_t *hist_len, float scale, void *o,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl("kvc_attn_decode", kBoth, cache, kvc::PagedGeom{}, layer0, n_layers, q, nullptr, nullptr, false,
                     Hq, N, hist_len, scale, o, workspace, workspace_bytes, stream);
}

kvc_status kvc_decode_step(const kvc_cache *cache, int32_t layer0, int32_t n_layers, const void *q,
                           const void *k_new, const void *v_new, int32_t Hq, int32_t N,
                           const int32_t *hist_len, float scale, void *o, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return decode_impl("kvc_decode_step", kBoth, cache, kvc::PagedGeom{}, layer0, n_layers, q, k_new, v_new, true, Hq,
                     N, hist_len, scale, o, workspace, workspace_bytes, stream);
}

kvc_status kvc_decode_step_noalloc(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                                   const void *q, const void *k_new, const void *v_new, int32_t Hq,
                                   int32_t N, const int32_t *hist_len, float scale, void *o,
                                   void *stream) {
  return decode_impl("kvc_decode_step_noalloc", kBoth, cache, kvc::PagedGeom{}, layer0, n_layers,
                     q, k_new, v_new, true, Hq, N, hist_len, scale, o, nullptr, 0, stream, false,
                     nullptr, 0, true);
}

kvc_status kvc_decode_step_dl(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                              const void *q, const void *k_new, const void *v_new, int32_t Hq,
                              int32_t N, const int32_t *hist_len_dev, int32_t hist_max, float scale,
                              void *o, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl("kvc_decode_step_dl", kBoth, cache, kvc::PagedGeom{}, layer0, n_layers, q,
                     k_new, v_new, true, Hq, N, nullptr, scale, o, workspace, workspace_bytes,
                     stream, true, hist_len_dev, hist_max);
}

kvc_status kvc_lengths_add(int32_t *hist_len_dev, int32_t B, int32_t n, void *stream) {
  if (B < 0) return fail(KVC_E_SHAPE, "kvc_lengths_add: B = %d < 0", B);
  if (B == 0 || n == 0) return ok();
  if (!hist_len_dev) return fail(KVC_E_NULL, "kvc_lengths_add: hist_len is NULL");
  if (((uintptr_t)hist_len_dev & 3u) != 0)
    return fail(KVC_E_SHAPE, "kvc_lengths_add: hist_len must be 4-byte aligned");
  hipError_t e = kvc::launch_lengths_add(hist_len_dev, B, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "kvc_lengths_add");
  return ok();
}

kvc_status kvc_decode_split(const kvc_cache *cache, int32_t layer0, int32_t n_layers, const void *q,
                            const void *k_new, const void *v_new, int32_t Hq, int32_t N,
                            const int32_t *hist_len, float scale, void *o, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(KVC_E_NULL, "kvc_decode_split: k_new and v_new must both be given or both NULL");
  return decode_impl("kvc_decode_split", kSplit, cache, kvc::PagedGeom{}, layer0, n_layers, q, k_new, v_new,
                     k_new != nullptr, Hq, N, hist_len, scale, o, workspace, workspace_bytes,
                     stream);
}

kvc_status kvc_decode_combine(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                              const void *q, const void *k_new, const void *v_new, int32_t Hq,
                              int32_t N, const int32_t *hist_len, float scale, void *o,
                              void *workspace, size_t workspace_bytes, void *stream) {
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(KVC_E_NULL, "kvc_decode_combine: k_new and v_new must both be given or both NULL");
  return decode_impl("kvc_decode_combine", kCombine, cache, kvc::PagedGeom{}, layer0, n_layers, q, k_new, v_new,
                     k_new != nullptr, Hq, N, hist_len, scale, o, workspace, workspace_bytes,
                     stream);
}

kvc_status kvc_attn_prefill(const kvc_cache *cache, int32_t layer0, int32_t n_layers, const void *q,
                            const void *k, const void *v, int32_t Hq, int32_t S, float scale, void *o,
                            void *stream) {
  static const char *fn = "kvc_attn_prefill";
  kvc_status st = check_cache(cache, layer0, n_layers, fn);
  if (st != KVC_OK) return st;
  if (S < 0) return fail(KVC_E_SHAPE, "%s: S = %d < 0", fn, S);
  if (Hq <= 0 || Hq % cache->Hkv != 0)
    return fail(KVC_E_SHAPE, "%s: Hq = %d is not a positive multiple of Hkv = %d", fn, Hq, cache->Hkv);
  if (!std::isfinite(scale)) return fail(KVC_E_SHAPE, "%s: scale is not finite", fn);
  if (S > cache->Tmax)
    return fail(KVC_E_CAPACITY, "%s: S = %d exceeds Tmax = %d", fn, S, cache->Tmax);
  if (S == 0 || n_layers == 0 || cache->B == 0) return ok();
  if ((st = check_cache_pointers(cache, fn)) != KVC_OK) return st;
  if (!q || !k || !v || !o) return fail(KVC_E_NULL, "%s: q, k, v or o is NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(KVC_E_SHAPE, "%s: q / k / v / o must be 16-byte aligned", fn);
  const int ks = prefill_ks(cache, n_layers, Hq, S);
  const int bm = kvc::prefill_query_tile(ks);
  const int64_t tiles = (S + bm - 1) / bm;
  if (tiles > 65535 || (int64_t)cache->B * Hq * S >= 4294967296LL)
    return fail(KVC_E_UNSUPPORTED, "%s: too many query tiles or rows for one launch", fn);

  // Padded layout [n_layers, B, H, S, D]: no history, S new tokens each.
  const int64_t B = cache->B;
  kvc::PrefillArgs a = prefill_args(cache, layer0, n_layers, q, k, v, Hq, scale, o);
  a.q_sl = B * Hq * S;
  a.q_sh = S;
  a.q_si = 1;
  a.kv_sl = B * cache->Hkv * S;
  a.kv_sh = S;
  a.kv_si = 1;
  for (int b0 = 0; b0 < cache->B; b0 += kvc::kMaxBatchPerLaunch) {
    set_slice(&a, b0, cache->B);
    for (int i = 0; i < a.nb; ++i) {
      a.hist[i] = 0;
      a.len[i] = S;
      a.q_row0[i] = (uint32_t)((int64_t)(b0 + i) * Hq * S);
      a.kv_row0[i] = (uint32_t)((int64_t)(b0 + i) * cache->Hkv * S);
    }
    a.q_tiles = (S + bm - 1) / bm;
    hipError_t e = kvc::launch_prefill(a, cache->dtype, cache->D, false, ks, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

kvc_status kvc_attn_prefill_varlen(const kvc_cache *cache, int32_t layer0, int32_t n_layers,
                                   const void *q, const void *k, const void *v, int32_t Hq,
                                   const int32_t *cu_seqlens, const int32_t *hist_len, float scale,
                                   void *o, void *stream) {
  return varlen_impl("kvc_attn_prefill_varlen", cache, kvc::PagedGeom{}, layer0, n_layers, q, k, v,
                     Hq, cu_seqlens, hist_len, scale, o, stream);
}

}  // extern "C"

// ---- paged cache -----------------------------------------------------------

extern "C" {

uint64_t kvc_paged_cache_bytes(int64_t L, int64_t num_blocks, int64_t Hkv, int64_t block_size,
                               int64_t D, int32_t dtype) {
  if (L < 0 || num_blocks < 0 || Hkv < 0 || block_size < 0 || D < 0) return 0;
  if (dtype != KVC_F32 && dtype != KVC_BF16) return 0;
  return (uint64_t)2 * L * num_blocks * Hkv * block_size * D * elem_bytes(dtype);
}

kvc_status kvc_paged_append(const kvc_paged_cache *cache, int32_t layer0, int32_t n_layers,
                            const void *k_new, const void *v_new, int32_t B, int32_t N,
                            const int32_t *hist_len, const int32_t *block_table,
                            int32_t max_blocks, void *stream) {
  static const char *fn = "kvc_paged_append";
  kvc_cache view;
  kvc::PagedGeom pg;
  kvc_status st = paged_view(cache, B, block_table, max_blocks, fn, &view, &pg);
  if (st != KVC_OK) return st;
  return append_impl(fn, &view, pg, layer0, n_layers, k_new, v_new, N, hist_len, stream);
}

size_t kvc_paged_decode_workspace_bytes(const kvc_paged_cache *cache, int32_t n_layers, int32_t B,
                                        int32_t Hq, int32_t N, int32_t max_blocks) {
  if (!cache || cache->block_size <= 0 || B < 0 || max_blocks < 0 ||
      (int64_t)max_blocks * cache->block_size > 2147483647LL)
    return 0;
  const kvc_cache view{cache->k, cache->v, cache->L, B, cache->Hkv,
                       max_blocks * cache->block_size, cache->D, cache->dtype};
  return kvc_decode_workspace_bytes(&view, n_layers, Hq, N);
}

kvc_status kvc_paged_attn_decode(const kvc_paged_cache *cache, int32_t layer0, int32_t n_layers,
                                 const void *q, int32_t Hq, int32_t B, int32_t N,
                                 const int32_t *hist_len, const int32_t *block_table,
                                 int32_t max_blocks, float scale, void *o, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  static const char *fn = "kvc_paged_attn_decode";
  kvc_cache view;
  kvc::PagedGeom pg;
  kvc_status st = paged_view(cache, B, block_table, max_blocks, fn, &view, &pg);
  if (st != KVC_OK) return st;
  return decode_impl(fn, kBoth, &view, pg, layer0, n_layers, q, nullptr, nullptr, false, Hq, N,
                     hist_len, scale, o, workspace, workspace_bytes, stream);
}

kvc_status kvc_paged_decode_step_dl(const kvc_paged_cache *cache, int32_t layer0,
                                    int32_t n_layers, const void *q, const void *k_new,
                                    const void *v_new, int32_t Hq, int32_t B, int32_t N,
                                    const int32_t *hist_len_dev, int32_t hist_max,
                                    const int32_t *block_table, int32_t max_blocks, float scale,
                                    void *o, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  static const char *fn = "kvc_paged_decode_step_dl";
  kvc_cache view;
  kvc::PagedGeom pg;
  kvc_status st = paged_view(cache, B, block_table, max_blocks, fn, &view, &pg);
  if (st != KVC_OK) return st;
  return decode_impl(fn, kBoth, &view, pg, layer0, n_layers, q, k_new, v_new, true, Hq, N, nullptr,
                     scale, o, workspace, workspace_bytes, stream, true, hist_len_dev, hist_max);
}

kvc_status kvc_paged_decode_step(const kvc_paged_cache *cache, int32_t layer0, int32_t n_layers,
                                 const void *q, const void *k_new, const void *v_new, int32_t Hq,
                                 int32_t B, int32_t N, const int32_t *hist_len,
                                 const int32_t *block_table, int32_t max_blocks, float scale,
                                 void *o, void *workspace, size_t workspace_bytes, void *stream) {
  static const char *fn = "kvc_paged_decode_step";
  kvc_cache view;
  kvc::PagedGeom pg;
  kvc_status st = paged_view(cache, B, block_table, max_blocks, fn, &view, &pg);
  if (st != KVC_OK) return st;
  return decode_impl(fn, kBoth, &view, pg, layer0, n_layers, q, k_new, v_new, true, Hq, N,
                     hist_len, scale, o, workspace, workspace_bytes, stream);
}

kvc_status kvc_linear_f32(const float *x, int32_t a_heads, int32_t M, int32_t K, const float *wt,
                          int32_t N, const float *bias, const float *ln_g, const float *ln_b,
                          float ln_eps, int32_t act, const float *res, float *y, int32_t y_qkv_heads,
                          void *stream) {
  static const char *fn = "kvc_linear_f32";
  if (!x || !wt || !y) return fail(KVC_E_NULL, "%s: x, wt or y is NULL", fn);
  if ((ln_g == nullptr) != (ln_b == nullptr))
    return fail(KVC_E_NULL, "%s: ln_g and ln_b must both be given or both NULL", fn);
  if (M < 1 || K < 4 || N < 1 || K % 4 != 0)
    return fail(KVC_E_SHAPE, "%s: M = %d, K = %d, N = %d (need M >= 1, K a positive multiple of 4, "
                "N >= 1)", fn, M, K, N);
  if (M > kvc::kMaxLinearRows || (int64_t)M * K > kvc::kMaxLinearInputs)
    return fail(KVC_E_UNSUPPORTED, "%s: M = %d rows of K = %d inputs exceed %d rows / %d inputs", fn, M,
                K, kvc::kMaxLinearRows, kvc::kMaxLinearInputs);
  if ((int64_t)N * K >= ((int64_t)1 << 31) || N > 65535 * 16)
    return fail(KVC_E_UNSUPPORTED, "%s: N = %d, K = %d too large for one launch", fn, N, K);
  if (act != 0 && act != 1) return fail(KVC_E_SHAPE, "%s: act = %d (0 or 1)", fn, act);
  if (ln_g && !(std::isfinite(ln_eps) && ln_eps >= 0.f))
    return fail(KVC_E_SHAPE, "%s: ln_eps must be finite and >= 0", fn);
  if (a_heads < 0 || (a_heads > 0 && (K % a_heads != 0 || (K / a_heads) % 4 != 0)))
    return fail(KVC_E_SHAPE, "%s: a_heads = %d must split K = %d into parts of a multiple of 4", fn,
                a_heads, K);
  if (a_heads > 0 && ln_g)
    return fail(KVC_E_UNSUPPORTED, "%s: the layer norm needs the row-major input", fn);
  if (y_qkv_heads < 0 ||
      (y_qkv_heads > 0 && (N % (3 * y_qkv_heads) != 0 || (N / (3 * y_qkv_heads)) % 4 != 0)))
    return fail(KVC_E_SHAPE, "%s: y_qkv_heads = %d must split N = %d into 3 x heads parts of a "
                "multiple of 4", fn, y_qkv_heads, N);
  if (y_qkv_heads > 0 && res)
    return fail(KVC_E_UNSUPPORTED, "%s: a residual needs the row-major output", fn);
  if (!aligned16(x) || !aligned16(wt) || !aligned16(y) || (res && !aligned16(res)) ||
      (ln_g && (((uintptr_t)ln_g & 3u) || ((uintptr_t)ln_b & 3u))))
    return fail(KVC_E_SHAPE, "%s: x, wt, res and y must be 16-byte aligned", fn);
  const char *xb = (const char *)x, *xe = xb + (size_t)M * K * sizeof(float);
  const char *yb = (const char *)y, *ye = yb + (size_t)M * N * sizeof(float);
  if (yb < xe && xb < ye) return fail(KVC_E_SHAPE, "%s: y overlaps x", fn);
  if (res && res != y) {
    const char *rb = (const char *)res, *re = rb + (size_t)M * N * sizeof(float);
    if (yb < re && rb < ye) return fail(KVC_E_SHAPE, "%s: y overlaps res without being it", fn);
  }
  kvc::LinearArgs a{};
  a.x = x;
  a.wt = wt;
  a.bias = bias;
  a.ln_g = ln_g;
  a.ln_b = ln_b;
  a.res = res;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.act = act;
  a.ln_eps = ln_eps;
  a.a_heads = M > 1 ? a_heads : 0;          // one row: every layout is row-major
  a.y_qkv_heads = M > 1 ? y_qkv_heads : 0;
  hipError_t e = kvc::launch_linear(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, fn);
  return ok();
}

size_t kvc_gemm_workspace_bytes(int32_t M, int32_t K, int32_t N) {
  if (M < 1 || K < 64 || N < 1 || K % 64 != 0) return 0;
  const int splits = merge_in_launch_supported() ? kvc::gemm_splits(M, K, N) : 1;
  return kvc::gemm_workspace_bytes(M, K, N, splits);
}

kvc_status kvc_gemm_f32(const float *a, int32_t a_heads, int32_t M, int32_t K, const float *wt,
                        int32_t N, const float *bias, int32_t act, const float *res, float *y,
                        int32_t y_qkv_heads, void *workspace, size_t workspace_bytes, void *stream) {
  static const char *fn = "kvc_gemm_f32";
  if (M < 0 || K < 64 || N < 1 || K % 64 != 0)
    return fail(KVC_E_SHAPE, "%s: M = %d, K = %d, N = %d (need M >= 0, K a positive multiple of 64, "
                "N >= 1)", fn, M, K, N);
  if (act != 0 && act != 1) return fail(KVC_E_SHAPE, "%s: act = %d (0 or 1)", fn, act);
  if (a_heads < 0 || (a_heads > 0 && (K % a_heads != 0 || (K / a_heads) % 64 != 0)))
    return fail(KVC_E_SHAPE, "%s: a_heads = %d must split K = %d into parts of a multiple of 64", fn,
                a_heads, K);
  if (y_qkv_heads < 0 ||
      (y_qkv_heads > 0 && (N % (3 * y_qkv_heads) != 0 || (N / (3 * y_qkv_heads)) % 4 != 0)))
    return fail(KVC_E_SHAPE, "%s: y_qkv_heads = %d must split N = %d into 3 x heads parts of a "
                "multiple of 4", fn, y_qkv_heads, N);
  if (y_qkv_heads > 0 && res)
    return fail(KVC_E_UNSUPPORTED, "%s: a residual needs the row-major output", fn);
  if ((int64_t)M * N >= ((int64_t)1 << 31) || (int64_t)M * K >= ((int64_t)1 << 31) ||
      (int64_t)K * N >= ((int64_t)1 << 31) || (M + 63) / 64 > 65535)
    return fail(KVC_E_UNSUPPORTED, "%s: M = %d, K = %d, N = %d too large for one launch", fn, M, K, N);
  if (M == 0) return ok();
  if (!a || !wt || !y) return fail(KVC_E_NULL, "%s: a, wt or y is NULL", fn);
  if (!aligned16(a) || !aligned16(wt) || !aligned16(y) || (res && !aligned16(res)) ||
      (bias && ((uintptr_t)bias & 3u)))
    return fail(KVC_E_SHAPE, "%s: a, wt, res and y must be 16-byte aligned", fn);
  const char *ab = (const char *)a, *ae = ab + (size_t)M * K * sizeof(float);
  const char *yb = (const char *)y, *ye = yb + (size_t)M * N * sizeof(float);
  if (yb < ae && ab < ye) return fail(KVC_E_SHAPE, "%s: y overlaps a", fn);
  if (res && res != y) {
    const char *rb = (const char *)res, *re = rb + (size_t)M * N * sizeof(float);
    if (yb < re && rb < ye) return fail(KVC_E_SHAPE, "%s: y overlaps res without being it", fn);
  }
  kvc::GemmArgs g{};
  g.a = a;
  g.wt = wt;
  g.bias = bias;
  g.res = res;
  g.y = y;
  g.M = M;
  g.K = K;
  g.N = N;
  g.act = act;
  g.a_heads = a_heads;
  g.y_qkv_heads = y_qkv_heads;
  g.splits = 1;
  g.tiles_m = (M + 63) / 64;
  g.tiles_n = (N + 63) / 64;
  if (workspace) {
    // split K when the output tiles alone leave the chip idle
    const int splits = merge_in_launch_supported() ? kvc::gemm_splits(M, K, N) : 1;
    const size_t need = kvc::gemm_workspace_bytes(M, K, N, splits);
    if (workspace_bytes < need)
      return fail(KVC_E_WORKSPACE, "%s: workspace of %zu bytes, need %zu (kvc_gemm_workspace_bytes)", fn,
                  workspace_bytes, need);
    if ((uintptr_t)workspace & 255u) return fail(KVC_E_SHAPE, "%s: workspace must be 256-byte aligned", fn);
    if (splits > 1) {
      g.splits = splits;
      g.ctr = (uint64_t *)workspace;
      g.part = (float *)((char *)workspace + kvc::kGemmCounterBytes);
    }
  }
  hipError_t e = kvc::launch_gemm(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, fn);
  return ok();
}

kvc_status kvc_layernorm_f32(const float *x, int32_t M, int32_t K, const float *g, const float *b,
                             float eps, float *y, void *stream) {
  static const char *fn = "kvc_layernorm_f32";
  if (M < 0 || K < 4 || K % 4 != 0 || K > 4096)
    return fail(KVC_E_SHAPE, "%s: M = %d, K = %d (need M >= 0, K a positive multiple of 4 up to 4096)",
                fn, M, K);
  if (!(std::isfinite(eps) && eps >= 0.f)) return fail(KVC_E_SHAPE, "%s: eps must be finite and >= 0", fn);
  if (M == 0) return ok();
  if (!x || !g || !b || !y) return fail(KVC_E_NULL, "%s: x, g, b or y is NULL", fn);
  if (!aligned16(x) || !aligned16(g) || !aligned16(b) || !aligned16(y))
    return fail(KVC_E_SHAPE, "%s: x, g, b and y must be 16-byte aligned", fn);
  kvc::LayerNormArgs p{};
  p.x = x;
  p.g = g;
  p.b = b;
  p.y = y;
  p.M = M;
  p.K = K;
  p.eps = eps;
  hipError_t e = kvc::launch_layernorm(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, fn);
  return ok();
}

kvc_status kvc_embed_f32(const float *wte, int32_t V, const float *wpe, int32_t T, int32_t d,
                         const int64_t *ids, int32_t N, int32_t pos0, const int32_t *pos, float *y,
                         void *stream) {
  static const char *fn = "kvc_embed_f32";
  if (V < 1 || T < 1 || d < 4 || d % 4 != 0 || N < 0 || N > 65535)
    return fail(KVC_E_SHAPE, "%s: V = %d, T = %d, d = %d, N = %d (need V, T >= 1, d a positive multiple "
                "of 4, 0 <= N <= 65535)", fn, V, T, d, N);
  if ((int64_t)V * d >= ((int64_t)1 << 40) || (int64_t)T * d >= ((int64_t)1 << 40))
    return fail(KVC_E_SHAPE, "%s: tables too large", fn);
  if (!pos && (pos0 < 0 || (int64_t)pos0 + N > T))
    return fail(KVC_E_SHAPE, "%s: positions %d .. %lld outside [0, %d)", fn, pos0, (long long)pos0 + N - 1,
                T);
  if (N == 0) return ok();
  if (!wte || !wpe || !ids || !y) return fail(KVC_E_NULL, "%s: wte, wpe, ids or y is NULL", fn);
  if (!aligned16(wte) || !aligned16(wpe) || !aligned16(y))
    return fail(KVC_E_SHAPE, "%s: wte, wpe and y must be 16-byte aligned", fn);
  const char *yb = (const char *)y, *ye = yb + (size_t)N * d * sizeof(float);
  const char *tb = (const char *)wte, *te = tb + (size_t)V * d * sizeof(float);
  const char *pb = (const char *)wpe, *pe = pb + (size_t)T * d * sizeof(float);
  if ((yb < te && tb < ye) || (yb < pe && pb < ye)) return fail(KVC_E_SHAPE, "%s: y overlaps a table", fn);
  kvc::EmbedArgs e{};
  e.wte = wte;
  e.wpe = wpe;
  e.ids = ids;
  e.pos = pos;
  e.y = y;
  e.V = V;
  e.T = T;
  e.d = d;
  e.N = N;
  e.pos0 = pos0;
  hipError_t err = kvc::launch_embed(e, (hipStream_t)stream);
  if (err != hipSuccess) return hip_status(err, fn);
  return ok();
}

kvc_status kvc_argmax_f32(const float *x, int64_t n, int64_t *index, int64_t *seq, int64_t *seq_pos,
                          int64_t seq_capacity, void *stream) {
  static const char *fn = "kvc_argmax_f32";
  if (n < 1 || n >= ((int64_t)1 << 31))
    return fail(KVC_E_SHAPE, "%s: n = %lld (need 1 <= n < 2^31)", fn, (long long)n);
  if (!x || !index) return fail(KVC_E_NULL, "%s: x or index is NULL", fn);
  if (!seq != !seq_pos) return fail(KVC_E_NULL, "%s: seq and seq_pos must both be given or both NULL", fn);
  if (seq && seq_capacity < 1)
    return fail(KVC_E_SHAPE, "%s: seq_capacity = %lld (need >= 1)", fn, (long long)seq_capacity);
  if (!aligned16(x)) return fail(KVC_E_SHAPE, "%s: x must be 16-byte aligned", fn);
  kvc::ArgmaxArgs a{};
  a.x = x;
  a.index = index;
  a.seq = seq;
  a.seq_pos = seq_pos;
  a.cap = seq ? seq_capacity : 0;
  a.n = (int32_t)n;
  hipError_t err = kvc::launch_argmax(a, (hipStream_t)stream);
  if (err != hipSuccess) return hip_status(err, fn);
  return ok();
}

kvc_status kvc_paged_attn_prefill_varlen(const kvc_paged_cache *cache, int32_t layer0,
                                         int32_t n_layers, const void *q, const void *k,
                                         const void *v, int32_t Hq, int32_t B,
                                         const int32_t *cu_seqlens, const int32_t *hist_len,
                                         const int32_t *block_table, int32_t max_blocks,
                                         float scale, void *o, void *stream) {
  static const char *fn = "kvc_paged_attn_prefill_varlen";
  kvc_cache view;
  kvc::PagedGeom pg;
  kvc_status st = paged_view(cache, B, block_table, max_blocks, fn, &view, &pg);
  if (st != KVC_OK) return st;
  return varlen_impl(fn, &view, pg, layer0, n_layers, q, k, v, Hq, cu_seqlens, hist_len, scale, o,
                     stream);
}

}  // extern "C"
