// kvc_gemm.hip -- the dense layers of a decoder block for a whole prompt:
// a row-wise layer norm and an fp32 matrix product on the matrix cores with
// its bias, GELU and residual fused into the store.
//
//   y[m][n] = act( sum_k a[m][k] wt[n][k] + bias[n] ) + res[m][n]
//
// [KV-2] openai-hub.com/news/2435, "千倍计算量为何只换来6倍速度": without the
// cache every step runs the projections and the MLP of every position of
// the context again -- products of the context length times the model
// width, dense contractions that belong on the matrix cores (the cached
// step runs them for the new token only, kvc_dense.hip).
//
// Layouts.  The weight comes transposed, wt [N][K] (output feature n's K
// input weights contiguous, the usual layout of a linear layer's weight),
// packed once when a model is loaded.  a is row-major [M][K], or
// "head-major" [H][M][K/H] -- the attention output as the prefill writes
// it -- so the output projection reads it without a transpose.  y is
// row-major [M][N], or for the QKV product the attention layout
// [3][H][M][N/(3H)] (q, k, v, each head's rows contiguous), which is what
// the prefill reads, so no permute runs between the two.
//
// Tiling.  A workgroup of 4 waves owns a 64 x 64 output tile; wave (wm, wn)
// computes its 32 x 32 quarter with v_mfma_f32_32x32x2_f32 (fp32 in, fp32
// accumulate: no reduced precision).  K advances 64 per tile.  Both
// operands sit in LDS k-contiguous, as they come from memory (rows of a,
// rows of wt), so staging is 16-byte stores; MFMA step s of a tile
// contracts feature 32 h + s in half-wave h, so each lane reads its 32
// operands of a tile with eight 16-byte LDS loads.  LDS is double-buffered
// and the pipeline keeps the matrix cores fed: while a tile's 32 MFMAs run,
// the same wave stages the next tile (already in registers) into the other
// buffer and issues the global loads of the tile after that, interleaved
// with the MFMAs, with one barrier per tile.  Rows past M and columns past
// N are clamped on load and skipped on store.
//
// Split K.  A product with few output tiles (a short prompt: M = 128 gives
// 24-96 tiles for 256 CUs) leaves most CUs idle while each workgroup walks
// all of K.  Given a workspace, such a product runs S workgroups per tile,
// each over a contiguous 1/S of the K tiles; each stores its partial tile,
// waits until the L2 has it and counts itself on the tile's arrival counter
// (the same counter as the decode step's in-launch merge, XCD check
// included); the last to arrive sums the S partials in split order -- the
// same sum whichever split came last -- applies the epilogue and clears the
// counter.  The 1-D grid puts every split of a tile on one XCD.
//
// Roofline: MFMA (fp32 matrix peak 157.3 TFLOP/s), 2 M N K flops per call.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GM = 64;  // tile rows
constexpr int GN = 64;  // tile columns
constexpr int GK = 64;  // tile depth
// LDS row stride: 4 floats past the tile depth, so the 16 lanes of one
// 128-bit access (rows i = 0..15 at one offset) fall on distinct banks.
constexpr int LDS_STRIDE = GK + 4;
constexpr int TILE_FLOATS = 64 * LDS_STRIDE;
constexpr int CHAINS = 2;  // independent accumulators per wave (step s feeds chain s % 2)

__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
  const float c = 0.7978845608028654f;
  return 0.5f * v * (1.f + tanhf(c * (v + 0.044715f * v * v * v)));
}

// Offset of output element (m, n): row-major, or the [3][H][M][DH] attention
// layout with DH = N / (3 H).
__device__ __forceinline__ size_t y_index(const GemmArgs &g, int m, int n) {
  if (g.y_qkv_heads > 0) {
    const int dh = g.N / (3 * g.y_qkv_heads);
    const int j = n / dh;  // which * H + head
    return ((size_t)j * g.M + m) * dh + (n - j * dh);
  }
  return (size_t)m * g.N + n;
}

__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ float al[2 * TILE_FLOATS];  // a tile: al[buf][m][k]
  __shared__ float wl[2 * TILE_FLOATS];  // wt tile: wl[buf][n][k]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = g.M, N = g.N, K = g.K;
  const int nt = K / GK;
  // Output tile and K range.  Without a split: the 2-D grid's tile, all of
  // K.  With one: a 1-D grid in which workgroup i runs on XCD i % 8 and the
  // S splits of a tile share that XCD (their partials meet in its L2):
  // i = 8 (S u + s) + x for tile 8 u + x, split s.
  const int S = g.splits;
  int tile = 0, split = 0, m0, n0;
  if (S > 1) {
    const int i = blockIdx.x, x = i & 7, j = i >> 3;
    split = j % S;
    tile = (j / S) * 8 + x;
    if (tile >= g.tiles_m * g.tiles_n) return;  // padding to a multiple of 8 tiles
    m0 = (tile / g.tiles_n) * GM;
    n0 = (tile % g.tiles_n) * GN;
  } else {
    m0 = blockIdx.y * GM;
    n0 = blockIdx.x * GN;
  }
  const int tb = (int)((long long)split * nt / S), te = (int)((long long)(split + 1) * nt / S);

  // This thread's share of a tile: features k0 + lc .. +3 of rows lr + 16 i
  // (i < 4) of a and of wt, one 16-byte vector each.  Row pointers are
  // fixed; a tile adds a uniform offset (k0, or for head-major a the
  // tile's head block and the offset inside it -- a head's K/H features
  // are a multiple of the tile depth).
  const int lr = tid >> 4, lc = 4 * (tid & 15);
  const float *ap[4], *wp[4];
  const int dh = g.a_heads > 0 ? K / g.a_heads : K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + lr + 16 * i;
    m = m < M ? m : M - 1;
    ap[i] = g.a + (size_t)m * dh + lc;
    int n = n0 + lr + 16 * i;
    n = n < N ? n : N - 1;
    wp[i] = g.wt + (size_t)n * K + lc;
  }
  auto a_off = [&](int t) -> size_t {
    const int k0 = t * GK;
    if (g.a_heads > 0) {
      const int h = k0 / dh;
      return (size_t)h * M * dh + (k0 - h * dh);
    }
    return (size_t)k0;
  };
  f32x4 av[2][4], wv[2][4];
  auto load = [&](int t, int r) {
    const size_t ao = a_off(t), wo = (size_t)t * GK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[r][i] = *reinterpret_cast<const f32x4 *>(ap[i] + ao);
      wv[r][i] = *reinterpret_cast<const f32x4 *>(wp[i] + wo);
    }
  };
  auto stage = [&](int r, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4 *>(&al[buf * TILE_FLOATS + (lr + 16 * i) * LDS_STRIDE + lc]) = av[r][i];
      *reinterpret_cast<f32x4 *>(&wl[buf * TILE_FLOATS + (lr + 16 * i) * LDS_STRIDE + lc]) = wv[r][i];
    }
  };

  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  const int half = lane >> 5, col = lane & 31;
  const int aoff = (32 * wm + col) * LDS_STRIDE + 32 * half;
  const int woff = (32 * wn + col) * LDS_STRIDE + 32 * half;

  // Tile t is multiplied from LDS buffer t % 2 while tile t + 1 (in
  // register set (t + 1) % 2) is staged into the other buffer and tile t + 3
  // is loaded into the freed registers: loads run two tiles ahead.
  auto iteration = [&](int t, int buf, int r_next) {
    f32x4 xa[8], xw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xa[j] = *reinterpret_cast<const f32x4 *>(&al[buf * TILE_FLOATS + aoff + 4 * j]);
      xw[j] = *reinterpret_cast<const f32x4 *>(&wl[buf * TILE_FLOATS + woff + 4 * j]);
    }
    // unconditional, so the interleaving below sees one basic block: past
    // the last tile the staging fills an unused buffer and the loads repeat
    // the last tile
    stage(r_next, buf ^ 1);
    load(t + 3 < te ? t + 3 : te - 1, r_next);
#pragma unroll
    for (int s = 0; s < 32; ++s)
      acc[s % CHAINS] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[s >> 2][s & 3], xw[s >> 2][s & 3],
                                                             acc[s % CHAINS], 0, 0, 0);
    // interleave: the operand reads first, then per four MFMAs one staging
    // store and one global load
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
    }
    __syncthreads();
  };
  // prologue: the first tile staged, the next two in flight
  load(tb, 0);
  stage(0, 0);
  if (tb + 1 < te) load(tb + 1, 1);
  if (tb + 2 < te) load(tb + 2, 0);
  __syncthreads();
  for (int t = tb; t < te; t += 2) {
    iteration(t, 0, 1);
    if (t + 1 >= te) break;
    iteration(t + 1, 1, 0);
  }
#pragma unroll
  for (int c = 1; c < CHAINS; ++c) acc[0] += acc[c];

  bool misplaced = false;
  if (S > 1) {
    // This split's partial tile, lane-contiguous per accumulator register.
    const size_t tiles = (size_t)g.tiles_m * g.tiles_n;
    float *pp = g.part + ((size_t)split * tiles + tile) * (GM * GN) + wave * 1024 + lane;
#pragma unroll
    for (int r = 0; r < 16; ++r) pp[64 * r] = acc[0][r];
    // every wave's stores acknowledged by the L2 before the arrival
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __shared__ int arrival;
    __syncthreads();
    if (tid == 0) {
      bool mis = false;
      const bool last = arrive_last(g.ctr + tile, S, mis);
      arrival = last ? (mis ? 2 : 1) : 0;
    }
    __syncthreads();
    const int arr = arrival;
    if (arr == 0) return;  // not the last split of this tile
    misplaced = arr == 2;
    // Sum the partials in split order (fixed, whichever split came last),
    // read through the L2 the writers stored to.
    f32x16 sum = f32x16{};
    for (int sp = 0; sp < S; ++sp) {
      const float *q = g.part + ((size_t)sp * tiles + tile) * (GM * GN) + wave * 1024 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += state_load(q + 64 * r);
    }
    acc[0] = sum;
    if (tid == 0) reset_counter(g.ctr + tile);
  }

  // Epilogue: accumulator r holds row 8 (r / 4) + 4 half + r % 4 of the
  // wave's quarter, column col.
  const int n = n0 + 32 * wn + col;
  if (n >= N) return;
  const float b = g.bias ? g.bias[n] : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 32 * wm + 8 * (r >> 2) + 4 * half + (r & 3);
    if (m < M) {
      float v = acc[0][r] + b;
      if (g.act == 1) v = gelu_tanh(v);
      if (g.res) v += g.res[(size_t)m * N + n];
      // splits from more than one XCD (never expected): NaN, not a wrong sum
      g.y[y_index(g, m, n)] = misplaced ? __builtin_nanf("") : v;
    }
  }
}

// Layer norm of each row of x [M][K]: (x - mean) / sqrt(var + eps) * gamma +
// beta, biased variance.  One wave per row, four rows per workgroup; lane j
// holds the 16-byte pieces j, j + 64, ... of the row (K a multiple of 4, at
// most 4096), the mean first, then the variance about it from the registers.
__global__ __launch_bounds__(256) void layernorm_kernel(LayerNormArgs p) {
  constexpr int MAXV = 16;  // 16-byte pieces per lane: K <= 4096
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.M) return;
  const int k4 = p.K / 4;
  const f32x4 *x = reinterpret_cast<const f32x4 *>(p.x + (size_t)row * p.K);
  f32x4 v[MAXV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < k4 ? x[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const float mean = s / (float)p.K;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (lane + 64 * i < k4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[i][e] - mean;
        q = fmaf(d, d, q);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
  const float rstd = 1.f / sqrtf(q / (float)p.K + p.eps);
  const f32x4 *gm = reinterpret_cast<const f32x4 *>(p.g);
  const f32x4 *bt = reinterpret_cast<const f32x4 *>(p.b);
  f32x4 *y = reinterpret_cast<f32x4 *>(p.y + (size_t)row * p.K);
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j < k4) {
      const f32x4 gg = gm[j], bb = bt[j];
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = fmaf((v[i][e] - mean) * rstd, gg[e], bb[e]);
      y[j] = out;
    }
  }
}

}  // namespace

// A K split when the output tiles leave most CUs idle (at most 128 tiles):
// the split count S <= 8 (the last workgroup reads every partial back), at
// least two K tiles per split, that minimises the K tiles the busiest CU
// runs, ceil(T S / 256) ceil(nt / S), plus one tile's worth for the
// reduction when S > 1 (ties: fewer splits).  Measured (fp32, M = 128):
// 3072 -> 768 70 -> 24 us, 768 -> 2304 25 -> 19 us, 768 -> 3072 25 -> 21 us.
// With more tiles the product is bound by the operand traffic of 64 x 64
// tiles, which a split does not reduce (M = 1000, 192 tiles: 3072 -> 768 71
// -> 69 us, 768 -> 768 25.5 -> 33 us at S = 4), so none is taken.
int gemm_splits(int M, int K, int N) {
  const long long T = (long long)((M + GM - 1) / GM) * ((N + GN - 1) / GN);
  const int nt = K / GK;
  if (T > 128 || nt < 4) return 1;
  int best = 1;
  long long best_cost = nt;
  for (int sp = 2; sp <= 8 && sp <= nt / 2; ++sp) {
    const long long cost = (T * sp + 255) / 256 * ((nt + sp - 1) / sp) + 1;
    if (cost < best_cost) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

// Workspace: a fixed block of 256 counters (a split happens only at 128
// tiles or fewer), so that calls of different shapes can share one workspace
// without one call's partials landing on another's counters; then the
// partials.
size_t gemm_workspace_bytes(int M, int K, int N, int splits) {
  (void)K;
  if (splits <= 1) return 0;
  const size_t T = (size_t)((M + GM - 1) / GM) * ((N + GN - 1) / GN);
  return kGemmCounterBytes + (size_t)splits * T * GM * GN * sizeof(float);
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  if (g.splits > 1) {
    const unsigned tiles8 = (unsigned)((g.tiles_m * g.tiles_n + 7) / 8 * 8);
    hipLaunchKernelGGL(gemm_kernel, dim3(tiles8 * (unsigned)g.splits), dim3(256), 0, s, g);
  } else {
    const dim3 grid((unsigned)((g.N + GN - 1) / GN), (unsigned)((g.M + GM - 1) / GM));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(const LayerNormArgs &p, hipStream_t s) {
  hipLaunchKernelGGL(layernorm_kernel, dim3((unsigned)((p.M + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
