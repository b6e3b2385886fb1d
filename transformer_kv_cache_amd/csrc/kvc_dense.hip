// kvc_dense.hip -- the dense layers of a decoder block for the few rows a
// cached decode step carries, fused with their neighbours:
//
//   y[m][n] = act( sum_k xh[m][k] wt[n][k] + bias[n] ) + res[m][n]
//   xh = LN(x) (optional, over each row of x) or x,  act = GELU (tanh) or none
//
// [KV-2] openai-hub.com/news/2435, "千倍计算量为何只换来6倍速度": with the cache a
// decode step runs the projections and the MLP for the new token only, so
// every weight matrix is read once for one (or a few) rows -- a
// matrix-vector product bound by HBM, not by the matrix cores.  The layer
// structure (pre-norm, GELU, residual) is the GPT-2 block the same section
// measures.
//
// Layout: the weight transposed, wt [N][K] (output feature n's K input
// weights contiguous, packed once per model, the layout kvc_gemm_f32 takes
// too); x / y / res row-major [M][K or N], M <= 8 rows, K a multiple of 4.
// As in kvc_gemm_f32, x may come head-major [H][M][K/H] (the attention
// output) and y may go out in the attention layout [3][H][M][N/(3H)] (q, k,
// v of the decode call); with one row both are the row-major layout.
//
// One input row (the usual decode step, K <= 3072): gemv_kernel, below --
// each wave holds all of x across its lanes, so it needs no LDS and no
// barrier (the layer norm's statistics are wave reductions); measured in a
// captured sequence of distinct 768-wide layers, the layer-norm forms drop
// from 5.4-6.3 to 4.3-5.2 us per call (the plain forms 3.8-4.5 -> 3.6-4.4),
// against 2.7 us for a call that reads nothing.
//
// Several rows (linear_kernel), or a longer K:
// one wave per RPW output features, four waves per workgroup.
// A wave reads its RPW rows of wt whole -- each lane 16-byte pieces j,
// j + 64, ... -- so a 768-wide row is three wave-wide 1 KB loads, and every
// load of the call is issued before anything waits: the whole matrix is in
// flight at once across the launch.  Meanwhile the workgroup stages x in
// LDS and, with the layer norm, normalises it there (mean, then the
// variance about it).  Each lane then dots its pieces with the same pieces
// of every x row, the wave sums the partials with lane exchanges, and the
// owning lane adds bias, GELU and residual and stores: one pass over the
// weight, no atomics, a fixed summation order.
//
// Roofline: HBM, K*N*4 bytes of wt per call (plus M*(K+N)*4 for x, y, res).
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
  const float c = 0.7978845608028654f;
  return 0.5f * v * (1.f + tanhf(c * (v + 0.044715f * v * v * v)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// MR: rows the registers are sized for (1, or kMaxLinearRows); RPW output
// features per wave; PPR 16-byte pieces of a row per lane and chunk (a row
// of K floats takes ceil(K / 256) pieces per lane, in chunks of PPR).
template <int MR, int RPW, int PPR>
__global__ __launch_bounds__(256) void linear_kernel(LinearArgs a) {
  extern __shared__ float xs[];  // [M][K] inputs, normalised in place
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = a.M, K = a.K, N = a.N;
  const int k4 = K / 4;
  const int pieces = (k4 + 63) / 64;  // per lane and row
  const int nb = (blockIdx.x * 4 + wave) * RPW;  // this wave's first output

  // 0. Every independent load first: the wave's rows of wt (first chunk),
  //    its bias and residual, x into LDS.
  const f32x4 *wrow[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = nb + r < N ? nb + r : N - 1;
    wrow[r] = reinterpret_cast<const f32x4 *>(a.wt) + (size_t)n * k4;
  }
  f32x4 wv[RPW][PPR];
  auto load_chunk = [&](int p0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int i = 0; i < PPR; ++i) {
        const int q = lane + 64 * (p0 + i);
        wv[r][i] = q < k4 ? wrow[r][q] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  load_chunk(0);
  float b_add[RPW], r_add[RPW][MR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = nb + r;
    b_add[r] = (a.bias && n < N) ? a.bias[n] : 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
      r_add[r][m] = (a.res && m < M && n < N) ? a.res[(size_t)m * N + n] : 0.f;
  }
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(a.x);
  f32x4 *xs4 = reinterpret_cast<f32x4 *>(xs);
  if (a.a_heads > 0) {
    // head-major x: piece q of row m sits in head 4 q / dh, row m of it
    const int dh4 = k4 / a.a_heads;
    for (int i = tid; i < M * k4; i += 256) {
      const int m = i / k4, q = i - m * k4, hh = q / dh4;
      xs4[i] = x4[((size_t)hh * M + m) * dh4 + (q - hh * dh4)];
    }
  } else {
    for (int i = tid; i < M * k4; i += 256) xs4[i] = x4[i];
  }
  __syncthreads();

  // 1. Layer norm of each x row in LDS: the mean, then the biased variance
  //    about it, each summed by all threads and across the waves in LDS.
  if (a.ln_g) {
    __shared__ float red[4][kMaxLinearRows];
    __shared__ float stat[2][kMaxLinearRows];
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < M) {
          const float *row = xs + (size_t)m * K;
          float s = 0.f;
          if (pass == 0) {
            for (int k = tid; k < K; k += 256) s += row[k];
          } else {
            const float mu = stat[0][m];
            for (int k = tid; k < K; k += 256) {
              const float d = row[k] - mu;
              s = fmaf(d, d, s);
            }
          }
          s = wave_sum(s);
          if (lane == 0) red[wave][m] = s;
        }
      }
      __syncthreads();
      if (tid < M) {
        const float s = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
        stat[pass][tid] = pass == 0 ? s / (float)K : 1.f / sqrtf(s / (float)K + a.ln_eps);
      }
      __syncthreads();
    }
    for (int i = tid; i < M * K; i += 256) {
      const int m = i / K, k = i - m * K;
      xs[i] = (xs[i] - stat[0][m]) * stat[1][m] * a.ln_g[k] + a.ln_b[k];
    }
    __syncthreads();
  }

  // 2. Dot products of this lane's pieces, chunk by chunk (one chunk for
  //    K <= 256 PPR).
  float acc[RPW][MR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
  for (int p0 = 0; p0 < pieces; p0 += PPR) {
    if (p0 > 0) load_chunk(p0);
#pragma unroll
    for (int i = 0; i < PPR; ++i) {
      const int q = lane + 64 * (p0 + i);
      if (q < k4) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const f32x4 xv = xs4[(size_t)m * k4 + q];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
              float t = acc[r][m];
              t = fmaf(xv[0], wv[r][i][0], t);
              t = fmaf(xv[1], wv[r][i][1], t);
              t = fmaf(xv[2], wv[r][i][2], t);
              t = fmaf(xv[3], wv[r][i][3], t);
              acc[r][m] = t;
            }
          }
        }
      }
    }
  }

  // 3. Sum over the wave; lane r * MR + m stores output (m, nb + r).
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = nb + r;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        const float v = wave_sum(acc[r][m]);
        if (lane == r * MR + m && n < N) {
          float y = v + b_add[r];
          if (a.act == 1) y = gelu_tanh(y);
          size_t yi = (size_t)m * N + n;
          if (a.y_qkv_heads > 0) {  // [3][H][M][dh]: row (which, head) = n / dh
            const int dh = N / (3 * a.y_qkv_heads), j = n / dh;
            yi = ((size_t)j * M + m) * dh + (n - j * dh);
          }
          a.y[yi] = y + r_add[r][m];
        }
      }
    }
  }
}

// One input row (M = 1, the common decode step), K <= 64 * 4 * NP: every
// wave holds the whole of x across its lanes (lane pieces lane + 64 i, the
// same pieces it takes of each wt row), so the layer norm's statistics are
// two wave reductions and the normalisation happens in registers -- no LDS,
// no barrier, each wave on its own from its first load to its store.  The
// loads of wt, x, bias, residual and the norm's gain / shift are all issued
// before any arithmetic.  Same formulas as linear_kernel (mean, then the
// biased variance about it; (x - mean) * rstd * g + b).
template <int RPW, int NP>
__global__ __launch_bounds__(256) void gemv_kernel(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K, N = a.N;
  const int k4 = K / 4;
  const int nb = (blockIdx.x * 4 + wave) * RPW;  // this wave's first output

  f32x4 wv[RPW][NP];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = nb + r < N ? nb + r : N - 1;
    const f32x4 *row = reinterpret_cast<const f32x4 *>(a.wt) + (size_t)n * k4;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = lane + 64 * i;
      wv[r][i] = q < k4 ? row[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(a.x);
  f32x4 xv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = lane + 64 * i;
    xv[i] = q < k4 ? x4[q] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float b_add[RPW], r_add[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = nb + r;
    b_add[r] = (a.bias && n < N) ? a.bias[n] : 0.f;
    r_add[r] = (a.res && n < N) ? a.res[n] : 0.f;
  }

  if (a.ln_g) {
    const f32x4 *g4 = reinterpret_cast<const f32x4 *>(a.ln_g);
    const f32x4 *s4 = reinterpret_cast<const f32x4 *>(a.ln_b);
    f32x4 gv[NP], sv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = lane + 64 * i;
      gv[i] = q < k4 ? g4[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      sv[i] = q < k4 ? s4[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) sum += (xv[i][0] + xv[i][1]) + (xv[i][2] + xv[i][3]);
    const float mu = wave_sum(sum) / (float)K;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (lane + 64 * i < k4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float d = xv[i][c] - mu;
          ss = fmaf(d, d, ss);
        }
      }
    }
    const float rstd = 1.f / sqrtf(wave_sum(ss) / (float)K + a.ln_eps);
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[i][c] = (xv[i][c] - mu) * rstd * gv[i][c] + sv[i][c];
  }

  // Dots (padding lanes hold zero weights), the wave sum, lane r stores
  // output nb + r.
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      t = fmaf(xv[i][0], wv[r][i][0], t);
      t = fmaf(xv[i][1], wv[r][i][1], t);
      t = fmaf(xv[i][2], wv[r][i][2], t);
      t = fmaf(xv[i][3], wv[r][i][3], t);
    }
    const float v = wave_sum(t);
    const int n = nb + r;
    if (lane == r && n < N) {
      float y = v + b_add[r];
      if (a.act == 1) y = gelu_tanh(y);
      a.y[n] = y + r_add[r];
    }
  }
}

// Input embedding: one workgroup per 1024 features of one token row; ids
// and positions out of range give NaN rows (nothing host-side can see them).
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs e) {
  const int i = blockIdx.y;
  const int d4 = e.d / 4;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= d4) return;
  const int64_t id = e.ids[i];
  const int64_t p = (int64_t)(e.pos ? e.pos[0] : e.pos0) + i;
  f32x4 v;
  if (id < 0 || id >= e.V || p < 0 || p >= e.T) {
    const float nan = __builtin_nanf("");
    v = f32x4{nan, nan, nan, nan};
  } else {
    v = reinterpret_cast<const f32x4 *>(e.wte)[id * d4 + q] + reinterpret_cast<const f32x4 *>(e.wpe)[p * d4 + q];
  }
  reinterpret_cast<f32x4 *>(e.y)[(size_t)i * d4 + q] = v;
}

// Greedy token choice: one workgroup of 1024 lanes scans x in 16-byte pieces
// (eight in flight per lane), keeping the first maximum it meets; lanes, then
// waves, keep the better of two (value, index) pairs -- a NaN beats every
// number, equal values go to the smaller index -- so the result is the first
// maximum whatever the scan order.  A 50257-wide row (200 KB) takes ~9 us in
// a graph, against ~18 us for a framework reduction, with no second pass.
__device__ __forceinline__ bool argmax_better(float v1, int i1, float v2, int i2) {
  const bool n1 = v1 != v1, n2 = v2 != v2;
  if (n1 != n2) return n1;
  if (!n1 && v1 != v2) return v1 > v2;
  return i1 < i2;
}

// Inside one lane indices only grow, so a later element wins only if it is
// the lane's first (bi < 0), larger, or a NaN after numbers.
__device__ __forceinline__ void argmax_take(float v, int i, float &bv, int &bi) {
  const bool take = (bi < 0) | (v > bv) | ((v != v) & (bv == bv));
  bv = take ? v : bv;
  bi = take ? i : bi;
}

__global__ __launch_bounds__(1024) void argmax_kernel(ArgmaxArgs a) {
  const int tid = threadIdx.x;
  float bv = -__builtin_inff();
  int bi = -1;
  const int n4 = a.n / 4;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(a.x);
  constexpr int U = 8;
  for (int q0 = tid; q0 < n4; q0 += 1024 * U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + 1024 * u;
      v[u] = x4[q < n4 ? q : n4 - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + 1024 * u;
      if (q < n4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) argmax_take(v[u][e], 4 * q + e, bv, bi);
      }
    }
  }
  for (int i = 4 * n4 + tid; i < a.n; i += 1024) argmax_take(a.x[i], i, bv, bi);
  if (bi < 0) bi = 0x7fffffff;  // a lane with no element loses every comparison
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (argmax_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (argmax_better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    a.index[0] = bi;
    if (a.seq) {
      const int64_t p = a.seq_pos[0] + 1;
      a.seq_pos[0] = p;
      if (p >= 0 && p < a.cap) a.seq[p] = bi;
    }
  }
}

template <int RPW, int NP>
void launch_gemv(const LinearArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 4 * RPW - 1) / (4 * RPW)));
  hipLaunchKernelGGL((gemv_kernel<RPW, NP>), grid, dim3(256), 0, s, a);
}

template <int MR, int RPW, int PPR>
void launch_shape(const LinearArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 4 * RPW - 1) / (4 * RPW)));
  const size_t lds = (size_t)a.M * a.K * sizeof(float);
  hipLaunchKernelGGL((linear_kernel<MR, RPW, PPR>), grid, dim3(256), lds, s, a);
}

template <int MR>
void launch_rows(const LinearArgs &a, hipStream_t s) {
  // outputs per wave so that a lane holds at most 12 pieces of wt
  const int pieces = (a.K / 4 + 63) / 64;
  if (pieces <= 3) launch_shape<MR, 4, 3>(a, s);
  else if (pieces <= 6) launch_shape<MR, 2, 6>(a, s);
  else launch_shape<MR, 1, 12>(a, s);
}

}  // namespace

hipError_t launch_linear(const LinearArgs &a, hipStream_t s) {
  const int pieces = (a.K / 4 + 63) / 64;
  const bool ln16 = !a.ln_g || ((((uintptr_t)a.ln_g | (uintptr_t)a.ln_b) & 15u) == 0);
  if (a.M == 1 && pieces <= 12 && ln16) {
    // one row: the barrier-free kernel (the norm's gain / shift read as
    // 16-byte pieces, so they must be 16-byte aligned)
    if (pieces <= 3) launch_gemv<4, 3>(a, s);
    else if (pieces <= 6) launch_gemv<2, 6>(a, s);
    else launch_gemv<1, 12>(a, s);
  } else if (a.M == 1) {
    launch_rows<1>(a, s);
  } else {
    launch_rows<kMaxLinearRows>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedArgs &e, hipStream_t s) {
  const dim3 grid((unsigned)((e.d / 4 + 255) / 256), (unsigned)e.N);
  hipLaunchKernelGGL(embed_kernel, grid, dim3(256), 0, s, e);
  return hipGetLastError();
}

}  // namespace kvc
