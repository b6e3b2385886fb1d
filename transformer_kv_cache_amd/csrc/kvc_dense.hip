// kvc_dense.hip -- the dense layers of a decoder block for the few rows a
// cached decode step carries, fused with their neighbours:
//
//   y[m][n] = act( sum_k xh[m][k] W[k][n] + bias[n] ) + res[m][n]
//   xh = LN(x) (optional, over each row of x) or x,  act = GELU (tanh) or none
//
// [KV-2] openai-hub.com/news/2435, "千倍计算量为何只换来6倍速度": with the cache a
// decode step runs the projections and the MLP for the new token only, so
// every weight matrix is read once for one (or a few) rows -- a
// matrix-vector product bound by HBM, not by the matrix cores.  The layer
// structure (pre-norm, GELU, residual) is the GPT-2 block the same section
// measures.
//
// Layout: W row-major [K][N] (input feature k, output feature n), x / y / res
// row-major [M][N or K], M <= 8 rows, K and N multiples of 4.
//
// Work split: a workgroup owns CPW output columns and all K inputs.  Its NT
// threads are CT = CPW/4 column threads (4 columns = one 16-byte load of a W
// row) times KG = NT/CT k-groups; k-group g takes rows g, g+KG, ...  A wave
// instruction therefore reads 64/CT consecutive W rows, CPW*4 contiguous
// bytes of each.  x (after the layer norm) sits in LDS and is read as a
// broadcast.  Partial sums are combined across the k-groups of a wave with
// lane exchanges and across the waves in LDS; the owning thread adds
// the bias, applies the activation and the residual and stores.  One pass,
// no atomics, a fixed summation order.  A single-row call uses 1024-thread
// workgroups: with only N / CPW workgroups (48 for a 768-wide layer), each
// must keep many W rows in flight to stream at HBM rate.
//
// Roofline: HBM, K*N*4 bytes of W per call (plus M*(K+N)*4 for x, y, res).
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
  const float c = 0.7978845608028654f;
  return 0.5f * v * (1.f + tanhf(c * (v + 0.044715f * v * v * v)));
}

// MR: rows the registers are sized for (1, or kMaxLinearRows); NT threads.
template <int CPW, int MR, int NT>
__global__ __launch_bounds__(NT) void linear_kernel(LinearArgs a) {
  constexpr int CT = CPW / 4;    // column threads
  constexpr int KG = NT / CT;    // k-groups
  constexpr int NW = NT / 64;    // waves
  extern __shared__ float xs[];  // [M][K] inputs (normalised) + LN params, then [NW][M][CPW] partials
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ct = tid % CT;
  const int kg = tid / CT;
  const int M = a.M, K = a.K, N = a.N;
  constexpr int U = 4;                        // W rows in flight per thread per batch
  constexpr int EP = (MR * CPW + NT - 1) / NT;  // epilogue outputs per thread

  // 0. Every load that does not depend on another is issued first, so the
  //    call pays one memory round trip before its arithmetic: this thread's
  //    first U rows of W, its epilogue's bias and residual, x and the
  //    layer-norm parameters.
  const int n0 = blockIdx.x * CPW + ct * 4;
  const bool col_ok = n0 < N;
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(a.w) + (col_ok ? n0 / 4 : 0);
  const int n4 = N / 4;  // 16-byte vectors per W row
  f32x4 wv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = kg + u * KG;
    wv[u] = (col_ok && k < K) ? w4[(size_t)k * n4] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float e_add[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const int t = tid + e * NT;
    const int m = t / CPW, n = blockIdx.x * CPW + t % CPW;
    float v = 0.f;
    if (m < M && n < N) {
      if (a.bias) v += a.bias[n];
      if (a.res && a.act == 0) v += a.res[(size_t)m * N + n];
    }
    e_add[e] = v;
  }
  float e_res[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const int t = tid + e * NT;
    const int m = t / CPW, n = blockIdx.x * CPW + t % CPW;
    e_res[e] = (a.res && a.act != 0 && m < M && n < N) ? a.res[(size_t)m * N + n] : 0.f;
  }
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(a.x);
  f32x4 *xs4 = reinterpret_cast<f32x4 *>(xs);
  float *lng = xs + (size_t)M * K, *lnb = lng + K;  // layer-norm parameters after x
  const bool ln = a.ln_g != nullptr;
  for (int i = tid; i < M * K / 4; i += NT) xs4[i] = x4[i];
  if (ln) {
    for (int i = tid; i < K / 4; i += NT) {
      reinterpret_cast<f32x4 *>(lng)[i] = reinterpret_cast<const f32x4 *>(a.ln_g)[i];
      reinterpret_cast<f32x4 *>(lnb)[i] = reinterpret_cast<const f32x4 *>(a.ln_b)[i];
    }
  }
  __syncthreads();

  // 1. Layer-norm statistics of each row in one pass over it, shifted by its
  //    first element against cancellation: with y = x - x[0],
  //    mean = x[0] + E[y] and var = E[y^2] - E[y]^2 (biased).  All threads
  //    share the work; the waves' partial sums meet in LDS.
  __shared__ float red[2][NW][kMaxLinearRows];
  float mean[MR], rstd[MR];
  if (ln) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        const float *row = xs + (size_t)m * K;
        const float x0 = row[0];
        float s1 = 0.f, s2 = 0.f;
        for (int k = tid; k < K; k += NT) {
          const float y = row[k] - x0;
          s1 += y;
          s2 += y * y;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          s1 += __shfl_xor(s1, o);
          s2 += __shfl_xor(s2, o);
        }
        if (lane == 0) {
          red[0][wave][m] = s1;
          red[1][wave][m] = s2;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          s1 += red[0][w][m];
          s2 += red[1][w][m];
        }
        const float ey = s1 / (float)K;
        const float var = fmaxf(s2 / (float)K - ey * ey, 0.f);
        mean[m] = xs[(size_t)m * K] + ey;
        rstd[m] = 1.f / sqrtf(var + a.ln_eps);
      }
    }
  }
  // Input feature k of row m as the product sees it.
  auto xin = [&](int m, int k) -> float {
    const float v = xs[(size_t)m * K + k];
    return ln ? (v - mean[m]) * rstd[m] * lng[k] + lnb[k] : v;
  };

  // 2. Partial sums over this k-group's rows, U rows per batch, the next
  //    batch's loads issued before this batch's arithmetic.
  f32x4 acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kg;; k += U * KG) {
    f32x4 nx[U];
    const bool more = k + U * KG < K;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + (U + u) * KG;
        nx[u] = (col_ok && kk < K) ? w4[(size_t)kk * n4] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + u * KG;
      if (kk < K) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
          if (m < M) acc[m] += xin(m, kk) * wv[u];
      }
    }
    if (!more) break;
#pragma unroll
    for (int u = 0; u < U; ++u) wv[u] = nx[u];
  }

  // 3. Sum over the k-groups of the wave (lanes ct, ct + CT, ...), then over
  //    the waves in LDS (the x rows are no longer read).
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < M) {
#pragma unroll
      for (int o = CT; o < 64; o <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] += __shfl_xor(acc[m][c], o);
      }
    }
  }
  __syncthreads();
  float *part = xs;  // [NW][M][CPW]
  if (lane < CT) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M)
        *reinterpret_cast<f32x4 *>(part + ((size_t)wave * M + m) * CPW + ct * 4) = acc[m];
  }
  __syncthreads();

  // 4. Epilogue: bias, activation, residual (operands already in registers).
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const int t = tid + e * NT;
    const int m = t / CPW;
    const int c = t % CPW;
    const int n = blockIdx.x * CPW + c;
    if (m >= M || n >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += part[((size_t)w * M + m) * CPW + c];
    v += e_add[e];
    if (a.act == 1) v = gelu_tanh(v);
    a.y[(size_t)m * N + n] = v + e_res[e];
  }
}

// Columns per workgroup: wide enough to stream whole cache lines of each W
// row, narrow enough to give the launch at least 64 workgroups.
int linear_columns_per_workgroup(int N) {
  if (N / 64 >= 128) return 64;
  if (N / 32 >= 64) return 32;
  return 16;
}

size_t linear_lds_bytes(int M, int K, bool ln, int cpw, int waves) {
  const size_t xb = ((size_t)M * K + (ln ? 2 * (size_t)K : 0)) * sizeof(float);
  const size_t pb = (size_t)waves * M * cpw * sizeof(float);
  return xb > pb ? xb : pb;
}

template <int MR, int NT>
void launch_rows(const LinearArgs &a, hipStream_t s) {
  const int cpw = linear_columns_per_workgroup(a.N);
  const dim3 grid((unsigned)((a.N + cpw - 1) / cpw));
  const size_t lds = linear_lds_bytes(a.M, a.K, a.ln_g != nullptr, cpw, NT / 64);
  if (cpw == 64)
    hipLaunchKernelGGL((linear_kernel<64, MR, NT>), grid, dim3(NT), lds, s, a);
  else if (cpw == 32)
    hipLaunchKernelGGL((linear_kernel<32, MR, NT>), grid, dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((linear_kernel<16, MR, NT>), grid, dim3(NT), lds, s, a);
}

}  // namespace

hipError_t launch_linear(const LinearArgs &a, hipStream_t s) {
  if (a.M == 1)
    launch_rows<1, 1024>(a, s);
  else
    launch_rows<kMaxLinearRows, 256>(a, s);
  return hipGetLastError();
}

}  // namespace kvc
