// kvc_decode_mfma.hip -- split-K decode for several query rows per KV head on
// the matrix cores.
//
// Same computation as kvc_decode.hip ([KV-4] jennyma11.github.io/infra/ch07-01.html,
// "Decode 阶段", listing 1-2; [KV-2] openai-hub.com/news/2435, "一个很容易漏掉的错误":
// row i of N new rows sees keys 0 .. P+i), for the case where a KV head
// serves R = G * N > 1 query rows -- GQA groups and chunked decode.  Then
// every K/V row meets R query rows and the work per byte is R times larger;
// on the vector ALUs each (key, row) pair needs its own cross-lane dot-product
// reduction, which made that path compute-bound.  Here the R rows (padded to
// a tile of 16) and a block of 16 keys form small dense products:
//   S^T = K . Q^T   v_mfma_f32_16x16x4_f32 (fp32) / v_mfma_f32_16x16x32_bf16
//                   (bf16); the K operand is exactly what each lane's
//                   16-byte global load brings in, so K never touches LDS
//   O^T += V^T P^T  v_mfma_f32_16x16x4_f32 for both element types (bf16 V is
//                   widened exactly; probabilities stay fp32); V goes through
//                   the wave's own slice of LDS to change lane ownership
// A lane owns one query row (column of S^T) and four keys of each block, so
// the softmax needs only two cross-lane exchanges per block.  A workgroup (4
// waves) covers 16 query rows and a split of 4 x KPW keys; the per-row softmax
// states of the waves merge in LDS and then follow the same path as the
// vector kernel: the output directly, or (max, sum, partial output) into the
// workspace for the split-combine kernel.  Calls with 2-8 fp32 rows of
// D = 64 or 2-8 bf16 rows of D = 128 or 64 run on the multi-row vector kernel
// (kvc_decode_rows.hip) instead, which streams faster.  In the fused step keys [P, P+N)
// are read straight from k_new / v_new, and the workgroups of row tile 0 that
// hold them write them to their cache slots (no workgroup reads those slots
// during the call).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// K/V loads: plain (non-temporal loads measured no faster here).
__device__ __forceinline__ u32x4 stream_load(const u32x4 *p) { return *p; }

// Which 16-byte vector of a key row lane group g loads as its j-th: the
// contraction over d may run in any order as long as the K and Q operands
// agree; vector 4 j + g, so a wave instruction covers the same quarter of 16
// rows (each lane reading one contiguous run instead measured no faster).
template <int J>
__device__ __forceinline__ int vec_index(int j, int g) {
  return 4 * j + g;
}

// KPW keys per wave (a multiple of 16), RM = 16 query rows per workgroup.
template <int DT, int D, int KPW, bool FUSED, bool PAGED, bool DEVLEN>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int EB = Dtype<DT>::kBytes;
  constexpr int EV = Dtype<DT>::kPer16B;   // elements per 16-byte vector
  constexpr int LPR = D * EB / 16;         // 16-byte vectors per key row
  constexpr int NB = KPW / 16;             // 16-key blocks per wave
  constexpr int SPLIT = 4 * KPW;
  // Per lane and block: J 16-byte vectors of the key row.  fp32: vector j
  // holds d = 16 j + 4 g .. +3; bf16: d = 32 j + 8 g .. +7 (g = lane / 16).
  constexpr int J = LPR / 4;
  constexpr int VS = D + 4;                // fp32 elements per V row in LDS
  static_assert(KPW % 16 == 0 && LPR % 4 == 0, "layout");

  __shared__ float sv[4][16 * VS];         // per wave: V block, later its output rows
  __shared__ float sm_m[4][16], sm_l[4][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;  // key (K/V loads, S^T rows) or query row (S^T columns)
  const int g = lane >> 4;

  const int split = blockIdx.x;
  const int bb = blockIdx.z;
  const int P = seq_hist<DEVLEN>(a, bb);
  const int rt = blockIdx.y % a.row_tiles;
  const int lh = blockIdx.y / a.row_tiles;
  const int l = div_magic(lh, a.Hkv, a.hkv_div);
  const int hkv = lh - l * a.Hkv;
  const int b = a.b0 + bb;
  const int nkeys = P + a.N;
  const int nsplit = (nkeys + SPLIT - 1) / SPLIT;
  if (split >= nsplit) return;

  const size_t crow0 = (((size_t)(a.layer0 + l) * a.B + b) * a.Hkv + hkv) * (size_t)a.Tmax;
  const u32x4 *kc = reinterpret_cast<const u32x4 *>(a.k_cache) + crow0 * LPR;
  const u32x4 *vc = reinterpret_cast<const u32x4 *>(a.v_cache) + crow0 * LPR;
  const size_t nrow0 = (((size_t)l * a.B + b) * a.Hkv + hkv) * (size_t)a.N * LPR;
  const u32x4 *kn = FUSED ? reinterpret_cast<const u32x4 *>(a.k_new) + nrow0 : nullptr;
  const u32x4 *vn = FUSED ? reinterpret_cast<const u32x4 *>(a.v_new) + nrow0 : nullptr;

  // Query row of this lane's S^T column: rr = g_head * N + i within the unit.
  const long long qrow0 = (((long long)l * a.B + b) * a.Hq + (long long)hkv * a.group) * a.N;
  const int rr = rt * 16 + c16;
  const bool row_ok = rr < a.rows;
  const int lim = row_ok ? P + rr % a.N : nkeys - 1;  // last visible key of this row

  // Issue every load up front: Q^T fragments, then K and V of each block.
  u32x4 qw[J];
  {
    const u32x4 *qp = reinterpret_cast<const u32x4 *>(a.q) + (qrow0 + (row_ok ? rr : a.rows - 1)) * LPR;
#pragma unroll
    for (int j = 0; j < J; ++j) qw[j] = qp[vec_index<J>(j, g)];
  }
  const int keyw = split * SPLIT + wave * KPW;  // first key of this wave
  u32x4 kw[NB][J], vw[NB][J];
  // Paged cache: each key's row index in the pools, looked up through the
  // block table (all lookups issued before any K/V load).
  size_t prow[NB];
  if constexpr (PAGED) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int key = keyw + 16 * nb + c16;
      prow[nb] = paged_row(a.pg, b, key < nkeys ? key : nkeys - 1, a.layer0 + l, hkv, a.Hkv);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int key = keyw + 16 * nb + c16;
    const int kidx = key < nkeys ? key : nkeys - 1;
    const bool fresh = FUSED && kidx >= P;
    const size_t nidx = (size_t)(fresh ? kidx - P : 0);
    const size_t crow = PAGED ? prow[nb] : (size_t)kidx;  // row within the K/V base below
    const u32x4 *kbase = PAGED ? reinterpret_cast<const u32x4 *>(a.k_cache) : kc;
    const u32x4 *vbase = PAGED ? reinterpret_cast<const u32x4 *>(a.v_cache) : vc;
    const u32x4 *kp = fresh ? kn + nidx * LPR : kbase + crow * LPR;
    const u32x4 *vp = fresh ? vn + nidx * LPR : vbase + crow * LPR;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      kw[nb][j] = stream_load(kp + vec_index<J>(j, g));
      vw[nb][j] = stream_load(vp + vec_index<J>(j, g));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Fused step: row tile 0 writes the new rows it read from k_new / v_new.
  if constexpr (FUSED) {
    if (rt == 0) {
      u32x4 *kd = reinterpret_cast<u32x4 *>(a.k_cache) + (PAGED ? 0 : crow0 * LPR);
      u32x4 *vd = reinterpret_cast<u32x4 *>(a.v_cache) + (PAGED ? 0 : crow0 * LPR);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int key = keyw + 16 * nb + c16;
        if (key >= P && key < nkeys) {
          const size_t drow = PAGED ? prow[nb] : (size_t)key;
#pragma unroll
          for (int j = 0; j < J; ++j) {
            kd[drow * LPR + vec_index<J>(j, g)] = kw[nb][j];
            vd[drow * LPR + vec_index<J>(j, g)] = vw[nb][j];
          }
        }
      }
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float *my_v = sv[wave];

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // S^T block: acc_s[i] = score of key keyw + 16 nb + 4 g + i for row rr.
    f32x4 acc_s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if constexpr (DT == KVC_BF16) {
        acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[nb][j]),
                                                        __builtin_bit_cast(bf16x8, qw[j]), acc_s, 0, 0, 0);
      } else {
        const f32x4 kf = __builtin_bit_cast(f32x4, kw[nb][j]);
        const f32x4 qf = __builtin_bit_cast(f32x4, qw[j]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc_s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], qf[t], acc_s, 0, 0, 0);
      }
    }
    // V block into this wave's LDS slice as fp32 rows (exact widening).  The
    // slice belongs to this wave alone; wave barriers keep the compiler from
    // moving its LDS accesses across the write/read hand-over between lanes.
    __builtin_amdgcn_wave_barrier();
    {
      float *row = my_v + c16 * VS;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float vf[EV];
        unpack16<DT>(vw[nb][j], vf);
        const int d0 = vec_index<J>(j, g) * EV;
#pragma unroll
        for (int e = 0; e < EV; e += 4)
          *reinterpret_cast<f32x4 *>(row + d0 + e) = f32x4{vf[e], vf[e + 1], vf[e + 2], vf[e + 3]};
      }
    }
    __builtin_amdgcn_wave_barrier();
    // Mask, scale, online softmax for this lane's row.
    const int kb0 = keyw + 16 * nb + 4 * g;
    float s[4];
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (kb0 + i <= lim) ? acc_s[i] * a.scale_log2 : kNegInf;
      mt = fmaxf(mt, s[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = rescale(m_run, m_new);
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = (m_new == kNegInf) ? 0.f : fast_exp2(s[i] - m_new);
      ps += p[i];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc_o[db] *= alpha;
    // O^T[d][row] += sum over the block's keys: A = V^T (LDS), B = P^T (registers).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float *vrow = my_v + (4 * g + i) * VS + c16;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], p[i], acc_o[db], 0, 0, 0);
    }
  }

  // Row sums over the wave (the four lanes g of a row hold disjoint keys).
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // This wave's state into LDS: output rows O[row][d] with d = 16 db + 4 g + i.
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<f32x4 *>(my_v + c16 * VS + 16 * db + 4 * g) = acc_o[db];
  if (g == 0) {
    sm_m[wave][c16] = m_run;
    sm_l[wave][c16] = l_run;
  }
  __syncthreads();

  // Merge the four waves; thread t handles (row, d) pairs.
  for (int t = tid; t < 16 * D; t += 256) {
    const int r = t / D;
    const int d = t % D;
    if (rt * 16 + r >= a.rows) continue;
    float M = sm_m[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][r]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = rescale(sm_m[w][r], M);
      o = fmaf(f, sv[w][r * VS + d], o);
      L = fmaf(f, sm_l[w][r], L);
    }
    const long long row = qrow0 + rt * 16 + r;
    if (nsplit == 1) {
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

template <int DT, int D, int KPW>
hipError_t launch_kpw(const DecodeArgs &a, int splits, bool fused, hipStream_t s) {
  const dim3 grid((unsigned)splits, (unsigned)(a.n_layers * a.Hkv * a.row_tiles), (unsigned)a.nb);
  const bool paged = a.pg.block_table != nullptr;
  if (a.hist_dev) {
    // device lengths: the fused step only
    if (!fused) return hipErrorInvalidValue;
    if (paged)
      hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, true, true, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, true, false, true>), grid, dim3(256), 0, s, a);
  } else if (fused && paged)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, true, true, false>), grid, dim3(256), 0, s, a);
  else if (fused)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, true, false, false>), grid, dim3(256), 0, s, a);
  else if (paged)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, false, true, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, KPW, false, false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Keys per wave: 32 for 256-byte rows (fp32 D = 64, bf16 D = 128), twice
// that for 128-byte rows and half for 512-byte rows, so that a workgroup
// always streams the same bytes (16 and 64 keys per wave measured worse for
// the GQA workload).
constexpr int kKpw = 32;
constexpr int kKpwSmall = kKpw >= 32 ? kKpw / 2 : 16;

int decode_mfma_split_keys(int dtype, int D) {
  const int row_bytes = D * (dtype == KVC_BF16 ? 2 : 4);
  return 4 * (row_bytes == 128 ? 2 * kKpw : row_bytes == 512 ? kKpwSmall : kKpw);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int D, int splits, bool fused,
                              hipStream_t s) {
  if (dtype == KVC_F32) {
    if (D == 64) return launch_kpw<KVC_F32, 64, kKpw>(a, splits, fused, s);
    return launch_kpw<KVC_F32, 128, kKpwSmall>(a, splits, fused, s);
  }
  if (D == 64) return launch_kpw<KVC_BF16, 64, 2 * kKpw>(a, splits, fused, s);
  return launch_kpw<KVC_BF16, 128, kKpw>(a, splits, fused, s);
}

}  // namespace kvc
