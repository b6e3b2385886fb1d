// kvc_append.hip -- slot write of new K/V rows into the preallocated cache.
//
// [KV-1] gitcode.csdn.net/69e62cef0a2f6a37c5a11c4f.html, "Decode Shape 示例":
// the new [1,H,1,D] rows join the cache along the sequence axis.  [KV-4]
// jennyma11.github.io/infra/ch07-01.html, "Decode 阶段": real systems write the
// new rows into their slots in place instead of concatenating.  Here the
// cache is allocated once at Tmax rows and a step writes rows
// [P_b, P_b + N) of each (layer, sequence, KV head): a pure byte copy, so it is
// bit-exact for every element type.  For a paged cache (pools of fixed-size
// blocks and a per-sequence block table) each row goes to its slot, row
// t % block_size of block block_table[b][t / block_size].
//
// Roofline: HBM, 2 x rows x D x elem bytes read and the same written.
#include "kvc_internal.h"

namespace kvc {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, long long total) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    // t enumerates (l, b - b0, h, i, c): c = 16-byte vector within the row.
    long long r = t;
    const int c = (int)(r % a.row_vec16);
    r /= a.row_vec16;
    const int i = (int)(r % a.N);
    r /= a.N;
    const int h = (int)(r % a.Hkv);
    r /= a.Hkv;
    const int bb = (int)(r % a.nb);
    const int l = (int)(r / a.nb);
    const int b = a.b0 + bb;
    const long long src = ((((long long)l * a.B + b) * a.Hkv + h) * a.N + i) * a.row_vec16 + c;
    const int t_pos = a.hist[bb] + i;
    const long long row =
        a.pg.block_table
            ? (long long)paged_row(a.pg, b, t_pos, a.layer0 + l, h, a.Hkv)
            : (((long long)(a.layer0 + l) * a.B + b) * a.Hkv + h) * a.Tmax + t_pos;
    const long long dst = row * a.row_vec16 + c;
    const u32x4 kv = reinterpret_cast<const u32x4 *>(a.k_new)[src];
    const u32x4 vv = reinterpret_cast<const u32x4 *>(a.v_new)[src];
    reinterpret_cast<u32x4 *>(a.k_cache)[dst] = kv;
    reinterpret_cast<u32x4 *>(a.v_cache)[dst] = vv;
  }
}

hipError_t launch_append(const AppendArgs &a, int /*dtype*/, int /*D*/, hipStream_t s) {
  const long long total = (long long)a.n_layers * a.nb * a.Hkv * a.N * a.row_vec16;
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

// hist[b] += n for b < B: the device-side length update of a captured
// decode step (kvc_lengths_add).
__global__ __launch_bounds__(64) void lengths_add_kernel(int32_t *hist, int B, int n) {
  const int b = (int)(blockIdx.x * 64 + threadIdx.x);
  if (b < B) hist[b] += n;
}

hipError_t launch_lengths_add(int32_t *hist, int B, int n, hipStream_t s) {
  hipLaunchKernelGGL(lengths_add_kernel, dim3((unsigned)((B + 63) / 64)), dim3(64), 0, s, hist, B, n);
  return hipGetLastError();
}

}  // namespace kvc
