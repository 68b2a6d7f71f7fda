// Data-movement kernels of libmoe (gfx950): the dispatch gather and the router-weighted
// combine.
//
// X-Stage paper, Introduction, MoE-layer paragraph: Dispatch sends every token's copy to its
// expert's rows, and Combine sums each token's k expert outputs weighted by the router.
//
//   dispatch  a wavefront per token: reads its row of x once and writes it to the k
//             dispatched rows pos[t*k + j] (the persistent GEMM can instead gather these rows
//             itself, in its Linear-1 loads).
//   combine   a wavefront per (token, column segment): out[t] = bf16(sum over j ascending of
//             w[t,j] * yd[pos[t*k + j]]), accumulated in fp32.
#include "moe_combine_dev.h"

namespace moe {
namespace {

// Dispatch, token-major: a wavefront reads token t's row once and writes it to the k
// dispatched rows pos[t*k + j] (the same bytes as gathering xd[r] = x[perm[r] / k]).
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* pos, const uint16_t* x, uint16_t* xd,
                                                       int T, int H, int k) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = H / 8;  // 16-byte chunks per row
  const int R = T * k;
  for (int t = blockIdx.x * 4 + wave; t < T; t += gridDim.x * 4) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
    const int32_t* pt = pos + (size_t)t * k;
    for (int c = lane; c < cpr; c += 128) {
      const bool two = c + 64 < cpr;
      const u32x4 v0 = src[c];
      const u32x4 v1 = two ? src[c + 64] : v0;
      for (int j = 0; j < k; ++j) {
        const int r = pt[j];
        if ((unsigned)r >= (unsigned)R) continue;
        u32x4* dst = reinterpret_cast<u32x4*>(xd + (size_t)r * H);
        dst[c] = v0;
        if (two) dst[c + 64] = v1;
      }
    }
  }
}

template <int KB>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* pos, const float* w,
                                                      const uint16_t* yd, uint16_t* out, int T,
                                                      int H, int k, int R, int segs) {
  combine_items<KB>(pos, w, yd, out, T, H, k, R, segs, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

inline int grid_rows(long long rows_per_block_units) {
  long long g = rows_per_block_units;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

}  // namespace

hipError_t launch_dispatch(const int32_t* pos, const uint16_t* x, uint16_t* xd, int T, int H, int k,
                           hipStream_t s) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(grid_rows((T + 3) / 4)), dim3(256), 0, s, pos, x, xd, T, H, k);
  return hipGetLastError();
}

hipError_t launch_combine(const int32_t* pos, const float* w, const uint16_t* yd, uint16_t* out, int T,
                          int H, int k, hipStream_t s) {
  const int segs = combine_segments(T, H);
  hipLaunchKernelGGL(combine_kernel<8>, dim3(grid_rows(((long long)T * segs + 3) / 4)), dim3(256), 0, s, pos, w, yd,
                     out, T, H, k, T * k, segs);
  return hipGetLastError();
}

}  // namespace moe
