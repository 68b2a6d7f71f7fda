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
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

__device__ inline float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(unsigned v) { return __uint_as_float(v & 0xffff0000u); }
__device__ inline unsigned pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (unsigned)__builtin_bit_cast(unsigned short, a) |
         ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}

// Combine: a wavefront per (token, column segment); a token's row is cut into `segs` segments
// when there are too few tokens to fill the GPU. Slot j's row and weight are held by lane j
// (k <= 64) and broadcast with readlane; each lane takes two 16-byte chunks of the row per
// step and issues the loads of up to KB slots before any is accumulated, so their latencies
// overlap. Every Yd row is read exactly once, so the loads are non-temporal. The sum runs over
// j in ascending order for every element.
template <int KB>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* pos, const float* w,
                                                      const uint16_t* yd, uint16_t* out, int T,
                                                      int H, int k, int R, int segs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = H / 8;                   // 16-byte chunks per row
  const int cps = (cpr + segs - 1) / segs;  // chunks per segment
  for (int item = blockIdx.x * 4 + wave; item < T * segs; item += gridDim.x * 4) {
    const int t = item / segs, c_lo = (item % segs) * cps, c_hi = min(cpr, c_lo + cps);
    int rv = 0;
    float wv = 0.f;
    if (lane < k) {
      rv = pos[(size_t)t * k + lane];
      wv = w[(size_t)t * k + lane];
      if ((unsigned)rv >= (unsigned)R) {  // never for a plan written by moe_plan
        rv = 0;
        wv = 0.f;
      }
    }
    for (int c = c_lo + lane; c < c_hi; c += 128) {
      const bool two = c + 64 < c_hi;
      float a0[8], a1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a0[i] = a1[i] = 0.f;
      for (int j0 = 0; j0 < k; j0 += KB) {
        u32x4 v0[KB], v1[KB];
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
          if (j0 + jj < k) {
            const int r = __builtin_amdgcn_readlane(rv, j0 + jj);
            const u32x4* src = reinterpret_cast<const u32x4*>(yd + (size_t)r * H);
            v0[jj] = __builtin_nontemporal_load(src + c);
            if (two) v1[jj] = __builtin_nontemporal_load(src + c + 64);
          }
        }
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
          if (j0 + jj < k) {
            const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), j0 + jj));
            const u32x4 x = v0[jj];
            a0[0] = fmaf(wj, bf16_lo(x.x), a0[0]);
            a0[1] = fmaf(wj, bf16_hi(x.x), a0[1]);
            a0[2] = fmaf(wj, bf16_lo(x.y), a0[2]);
            a0[3] = fmaf(wj, bf16_hi(x.y), a0[3]);
            a0[4] = fmaf(wj, bf16_lo(x.z), a0[4]);
            a0[5] = fmaf(wj, bf16_hi(x.z), a0[5]);
            a0[6] = fmaf(wj, bf16_lo(x.w), a0[6]);
            a0[7] = fmaf(wj, bf16_hi(x.w), a0[7]);
            if (two) {
              const u32x4 y = v1[jj];
              a1[0] = fmaf(wj, bf16_lo(y.x), a1[0]);
              a1[1] = fmaf(wj, bf16_hi(y.x), a1[1]);
              a1[2] = fmaf(wj, bf16_lo(y.y), a1[2]);
              a1[3] = fmaf(wj, bf16_hi(y.y), a1[3]);
              a1[4] = fmaf(wj, bf16_lo(y.z), a1[4]);
              a1[5] = fmaf(wj, bf16_hi(y.z), a1[5]);
              a1[6] = fmaf(wj, bf16_lo(y.w), a1[6]);
              a1[7] = fmaf(wj, bf16_hi(y.w), a1[7]);
            }
          }
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)t * H);
      u32x4 o;
      o.x = pack_bf16(a0[0], a0[1]);
      o.y = pack_bf16(a0[2], a0[3]);
      o.z = pack_bf16(a0[4], a0[5]);
      o.w = pack_bf16(a0[6], a0[7]);
      dst[c] = o;
      if (two) {
        o.x = pack_bf16(a1[0], a1[1]);
        o.y = pack_bf16(a1[2], a1[3]);
        o.z = pack_bf16(a1[4], a1[5]);
        o.w = pack_bf16(a1[6], a1[7]);
        dst[c + 64] = o;
      }
    }
  }
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
  // with few tokens, cut rows into up to 4 segments of at least 128 chunks (one step of a
  // wavefront) so that about 4096 wavefronts run
  const int cpr = H / 8;
  int segs = (4096 + T - 1) / T;
  segs = segs < 1 ? 1 : segs > 4 ? 4 : segs;
  while (segs > 1 && cpr / segs < 128) --segs;
  hipLaunchKernelGGL(combine_kernel<8>, dim3(grid_rows(((long long)T * segs + 3) / 4)), dim3(256), 0, s, pos, w, yd,
                     out, T, H, k, T * k, segs);
  return hipGetLastError();
}

}  // namespace moe
