// Device code of libmoe's combine (gfx950), shared by its own kernel (moe_combine.hip) and the
// single-launch layer kernel (moe_gemm.hip).
//
// X-Stage paper, Introduction, MoE-layer paragraph: Combine sums each token's k expert outputs
// weighted by the router weights: out[t] = bf16(sum over j ascending of w[t,j] * yd[pos[t*k+j]]),
// accumulated in fp32.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
// The combine over items first, first + stride, ... (an item is one (token, column segment)),
// on one wavefront; the kernel below and the single-launch layer kernel deal the items to
// their wavefronts.
template <int KB>
__device__ void combine_items(const int32_t* pos, const float* w, const uint16_t* yd, uint16_t* out, int T, int H,
                              int k, int R, int segs, int first, int stride) {
  const int lane = threadIdx.x & 63;
  const int cpr = H / 8;                   // 16-byte chunks per row
  const int cps = (cpr + segs - 1) / segs;  // chunks per segment
  for (int item = first; item < T * segs; item += stride) {
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

}  // namespace
}  // namespace moe
