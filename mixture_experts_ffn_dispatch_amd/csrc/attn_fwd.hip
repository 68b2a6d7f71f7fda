// Attention forward of libmoe (gfx950): full, non-causal softmax(Q K^T / sqrt(d)) V with the
// output tile stored at each tile boundary (X-Stage paper, Section 4.3, FlashAttention-A2A).
//
//  * A persistent grid of 256-thread workgroups (two per CU) walks the (batch, head, 128-query
//    tile) items: workgroup w takes items w, w + G, ...; consecutive items of a head are
//    consecutive query tiles, so the workgroups of one XCD (w mod 8) read the same keys and
//    values through its L2. The two workgroups of a CU synchronise separately, so their phases
//    drift apart and one's softmax overlaps the other's MFMAs on the same SIMDs.
//  * Each wavefront owns 32 queries. Q stays in registers for the whole key loop, as the B
//    operand of v_mfma_f32_32x32x16_bf16: the scores are computed transposed, S^T = K Q^T, so
//    a lane holds one query's scores for 32 of the tile's 64 keys (its half of the wavefront
//    the other 32): the online softmax is lane-local plus one exchange between the halves.
//  * The output is accumulated transposed too, O^T = V^T P^T, so all 64 accumulators of a lane
//    belong to its query: the softmax rescale and the final division are lane-local. The
//    lane's own P values are the B operand as they are: the key order of each 16-deep step is
//    permuted to match the score layout ({4h..4h+3, 8+4h..8+4h+3} for lane half h), and V^T
//    is read in the same order.
//  * Keys go from global memory straight into LDS (buffer->LDS loads), 16-byte chunks XOR-
//    swizzled by row so that the 16-byte operand reads of 32 rows are free of conflicts;
//    values go through registers and are written transposed ([d][key], rows padded to 136
//    bytes: the 8-byte operand reads of 32 d-rows hit distinct banks). Both double buffered.
//  * Scores and the softmax in fp32 (exp2 of the scores scaled by log2(e) / sqrt(d)), P rounded
//    to bf16 for the second product, fp32 accumulation, O rounded to bf16 at the end of the
//    tile and stored with the log-sum-exp of each query.
#include <math.h>

#include <type_traits>

#include "attn.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAD = 128;       // head dimension
constexpr int kAWaves = ATTN_TILE_QUERIES / 32;  // wavefronts per workgroup, 32 queries each
constexpr int kABM = 32 * kAWaves;  // queries per tile
constexpr int kABN = 64;       // keys per step of the key loop
constexpr int kAThreads = 64 * kAWaves;
constexpr int kAPerCU = ATTN_WORKGROUPS_PER_CU;  // workgroups per CU (their phases drift apart: one's softmax
                               // overlaps the other's MFMAs)
constexpr int kVtStride = kABN + 4;  // bf16 per transposed value row (136 bytes)
constexpr float kLazy = 8.0f;        // log2 headroom of the lazy running maximum
constexpr unsigned kRsrcWord3 = 0x00020000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voffset, 0, 0, 0);
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int M;
  int qtiles;       // query tiles per (batch, head)
  int items;        // (batch, head) pairs x qtiles
  float scale_log2; // log2(e) / sqrt(d)
};

__global__ __launch_bounds__(kAThreads, kAPerCU) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kABN * kAD];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kAD * kVtStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ql = lane & 31;
  const int M = a.M;
  const int nkv = (M + kABN - 1) / kABN;
  const uint32_t head_bytes = (uint32_t)M * (uint32_t)(kAD * 2);
  // staging assignments: key rows (direct to LDS; a wavefront loads 4 rows of 256 bytes per
  // instruction) and value rows (through registers: one key row, VD consecutive d's)
  constexpr int KI = kABN / 4 / kAWaves;  // key-load instructions per wavefront
  constexpr int VD = kAD * kABN / kAThreads;  // d's of a value row per thread
  const int krow0 = wave * 4 * KI + (lane >> 4);  // + 4 i
  const int kslot = lane & 15;
  const int vkey = tid & 63, vd0 = (tid >> 6) * VD;

  for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int bh = item / a.qtiles, qt = item - bh * a.qtiles;
    const size_t hoff = (size_t)bh * M * kAD;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + hoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + hoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + hoff, head_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + hoff, head_bytes);
    const int qrow = qt * kABM + wave * 32 + ql;  // this lane's query (past M: reads zero, no store)

    // Q as the B operand: d-step s holds Q[q][16 s + 8 hf + 0..7]
    bf16x8 qf[kAD / 16];
#pragma unroll
    for (int s = 0; s < kAD / 16; ++s) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)qrow * (kAD * 2) + (16 * s + 8 * hf) * 2, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
    f32x16 oacc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
    // running maximum (log2 units) and sum; the first block always raises the maximum (its
    // eager sum against -1e30 is infinite). A finite start keeps every value NaN-free (masked
    // keys are -inf, and -inf - (-1e30) is -inf), which lets this file be compiled without
    // NaN semantics (-fno-honor-nans): the maxima then need no canonicalising instructions.
    float m_run = -1.0e30f, l_run = 0.f;

    auto issue_k = [&](int t, int st) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int row = krow0 + 4 * i;
        const uint32_t chunk = (uint32_t)(kslot ^ (row & 15));
        load_lds16(rk, &s_k[st][(wave * 4 * KI + 4 * i) * kAD], (uint32_t)(t * kABN + row) * (kAD * 2) + chunk * 16);
      }
    };
    auto load_v = [&](int t, u32x4 (&vr)[VD / 8]) {
      const uint32_t off = (uint32_t)(t * kABN + vkey) * (kAD * 2) + vd0 * 2;
#pragma unroll
      for (int j = 0; j < VD / 8; ++j) vr[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, off + 16 * j, 0, 0);
    };
    auto store_vt = [&](int st, const u32x4 (&vr)[VD / 8]) {
      uint16_t* dst = &s_vt[st][vd0 * kVtStride + vkey];
#pragma unroll
      for (int j = 0; j < VD / 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[(8 * j + 2 * e) * kVtStride] = (uint16_t)(vr[j][e] & 0xFFFFu);
          dst[(8 * j + 2 * e + 1) * kVtStride] = (uint16_t)(vr[j][e] >> 16);
        }
    };

    // prologue: key tile 0 into stage 0
    u32x4 vr[VD / 8];
    issue_k(0, 0);
    load_v(0, vr);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_vt(0, vr);
    __syncthreads();

    // one step of the key loop; RAGGED (a compile-time switch) masks the keys past M, which
    // only the last step of a ragged sequence holds, so the other steps carry no branch
    // inside their scheduling regions
    auto key_step = [&](int t, auto ragged_tag) {
      constexpr bool RAGGED = decltype(ragged_tag)::value;
      const int st = t & 1;
      const bool more = t + 1 < nkv;
      if (more) {  // the next tile lands in the other stage meanwhile
        issue_k(t + 1, st ^ 1);
        load_v(t + 1, vr);
      }
      // One step of 64 keys in four scheduling regions, so that each block's softmax issues
      // among the other block's MFMAs (the two are independent):
      //   1. K fragments of block 0; block 0's score MFMAs with block 1's fragment reads
      //   2. block 1's score MFMAs with block 0's maximum, exponentials and sum, and the V^T
      //      fragments of block 0
      //   3. block 0's P V MFMAs with block 1's softmax and the V^T fragments of block 1
      //   4. block 1's P V MFMAs with the transposed value writes for the next step
      // The O rescale (skipped while no query of the wavefront has a new maximum) sits
      // between regions. S^T = K Q^T; O^T += V^T P^T with, for d-block c and key step u of
      // block b, V^T[32 c + ql][32 b + 16 u + {4 hf..4 hf+3, 8+4 hf..8+4 hf+3}].
      auto read_kf = [&](int b, bf16x8 (&kf)[kAD / 16]) {
        const int r = 32 * b + ql;
#pragma unroll
        for (int s = 0; s < kAD / 16; ++s)
          kf[s] = *reinterpret_cast<const bf16x8*>(&s_k[st][r * kAD + (((2 * s + hf) ^ (r & 15)) * 8)]);
      };
      auto read_vf = [&](int b, bf16x8 (&vf)[2][4]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint16_t* row = &s_vt[st][(32 * c + ql) * kVtStride + 32 * b + 16 * u + 4 * hf];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8);
            vf[u][c] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
          }
      };
      auto scores = [&](const bf16x8 (&kf)[kAD / 16], f32x16& acc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < kAD / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
      };
      // keys past M (key of value (b, i): 64 t + 32 b + 8 (i / 4) + 4 hf + i % 4)
      auto mask = [&](int b, f32x16& acc) {
        if constexpr (RAGGED) {
          const int kbase = t * kABN + 32 * b + 4 * hf;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kbase + 8 * (i >> 2) + (i & 3) >= M) acc[i] = -INFINITY;
        }
      };
      // Softmax of one block with a lazy maximum: the probabilities exp2(fma(s, c, -m)) (c =
      // log2(e) / sqrt(d)) are formed against the running maximum m before the block's own
      // maximum is known, so they do not wait for its cross-lane reduction. O / l does not
      // depend on m; m only keeps the exponentials in range, and it is raised (O and l
      // rescaled, the block's probabilities formed again) only when a query's block maximum
      // exceeds it by more than kLazy (log2 units, so every probability stays below
      // 2^kLazy), which after the first tile is rare. The maximum is taken on the raw
      // scores (the scale is positive).
      auto probs = [&](const f32x16& acc, bf16x8 (&pf)[2], float m) -> float {
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], a.scale_log2, -m));
          lsum += p;
          pf[i >> 3][i & 7] = (__bf16)p;
        }
        return lsum;
      };
      auto block_max = [&](const f32x16& acc) -> float {
        float mt = fmaxf(acc[0], acc[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mt = fmaxf(mt, fmaxf(acc[i], acc[i + 1]));
        return fmaxf(mt, __shfl_xor(mt, 32)) * a.scale_log2;
      };
      // settles the block after its eager probabilities: raises the maximum if it must, or if
      // the eager sum is not finite (the first block, against the starting maximum of -1e30);
      // testing the sum also keeps the eager exponentials ahead of the branch
      auto settle = [&](const f32x16& acc, bf16x8 (&pf)[2], float mt, float lsum) {
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy || !(lsum <= 3.0e38f))) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
          l_run *= alpha;
          m_run = m_new;
          lsum = probs(acc, pf, m_new);
        }
        l_run += lsum;
      };
      auto pv = [&](const bf16x8 (&vf)[2][4], const bf16x8 (&pf)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][c], pf[u], oacc[c], 0, 0, 0);
      };

      f32x16 s0, s1;
      bf16x8 kf0[kAD / 16], kf1[kAD / 16], vf0[2][4], vf1[2][4], p0[2], p1[2];
      // region 1
      __builtin_amdgcn_sched_barrier(0);
      read_kf(0, kf0);
      read_kf(1, kf1);
      scores(kf0, s0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // block 0's fragments
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA of block 0
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a fragment of block 1
      }
      __builtin_amdgcn_sched_barrier(0);
      // region 2
      mask(0, s0);
      __builtin_amdgcn_sched_barrier(0);
      scores(kf1, s1);
      mask(1, s1);
      float lsum0 = probs(s0, p0, m_run);
      const float mt0 = block_max(s0);
      read_vf(0, vf0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA of block 1's scores
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // block 0's softmax
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // V^T fragments of block 0
      }
      __builtin_amdgcn_sched_barrier(0);
      settle(s0, p0, mt0, lsum0);
      // region 3
      __builtin_amdgcn_sched_barrier(0);
      pv(vf0, p0);
      float lsum1 = probs(s1, p1, m_run);
      const float mt1 = block_max(s1);
      read_vf(1, vf1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA of block 0's P V
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // block 1's softmax
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // V^T fragments of block 1
      }
      __builtin_amdgcn_sched_barrier(0);
      settle(s1, p1, mt1, lsum1);
      // region 4
      __builtin_amdgcn_sched_barrier(0);
      pv(vf1, p1);
      if (more) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        store_vt(st ^ 1, vr);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    const bool ragged = (M & (kABN - 1)) != 0;
    for (int t = 0; t < nkv - (ragged ? 1 : 0); ++t) key_step(t, std::false_type{});
    if (ragged) key_step(nkv - 1, std::true_type{});

    // the tile boundary: O = O^T / l for this lane's query, stored 4 d's (8 bytes) at a time
    const float l_all = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_all;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(oacc[c][4 * g + j] * inv);
        const int d0 = 32 * c + 8 * g + 4 * hf;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ov), ro,
                                              (uint32_t)qrow * (kAD * 2) + d0 * 2, 0, 0);
      }
    if (a.lse && hf == 0 && qrow < M)
      a.lse[(size_t)bh * M + qrow] = (m_run + __log2f(l_all)) * 0.69314718055994530942f;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status attn_forward(const attn_config* c, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, void* stream) {
  if (!c || !q || !k || !v || !o) return MOE_ERR_INVALID_ARG;
  if (c->B < 1 || c->heads < 1 || c->M < 1 || c->d < 1 || c->num_workgroups < 0) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (c->reserved[i] != 0) return MOE_ERR_INVALID_ARG;
  if (c->d != ATTN_HEAD_DIM) return MOE_ERR_UNSUPPORTED;
  // one head's [M, d] block is addressed by 32-bit buffer offsets
  if ((long long)c->M * kAD * 2 >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  const long long qtiles = ((long long)c->M + kABM - 1) / kABM;
  const long long items = (long long)c->B * c->heads * qtiles;
  if (items >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_kernel, kAThreads, 0) != hipSuccess)
    return MOE_ERR_HIP;
  const long long slots = (long long)cus * (per_cu > 0 ? per_cu : 1);
  long long grid = c->num_workgroups > 0 && c->num_workgroups < slots ? c->num_workgroups : slots;
  if (grid > items) grid = items;
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.M = c->M;
  a.qtiles = (int)qtiles;
  a.items = (int)items;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)c->d));
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(kAThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
