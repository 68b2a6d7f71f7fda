// Device code of libmoe's planner (gfx950), shared by its own kernels (moe_plan.hip, 1024-thread
// workgroups) and the single-launch layer kernel (moe_gemm.hip, the GEMM's workgroups): routing
// of a token chunk, the one-workgroup scan and schedule step, the scatter of a token chunk and
// the tile placement, each templated on the workgroup size NT. The steps and their sources on
// the page are described in moe_plan.hip.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {


// Order-preserving key of a logit: a larger float gives a larger key and -0, +0 give the same
// key (IEEE comparison), so equal keys are equal logits. Every key of a logit is above 0,
// which marks a slot that is taken or holds no expert. NaN is not a valid logit and is read
// as -inf, so selection stays in range.
__device__ inline unsigned logit_key(float x) {
  unsigned u = __float_as_uint(x != x ? -INFINITY : x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_logit(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// max(x, x of the lane that the DPP pattern CTRL names); the patterns used here stay inside
// a row of 16 lanes and name an active lane
template <int CTRL>
__device__ inline unsigned dpp_max(unsigned x) {
  return max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false));
}

// Maximum over every aligned group of S lanes, in each lane of the group (all lanes active).
// Inside a row: quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors; the
// rows of a 32- or 64-lane group are combined through readlane.
template <int S>
__device__ inline unsigned group_max(unsigned x) {
  if (S >= 2) x = dpp_max<0xB1>(x);
  if (S >= 4) x = dpp_max<0x4E>(x);
  if (S >= 8) x = dpp_max<0x141>(x);
  if (S >= 16) x = dpp_max<0x140>(x);
  if (S >= 32) {
    const unsigned r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
    const unsigned r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
    if (S == 32) x = (threadIdx.x & 32) ? max(r2, r3) : max(r0, r1);
    else x = max(max(r0, r1), max(r2, r3));
  }
  return x;
}

constexpr int kPlanThreads = 1024;  // 16 wavefronts per block in the planner's own kernels
constexpr int kPlaceBlocks = 256;   // blocks that place the tile list

// Top-k selection, one round per kept slot: the largest key among the candidates (descending
// logit) is found with group_max, and of the lanes holding it the lowest expert id wins (ties
// go to the lower id): in route_hist the first 64-expert block with a match, and in it the
// lowest lane, found with a ballot.
// One token chunk of a workgroup of NT threads; cnt is an LDS array of E ints.
template <int R, int NT>  // logits held per lane: experts lane, lane + 64, ..., E <= 64 * R
__device__ void route_hist_chunk(const PlanArgs& a, int chunk, int* cnt) {
  constexpr int kPlanWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < a.E; e += NT) cnt[e] = 0;
  __syncthreads();

  const int t_end = min(a.T, (chunk + 1) * a.chunk_tokens);
  for (int t = chunk * a.chunk_tokens + wave; t < t_end; t += kPlanWaves) {
    const float* row = a.logits + (size_t)t * a.E;
    unsigned key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = lane + 64 * r;
      key[r] = e < a.E ? logit_key(row[e]) : 0u;
    }
    float my_v = 0.f, top = 0.f;
    int my_e = 0;
    for (int j = 0; j < a.k; ++j) {
      unsigned lm = 0u;
#pragma unroll
      for (int r = 0; r < R; ++r) lm = max(lm, key[r]);
      const unsigned m = group_max<64>(lm);  // > 0: k <= E leaves a candidate every round
      int be = -1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const unsigned long long b = __ballot(key[r] == m);
        if (b) {
          be = 64 * r + __ffsll((long long)b) - 1;
          break;
        }
      }
      if (lane == (be & 63)) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r == (be >> 6)) key[r] = 0u;
      }
      if (lane == j) {
        my_v = key_logit(m);
        my_e = be;
      }
      if (j == 0) top = key_logit(m);
    }
    // softmax restricted to the kept logits; the full denominator cancels
    const float ex = lane < a.k ? expf(my_v - top) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);  // same on every lane
    if (lane < a.k) {
      const size_t f = (size_t)t * a.k + lane;
      a.topk_ids[f] = my_e;
      a.topk_w[f] = ex / sum;
      atomicAdd(&cnt[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += NT) a.chunk_counts[(size_t)e * a.cstride + chunk] = cnt[e];
  __syncthreads();  // cnt may be reused by the next chunk
}

// Routing for E <= 64: one token per S-lane segment of a wavefront (S = a power of two >= E),
// so 64 / S tokens are routed at once. Same selection and weights as route_hist_kernel; the
// maxima and the weight sums stay inside a segment.
template <int S, int NT>
__device__ void route_small_chunk(const PlanArgs& a, int chunk, int* cnt) {
  constexpr int kPlanWaves = NT / 64;
  constexpr int TPW = 64 / S;  // tokens per wavefront step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane / S, sl = lane % S;
  for (int e = tid; e < a.E; e += NT) cnt[e] = 0;
  __syncthreads();
  const int t_end = min(a.T, (chunk + 1) * a.chunk_tokens);
  for (int t0 = chunk * a.chunk_tokens + wave * TPW; t0 < t_end; t0 += kPlanWaves * TPW) {
    const int t = t0 + seg;
    const bool live = t < t_end;
    unsigned key = live && sl < a.E ? logit_key(a.logits[(size_t)t * a.E + sl]) : 0u;
    float my_v = 0.f, top = 0.f;
    int my_e = 0;
    for (int j = 0; j < a.k; ++j) {
      const unsigned m = group_max<S>(key);  // 0 only in a segment past the chunk's end
      unsigned long long b = __ballot(key == m && key != 0u);
      if (S < 64) b = (b >> (seg * S)) & ((1ull << (S & 63)) - 1ull);
      const int be = b ? __ffsll((long long)b) - 1 : -1;
      if (be == sl) key = 0u;
      if (sl == j) {
        my_v = key_logit(m);
        my_e = be;
      }
      if (j == 0) top = key_logit(m);
    }
    const float ex = sl < a.k ? expf(my_v - top) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = S / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (live && sl < a.k) {
      const size_t f = (size_t)t * a.k + sl;
      a.topk_ids[f] = my_e;
      a.topk_w[f] = ex / sum;
      atomicAdd(&cnt[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += NT) a.chunk_counts[(size_t)e * a.cstride + chunk] = cnt[e];
  __syncthreads();  // cnt may be reused by the next chunk
}

// One token chunk routed by the kernel shape that suits E (as the planner's launcher picks).
template <int NT>
__device__ void route_chunk(const PlanArgs& a, int chunk, int* cnt) {
  const int R = (a.E + 63) / 64;
  if (a.E <= 8) route_small_chunk<8, NT>(a, chunk, cnt);
  else if (a.E <= 16) route_small_chunk<16, NT>(a, chunk, cnt);
  else if (a.E <= 32) route_small_chunk<32, NT>(a, chunk, cnt);
  else if (R <= 1) route_small_chunk<64, NT>(a, chunk, cnt);
  else if (R <= 2) route_hist_chunk<2, NT>(a, chunk, cnt);
  else if (R <= 4) route_hist_chunk<4, NT>(a, chunk, cnt);
  else if (R <= 8) route_hist_chunk<8, NT>(a, chunk, cnt);
  else route_hist_chunk<16, NT>(a, chunk, cnt);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline int units_of(int tiles) { return (tiles + kUnit - 1) / kUnit; }

// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active), in DPP: row
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then lane 15 of rows 0 and 2 added into
// rows 1 and 3 (row_bcast15) and lane 31 into rows 2 and 3 (row_bcast31). Lanes whose source
// lies outside the row, or rows outside the row mask, add 0.
__device__ inline int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Exclusive scan of one int per thread over an NT-thread workgroup; `total` gets the sum.
// Every wavefront scans the NT / 64 wavefront totals itself, so one barrier publishes them.
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  const int w = wave_inclusive_scan(lane < NT / 64 ? s_tmp[lane] : 0);
  const int base = wave ? __builtin_amdgcn_readlane(w, wave - 1) : 0;
  total = __builtin_amdgcn_readlane(w, NT / 64 - 1);
  __syncthreads();  // s_tmp may be reused by the next call
  return base + x - v;
}

// Minimum over each wavefront (all lanes active): the mirror patterns of group_max, then the
// four row minima through readlane.
__device__ inline int wave_min(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Minimum of one int per thread over an NT-thread workgroup (the same value on every thread).
template <int NT>
__device__ int block_min(int v, int* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_min(v);
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  const int w = wave_min(lane < NT / 64 ? s_tmp[lane] : 0x7fffffff);
  __syncthreads();  // s_tmp may be reused by the next call
  return w;
}

// The wave table: what the tile placement (step 4, in scatter_kernel) needs from the schedule
// builder, written to the workspace by scan_schedule_kernel. A head of kWaveTableHead ints
// (the scalars below and the group offsets), then eight arrays of nw + 1 entries indexed by
// expert wave, then the first m-block of each expert (E + 1 entries, the last = all m-blocks)
// and the expert offsets (E + 1 entries, the last = T k).
enum : int { kWtLead = 0, kWtL1Units = 1, kWtL2Units = 2, kWtUnits = 3, kWtInterleaved = 4, kWtGoff = 8 };
static_assert(kWtGoff + kGroups + 1 <= kWaveTableHead, "wave table head");
struct WaveTable {
  int* head;
  int* a;    // Linear-1 tiles of each wave
  int* b;    // Linear-2 tiles of each wave
  int* p1;   // Linear-1 units of all earlier waves
  int* p2;   // Linear-2 units of all earlier waves
  int* l1s;  // list position of each wave's Linear-1 run
  int* l2s;  // list position of each wave's Linear-2 run
  int* l1u;  // unit index of each wave's first Linear-1 unit
  int* l2u;  // unit index of each wave's first Linear-2 unit
  int* mb;   // first m-block of each expert
  int* off;  // first dispatched row of each expert
  __device__ WaveTable(int* t, int nw, int E) : head(t) {
    int* p = t + kWaveTableHead;
    a = p;
    b = a + nw + 1;
    p1 = b + nw + 1;
    p2 = p1 + nw + 1;
    l1s = p2 + nw + 1;
    l2s = l1s + nw + 1;
    l1u = l2s + nw + 1;
    l2u = l1u + nw + 1;
    mb = l2u + nw + 1;
    off = mb + E + 1;
  }
};
__device__ inline int wave_table_len(int nw, int E) { return kWaveTableHead + 8 * (nw + 1) + 2 * (E + 1); }
// LDS ints that hold the largest wave table
constexpr int kWaveTableLds = kWaveTableHead + 10 * (MOE_MAX_EXPERTS + 1);

// Scans and minima for step 3: over wavefront 0 alone (ONE, at most 64 expert waves; no
// barriers), else over the whole workgroup.
template <bool ONE, int NT>
__device__ inline int step_scan(int v, int* s_tmp, int& total) {
  if constexpr (ONE) {
    const int x = wave_inclusive_scan(v);
    total = __builtin_amdgcn_readlane(x, 63);
    return x - v;
  } else {
    return block_exclusive_scan<NT>(v, s_tmp, total);
  }
}
template <bool ONE, int NT>
__device__ inline int step_min(int v, int* s_tmp) {
  if constexpr (ONE) return wave_min(v);
  else return block_min<NT>(v, s_tmp);
}
// Publishes LDS writes of the wave-table step to the other lanes (ONE: the lanes of
// wavefront 0 exchange values through LDS, e.g. lane i writes a[i] and lane i - D reads it).
// The fences order the LDS accesses at wavefront scope, so the compiler may not move a later
// load of another lane's entry above this lane's store, and the wave barrier keeps the
// scheduler from moving code across.
template <bool ONE>
__device__ inline void step_sync() {
  if constexpr (ONE) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// The MOE_SCHED_AUTO rule (include/moe.h) prices each candidate order: D = 0 is the
// Expert-Wave order, D >= 1 the interleaved order with lead D. Its model of the GEMM's tile
// main loops and bursts, and the dependency-distance test (as for lead 0 above).
struct AutoModel {
  double t1, t2, vt, R, T0, Q;
  long long den, need;
  __device__ AutoModel(const PlanArgs& a, long long A, long long B) {
#pragma clang fp contract(off)
    const double G = (double)a.grid, BM = (double)a.tile_m;
    t1 = G * fmax(2.0 * BM * 256.0 * (double)a.H / kAutoMfmaFlops, 512.0 * (double)a.H / kAutoStreamBytes);
    t2 = G * fmax(2.0 * BM * 256.0 * (double)a.I / kAutoMfmaFlops, 512.0 * (double)a.I / kAutoStreamBytes);
    vt = BM * 256.0 * 2.0;
    R = a.xs_drain_bps;
    T0 = a.xs_issue_s;
    Q = a.xs_capacity_b;
    den = A * a.H + B * a.I;
    need = (long long)a.grid * a.H * (A + B);
  }
};

// Wave i's share of candidate D's price: the X-Stage stall of its Linear-2 bursts (>= 0),
// returned with the sign bit set when its Linear-2 tiles can be reached before its Linear-1
// tiles are done (a dependency stall of half a Linear-1 tile); +0 for a wave with no
// Linear-2 tiles. The same double-precision steps as the rule's statement, without fused
// multiply-adds, so a host model can reproduce the choice exactly.
__device__ double auto_term(const PlanArgs& a, const WaveTable& t, const AutoModel& m, int nw, int D, int i) {
#pragma clang fp contract(off)
  const int b = t.b[i];
  if (b == 0) return 0.0;
  // the producers whose Linear-2 boundaries align: those on Linear-2 tiles at a time, the
  // Linear-2 share of the segment's work when Linear-1 tiles of wave i + D are spread in it
  const int an = (D > 0 && i + D < nw) ? t.a[i + D] : 0;
  const double share = ((double)b * m.t2) / ((double)b * m.t2 + (double)an * m.t1);
  const double kact = fmax(1.0, (double)min(a.grid, b) * share);
  const double V = kact * m.vt;
  const double g = m.t2;
  double T = fmax(m.T0, V / m.R - g);
  if (V - m.R * m.T0 > m.Q) T = fmax(T, (V - m.Q) / m.R);
  const double xs = ((double)b / kact) * (T - m.T0);
  bool reach = true;
  if (D > 0) {
    const long long dist =
        (long long)t.p2[i] - t.p2[max(0, i - D + 1)] + t.p1[min(i + D, nw)] - t.p1[min(i + 1, nw)];
    reach = dist * m.den < m.need;
  }
  return reach ? -xs : xs;
}

// Candidate D's price from its waves' terms (term(i) gives wave i's auto_term), summed in
// wave order, plus the locality cost when the GEMM is HBM-bound: the activation bytes live
// while a wave's Linear-2 tiles run (waves i .. i + D) beyond the last-level cache.
template <class Term>
__device__ double auto_price(const PlanArgs& a, const WaveTable& t, const AutoModel& m, int nw, int D,
                             bool hbm_bound, Term term) {
#pragma clang fp contract(off)
  double xs = 0.0, dep = 0.0, over = 0.0;
  for (int i = 0; i < nw; ++i) {
    const int last = D > 0 ? min(i + D, nw - 1) : i;
    const double ws = (double)(t.off[min(a.E, (last + 1) * a.W)] - t.off[i * a.W]) * (double)a.I * 2.0;
    over = fmax(over, ws - kAutoCacheBytes);
    const double v = term(i);
    xs += fabs(v);
    if (__double_as_longlong(v) < 0) dep += m.t1 / 2.0;
  }
  return xs + dep + (hbm_bound ? over / kAutoStreamBytes : 0.0);
}
// Candidates of up to this many expert waves are priced with one lane per (lead, wave) term,
// held in the (nw + 1) x nw doubles of s_cost, and one lane per lead summing them.
constexpr int kAutoPairWaves = 31;
static_assert((kAutoPairWaves + 1) * kAutoPairWaves <= MOE_MAX_EXPERTS, "s_cost holds the terms");

// 3. tile counts per expert wave and where each wave's runs start in the list. A run (one
//    wave's Linear-1 or Linear-2 tiles) is cut into units of kUnit consecutive tiles (the
//    last unit may be shorter); the orders are defined on units, so every unit is one
//    contiguous stretch of the list holding tiles of a single run. Thread i handles wave i.
// ONE: on wavefront 0 alone (at most 64 expert waves); else on all NT threads (nw <= NT).
template <bool ONE, int NT>
__device__ void schedule_waves(const PlanArgs& a, const WaveTable& t, int nw, int* s_tmp, double* s_cost) {
  const int tid = threadIdx.x, E = a.E, W = a.W;
  bool interleaved = a.schedule == MOE_SCHED_INTERLEAVED;
  const bool automatic = a.schedule == MOE_SCHED_AUTO;
  int aw = 0, bw = 0;
  if (tid < nw) {
    const int m = t.mb[min(E, (tid + 1) * W)] - t.mb[tid * W];
    aw = m * a.n1;
    bw = m * a.n2;
    t.a[tid] = aw;
    t.b[tid] = bw;
  }
  step_sync<ONE>();
  // Lead 0 picks D from the tile counts. A Linear-2 tile of wave i must not be taken before
  // the last Linear-1 tile of wave i has finished. With `grid` tiles in flight, list
  // positions are taken at about grid per mean tile duration, so a Linear-1 tile finishes
  // about grid * t1 / t_mean positions after it was taken (t1, t_mean: Linear-1 and mean
  // tile durations, proportional to K = H for Linear-1 and I for Linear-2). In the interleaved
  // list the last Linear-1 tile of wave i ends segment i - D (or the lead prefix) and Linear-2
  // of wave i starts segment i, so with a_j, b_j the Linear-1 / Linear-2 tiles of wave j and
  // PA, PB their prefix sums the tiles between them number
  //   dist_i(D) = PB[i] - PB[max(0, i - D + 1)] + PA[min(i + D, nw)] - PA[min(i + 1, nw)].
  // D is the smallest lead with dist_i(D) * (A H + B I) >= grid * H * (A + B) for every wave
  // with Linear-2 tiles (A, B: all Linear-1 / Linear-2 tiles), else nw. The prefix sums use
  // p1 / p2, which hold unit prefix sums only after the lead is known.
  int D = a.lead;
  {
    int A, B;
    const int pa = step_scan<ONE, NT>(aw, s_tmp, A);
    const int pb = step_scan<ONE, NT>(bw, s_tmp, B);
    if ((interleaved && D == 0) || automatic) {
      if (tid < nw) {
        t.p1[tid] = pa;
        t.p2[tid] = pb;
      }
      if (tid == 0) {
        t.p1[nw] = A;
        t.p2[nw] = B;
      }
      step_sync<ONE>();
      if (!automatic) {
        const long long den = (long long)A * a.H + (long long)B * a.I;
        const long long need = (long long)a.grid * a.H * (A + B);
        int cand = nw;  // thread t tests lead t + 1
        if (tid < nw) {
          const int Dc = tid + 1;
          bool ok = true;
          for (int i = 0; i < nw && ok; ++i) {
            if (t.b[i] == 0) continue;
            const long long dist = (long long)t.p2[i] - t.p2[max(0, i - Dc + 1)] + t.p1[min(i + Dc, nw)] -
                                   t.p1[min(i + 1, nw)];
            ok = dist * den >= need;
          }
          if (ok) cand = Dc;
        }
        D = step_min<ONE, NT>(cand, s_tmp);
      }
    }
    if (automatic) {
      // MOE_SCHED_AUTO: every candidate is priced and all threads read all prices, so all
      // take the same choice
      constexpr int kStride = ONE ? 64 : NT;
      int act = 0;
      for (int e = tid; e < E; e += kStride) act += t.off[e + 1] > t.off[e] ? 1 : 0;
      int active;
      (void)step_scan<ONE, NT>(act, s_tmp, active);
      const long long rows = t.off[E];
      const double flops = 6.0 * (double)rows * (double)a.H * (double)a.I;
      const double bytes = (double)rows * (double)a.H * 4.0 + (double)active * 6.0 * (double)a.H * (double)a.I +
                           (double)rows * (double)a.I * 4.0;
      const bool hbm_bound = bytes / kAutoStreamBytes > flops / kAutoMfmaFlops;
      const AutoModel m(a, A, B);
      double ew;
      if (ONE && nw <= kAutoPairWaves) {
        // s_cost[D * nw + i] = wave i's term of candidate D (D = 0 .. nw); then lane D sums its
        // row and the prices go to s_cost[D - 1] (lead D) and s_cost[nw] (Expert-Wave)
        for (int p = tid; p < (nw + 1) * nw; p += kStride) s_cost[p] = auto_term(a, t, m, nw, p / nw, p % nw);
        step_sync<ONE>();
        double price = 0.0;
        if (tid <= nw)
          price = auto_price(a, t, m, nw, tid, hbm_bound, [&](int i) { return s_cost[tid * nw + i]; });
        step_sync<ONE>();
        if (tid <= nw) s_cost[tid == 0 ? nw : tid - 1] = price;
        step_sync<ONE>();
        ew = s_cost[nw];
      } else {
        // thread t prices the interleaved order with lead t + 1, every thread the Expert-Wave one
        if (tid < nw)
          s_cost[tid] = auto_price(a, t, m, nw, tid + 1, hbm_bound,
                                   [&](int i) { return auto_term(a, t, m, nw, tid + 1, i); });
        ew = auto_price(a, t, m, nw, 0, hbm_bound, [&](int i) { return auto_term(a, t, m, nw, 0, i); });
        step_sync<ONE>();
      }
      double best = s_cost[0];
      int bestD = 1;
      for (int d = 1; d < nw; ++d)
        if (s_cost[d] <= best) {  // ties go to the larger lead
          best = s_cost[d];
          bestD = d + 1;
        }
      interleaved = !(ew < best);  // ties go to the interleaved order
      D = bestD;
    }
    D = min(max(D, 1), max(nw, 1));
  }
  const int auw = units_of(aw), buw = units_of(bw);
  int n_l1_units, n_l2_units;
  {
    const int p1 = step_scan<ONE, NT>(tid < nw ? auw : 0, s_tmp, n_l1_units);
    const int p2 = step_scan<ONE, NT>(tid < nw ? buw : 0, s_tmp, n_l2_units);
    if (tid < nw) {
      t.p1[tid] = p1;
      t.p2[tid] = p2;
    }
    if (tid == 0) {
      t.p1[nw] = n_l1_units;
      t.p2[nw] = n_l2_units;
    }
  }
  int total_units;
  if (!interleaved) {
    // Expert-Wave order: L1(0) L2(0) L1(1) L2(1) ...
    int unused;
    const int st = step_scan<ONE, NT>(aw + bw, s_tmp, unused);
    const int su = step_scan<ONE, NT>(auw + buw, s_tmp, total_units);
    if (tid < nw) {
      t.l1s[tid] = st;
      t.l2s[tid] = st + aw;
      t.l1u[tid] = su;
      t.l2u[tid] = su + auw;
    }
  } else {
    // interleaved: L1(0) .. L1(D-1), then segment i = L2(i) merged with L1(i + D)
    int prefix_total, prefix_units, unused, seg_units;
    const bool lead = tid < min(D, nw);
    step_sync<ONE>();  // t.a of every wave (written above) is read across lanes below
    const int p = step_scan<ONE, NT>(lead ? aw : 0, s_tmp, prefix_total);
    const int pu = step_scan<ONE, NT>(lead ? auw : 0, s_tmp, prefix_units);
    const int a_next = tid + D < nw ? t.a[tid + D] : 0;
    const int seg = tid < nw ? bw + a_next : 0;
    const int segu = tid < nw ? buw + units_of(a_next) : 0;
    const int q = prefix_total + step_scan<ONE, NT>(seg, s_tmp, unused);
    const int qu = prefix_units + step_scan<ONE, NT>(segu, s_tmp, seg_units);
    total_units = prefix_units + seg_units;
    if (tid < nw) {
      t.l2s[tid] = q;  // segment tid starts with L2(tid)
      t.l2u[tid] = qu;
      if (tid < D) {  // lead prefix
        t.l1s[tid] = p;
        t.l1u[tid] = pu;
      }
      if (tid + D < nw) {  // L1(tid + D) lives in segment tid
        t.l1s[tid + D] = q;
        t.l1u[tid + D] = qu;
      }
    }
  }
  // first entry of each locality group's unit list (group g gets units g, g + G, ... of each
  // phase)
  if (tid <= kGroups) {
    int goff = 0;
    for (int h = 0; h < tid; ++h)
      goff += (n_l1_units - h + kGroups - 1) / kGroups + (n_l2_units - h + kGroups - 1) / kGroups;
    t.head[kWtGoff + tid] = goff;
  }
  if (tid == 0) {
    t.head[kWtLead] = D;
    t.head[kWtInterleaved] = interleaved ? 1 : 0;
    t.head[kWtL1Units] = n_l1_units;
    t.head[kWtL2Units] = n_l2_units;
    t.head[kWtUnits] = total_units;
  }
}

// The schedule step on one NT-thread workgroup. LDS: s_tmp[32], s_cnt[MOE_MAX_EXPERTS] (rows
// routed to each expert), s_tab[kWaveTableLds] (the wave table), s_cost[MOE_MAX_EXPERTS]
// (MOE_SCHED_AUTO: the prices of the candidate orders and their per-wave terms). With more than 64 expert waves it needs
// nw <= NT (the host checks).
template <int NT>
__device__ void scan_schedule_block(const PlanArgs& a, int* s_tmp, int* s_cnt, int* s_tab, double* s_cost) {
  const int tid = threadIdx.x;
  const int E = a.E, BM = a.tile_m;
  const int nw = (E + a.W - 1) / a.W;
  const WaveTable t(s_tab, nw, E);
  int* const s_off = t.off;  // expert offsets
  // the table's unused slots (in the head, past the last wave) are written out with the rest:
  // zero, so a plan's bytes are fixed
  for (int i = tid; i < wave_table_len(nw, E); i += NT) s_tab[i] = 0;
  // 1. per-expert exclusive scans of the (expert, chunk) count table, in place: entry (e, c)
  //    becomes the first row of chunk c's slots among expert e's rows (the scatter adds the
  //    expert's offset), and the row total is the expert's count. Wavefront w owns rows
  //    w, w + 16, ...; each row is cut into segments of 256 entries (4 consecutive per lane,
  //    one 16-byte access each way; rows are padded to a multiple of 4 entries, the padding
  //    reads as zero), with a shuffle scan across the lanes. A wavefront loads up to 8
  //    segments before scanning them, so their load latencies overlap.
  {
    constexpr int SEG = 256, BATCH = 8, NW = NT / 64;
    const int lane = tid & 63, wave = tid >> 6;
    const int segs_row = (a.chunks + SEG - 1) / SEG;
    const int rows_w = wave < E ? (E - wave + NW - 1) / NW : 0;
    const int nseg = rows_w * segs_row;
    int run = 0;
    for (int s0 = 0; s0 < nseg; s0 += BATCH) {
      int v[BATCH][4];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int sg = s0 + b;
        const int e = wave + NW * (sg / segs_row), i0 = (sg % segs_row) * SEG + lane * 4;
        i32x4 q = {0, 0, 0, 0};
        if (sg < nseg && i0 < a.cstride) q = *reinterpret_cast<const i32x4*>(a.chunk_counts + (size_t)e * a.cstride + i0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[b][i] = i0 + i < a.chunks ? q[i] : 0;
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int sg = s0 + b;
        if (sg >= nseg) break;
        const int e = wave + NW * (sg / segs_row), c0 = (sg % segs_row) * SEG, i0 = c0 + lane * 4;
        if (c0 == 0) run = 0;
        const int sum = v[b][0] + v[b][1] + v[b][2] + v[b][3];
        const int x = wave_inclusive_scan(sum);
        int r = run + x - sum;  // exclusive prefix of this lane's first entry
        i32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[i] = r;
          r += v[b][i];
        }
        if (i0 < a.cstride) *reinterpret_cast<i32x4*>(a.chunk_counts + (size_t)e * a.cstride + i0) = q;
        run += __builtin_amdgcn_readlane(x, 63);
        if (c0 + SEG >= a.chunks && lane == 0) s_cnt[e] = run;
      }
    }
  }
  __syncthreads();

  // 2. counts, offsets and the m-block table; thread i handles experts [i ept, (i + 1) ept)
  const int ept = (E + NT - 1) / NT, e0 = tid * ept;
  int csum = 0, msum = 0;
  for (int q = 0; q < ept; ++q) {
    const int e = e0 + q;
    if (e < E) {
      const int c = s_cnt[e];
      csum += c;
      msum += (c + BM - 1) / BM;
      a.counts[e] = c;
    }
  }
  int off_total, total_mb;
  int ebase = block_exclusive_scan<NT>(csum, s_tmp, off_total);
  int mbase = block_exclusive_scan<NT>(msum, s_tmp, total_mb);
  for (int q = 0; q < ept; ++q) {
    const int e = e0 + q;
    if (e >= E) break;
    const int c = s_cnt[e], nmb = (c + BM - 1) / BM;
    s_off[e] = ebase;
    t.mb[e] = mbase;
    for (int i = 0; i < nmb; ++i) {
      a.mb_expert[mbase + i] = e;
      a.mb_row0[mbase + i] = ebase + i * BM;
      const int rows = min(BM, c - i * BM);
      a.mb_rows[mbase + i] = rows | (a.wide_tails && 2 * rows <= BM ? kRowsWide : 0) | (nmb == 1 ? kRowsOnce : 0);
    }
    ebase += c;
    mbase += nmb;
  }
  if (tid == 0) {
    s_off[E] = off_total;  // = T * k
    t.mb[E] = total_mb;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += NT) a.offsets[e] = s_off[e];
  for (int i = tid; i < total_mb; i += NT) a.mb_ready[i] = 0;
  __syncthreads();

  // 3. on wavefront 0 alone when it can (the common case: a few expert waves)
  if (nw <= 64) {
    if (tid < 64) schedule_waves<true, NT>(a, t, nw, s_tmp, s_cost);
  } else {
    schedule_waves<false, NT>(a, t, nw, s_tmp, s_cost);
  }
  __syncthreads();

  // publish the wave table (scatter_kernel places the tiles from it) and the header
  for (int i = tid; i < wave_table_len(nw, E); i += NT) a.wtab[i] = s_tab[i];
  const int total_tiles = total_mb * (a.n1 + a.n2);
  const int total_units = t.head[kWtUnits];
  if (tid == 0) a.unit_start[total_units] = total_tiles;
  if (tid <= kGroups) {
    a.hdr[HDR_GTASK_OFF + tid] = t.head[kWtGoff + tid] * kUnit;
    a.hdr[HDR_GROUP_OFF + tid] = t.head[kWtGoff + tid];
  }
  if (tid < kGroups) a.hdr[HDR_GROUP_CURSOR + tid] = 0;
  if (tid == 0) {
    a.hdr[HDR_ERROR] = 0;
    a.hdr[HDR_CURSOR] = 0;
    a.hdr[HDR_NTASKS] = total_tiles;
    a.hdr[HDR_NMBLK] = total_mb;
    a.hdr[HDR_TILE_M] = BM;
    a.hdr[HDR_N1] = a.n1;
    a.hdr[HDR_N2] = a.n2;
    a.hdr[HDR_DONE] = 0;
    a.hdr[HDR_NUNITS] = total_units;
    a.hdr[HDR_LEAD] = t.head[kWtInterleaved] ? t.head[kWtLead] : 0;
    a.hdr[HDR_SCHED] = t.head[kWtInterleaved] ? MOE_SCHED_INTERLEAVED : MOE_SCHED_EXPERT_WAVE;
    a.hdr[HDR_PLAN_GRID] = a.grid;
  }
  __syncthreads();  // the LDS arrays may be reused once every thread is done with them
}

// 4. one tile of the list and its record. Inside a run the tiles of each expert are cut into
//    blocks of up to kBlockM m-blocks x kBlockN n-tiles and emitted block by block (n-tile
//    major inside a block: consecutive positions share a weight slab, which the workgroups of
//    an XCD then read while it is still in their L2). Every tile is placed independently from
//    the wave table. In a merged segment, Linear-1 unit v goes right after Linear-2 unit
//    ceil((v+1) * bu / au) (bu, au: unit counts), which spreads the Linear-1 units evenly and
//    ends the segment with the last Linear-1 unit. Each tile also writes its record into its
//    group's record list, where every unit owns kUnit consecutive slots (a short unit's spare
//    slots hold no-op records): so a tile's slot is (the unit's index in the groups' unit
//    lists) * kUnit + its offset in the unit.
__device__ void place_tile(const PlanArgs& a, const WaveTable& t, int nw, int ph, int mb, int nt) {
  const int n = ph ? a.n2 : a.n1;
  const int BM = a.tile_m, D = t.head[kWtLead];
  const bool interleaved = t.head[kWtInterleaved] != 0;
  int e = 0;  // the expert e with t.mb[e] <= mb < t.mb[e + 1] (the last of equal starts)
  for (int hi = a.E - 1; e < hi;) {
    const int mid = (e + hi + 1) >> 1;
    if (t.mb[mid] <= mb) e = mid;
    else hi = mid - 1;
  }
  const int w = e / a.W;
  const int nmb = t.mb[e + 1] - t.mb[e], ml = mb - t.mb[e];
  const int mg = ml / kBlockM, ng = nt / kBlockN;
  const int bm_act = min(kBlockM, nmb - mg * kBlockM);
  const int q = (t.mb[e] - t.mb[w * a.W]) * n + mg * kBlockM * n + ng * bm_act * kBlockN +
                (nt - ng * kBlockN) * bm_act + (ml - mg * kBlockM);
  const int ur = q / kUnit, o = q % kUnit;  // unit of the run, offset in the unit
  // positions and unit counts stay below 2^31 (the host caps the tile count), so 32-bit
  // unsigned arithmetic is exact here
  unsigned at;
  int unit, other_before;  // other_before: units of the other phase earlier in the list
  if (!interleaved) {
    at = (unsigned)(ph ? t.l2s[w] : t.l1s[w]) + q;
    unit = (ph ? t.l2u[w] : t.l1u[w]) + ur;
    other_before = ph ? t.p1[w + 1] : t.p2[w];
  } else if (ph == 0 && w < D) {  // lead prefix
    at = (unsigned)t.l1s[w] + q;
    unit = t.l1u[w] + ur;
    other_before = 0;
  } else if (ph == 1) {  // Linear-2 unit ur of segment w
    const int bu = units_of(t.b[w]);
    const int au = w + D < nw ? units_of(t.a[w + D]) : 0;
    const int l1_before = au ? (int)((unsigned)ur * au / bu) : 0;  // all full units
    at = (unsigned)t.l2s[w] + (unsigned)(ur + l1_before) * kUnit + o;
    unit = t.l2u[w] + ur + l1_before;
    other_before = t.p1[min(w + D, nw)] + l1_before;
  } else {  // Linear-1 unit ur of wave w, in segment w - D
    const int b = t.b[w - D], bu = units_of(b), au = units_of(t.a[w]);
    const int c = bu ? (int)(((unsigned)(ur + 1) * bu + au - 1) / au) : 0;  // L2 units before
    at = (unsigned)t.l1s[w] + (unsigned)ur * kUnit + (c == bu ? b : c * kUnit) + o;
    unit = t.l1u[w] + ur + c;
    other_before = t.p2[w - D] + c;
  }
  a.tasks[at] = make_task(ph, mb, nt);
  // Units of each phase are dealt round-robin to the groups in list order: this unit is
  // number pidx of its phase, so it goes to group pidx % G; its place in that group's list
  // counts the group's earlier units of both phases.
  const int pidx = (ph ? t.p2[w] : t.p1[w]) + ur;
  const int g = pidx % kGroups;
  const int rank = pidx / kGroups + (other_before - g + kGroups - 1) / kGroups;
  const int goff = t.head[kWtGoff + g];
  const size_t slot0 = (size_t)(goff + rank) * kUnit;
  // the record: task word, expert, first dispatched row and rows of the m-block
  const int off_e = t.off[e], cnt_e = t.off[e + 1] - off_e;
  i32x4 rec;
  rec[0] = make_task(ph, mb, nt);
  rec[1] = e;
  rec[2] = off_e + ml * BM;
  rec[3] = min(BM, cnt_e - ml * BM);
  if (nmb == 1) rec[3] |= kRowsOnce;
  if (a.wide_tails && 2 * (rec[3] & ~kRowsFlags) <= BM) {  // a wide m-block: even n-tiles cover two
    rec[3] |= kRowsWide;
    if (nt & 1) rec = i32x4{kNopTask, -1, 0, 0};
  }
  *reinterpret_cast<i32x4*>(a.gtasks + 4 * (slot0 + o)) = rec;
  if (o == 0) {
    a.unit_start[unit] = (int)at;
    a.group_units[goff + rank] = unit;
    const int size = min(kUnit, (ph ? t.b[w] : t.a[w]) - ur * kUnit);
    for (int s = size; s < kUnit; ++s)  // a short unit's spare slots
      *reinterpret_cast<i32x4*>(a.gtasks + 4 * (slot0 + s)) = i32x4{kNopTask, -1, 0, 0};
  }
}

// Stable ranks of a run of slots inside their experts, 64 slots per step: every lane reads
// the run's running count `run[e]` (LDS) of its expert, lanes holding the same expert are
// found with a ballot per distinct expert (the leader's expert broadcast by readlane) and
// ranked by lane order, and the expert's last lane advances `run[e]` by their number. With
// `emit`, rows are written out.
template <bool emit>
__device__ void rank_run(const PlanArgs& a, int f0, int f1, int* run) {
  const int lane = threadIdx.x & 63;
  const int R = a.T * a.k;
  for (int s = f0; s < f1; s += 64) {
    const int f = s + lane;
    int e = f < f1 ? a.topk_ids[f] : -1;
    if ((unsigned)e >= (unsigned)a.E) e = -1;
    const int base = e >= 0 ? run[e] : 0;
    unsigned long long remaining = __ballot(e >= 0);
    int rank = 0, cnt = 0;
    while (remaining) {
      const int leader = __ffsll((long long)remaining) - 1;
      const int ev = __builtin_amdgcn_readlane(e, leader);
      const unsigned long long m = __ballot(e == ev);
      if (e == ev) {
        rank = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        cnt = __popcll(m);
      }
      remaining &= ~m;
    }
    const int row = base + rank;
    if (e >= 0 && rank == cnt - 1) run[e] = base + cnt;
    if (emit && e >= 0 && (unsigned)row < (unsigned)R) {
      a.perm[row] = f;
      a.pos[f] = row;
    }
  }
}

// The scatter of one token chunk on an NT-thread workgroup. run: LDS of NT / 64 rows of
// MOE_MAX_EXPERTS ints, the per-wavefront running counts (first the wave's own counts, then
// its first rows).
template <int NT>
__device__ void scatter_chunk(const PlanArgs& a, int chunk, int* run_lds) {
  constexpr int kPlanWaves = NT / 64;
  int (*run)[MOE_MAX_EXPERTS] = reinterpret_cast<int (*)[MOE_MAX_EXPERTS]>(run_lds);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int R = a.T * a.k;
  const int c0 = chunk * a.chunk_tokens * a.k;
  const int c1 = min(R, c0 + a.chunk_tokens * a.k);
  const int per_wave = (c1 - c0 + kPlanWaves - 1) / kPlanWaves;  // every wavefront takes a share
  const int f0 = min(c1, c0 + wave * per_wave), f1 = min(c1, f0 + per_wave);
  for (int e = tid; e < a.E; e += NT)
    for (int w = 0; w < kPlanWaves; ++w) run[w][e] = 0;
  __syncthreads();
  rank_run<false>(a, f0, f1, run[wave]);  // counts of this wave's slots per expert
  __syncthreads();
  for (int e = tid; e < a.E; e += NT) {
    // chunk's first row of expert e: the expert's offset plus its rows in earlier chunks
    int r = a.offsets[e] + a.chunk_counts[(size_t)e * a.cstride + chunk];
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = run[w][e];
      run[w][e] = r;
      r += c;
    }
  }
  __syncthreads();
  rank_run<true>(a, f0, f1, run[wave]);
  __syncthreads();  // run may be reused by the next chunk
}

// 4. the tile list: tile u of all (m-block, n-tile) pairs, Linear-1 then Linear-2, goes to
//    block u % nb of nb placing blocks (blk is this one); the wave table is copied into s_tab
//    (LDS of kWaveTableLds ints)
template <int NT>
__device__ void place_tiles(const PlanArgs& a, int blk, int nb, int* s_tab) {
  const int tid = threadIdx.x;
  const int nw = (a.E + a.W - 1) / a.W, len = wave_table_len(nw, a.E);
  const int total_mb = a.wtab[len - a.E - 2], t1 = total_mb * a.n1, total = t1 + total_mb * a.n2;
  if (blk >= min(nb, total)) return;
  for (int i = tid; i < len; i += NT) s_tab[i] = a.wtab[i];
  __syncthreads();
  const WaveTable t(s_tab, nw, a.E);
  for (int u = blk + nb * tid; u < total; u += nb * NT) {
    const int ph = u >= t1 ? 1 : 0;
    const int n = ph ? a.n2 : a.n1, v = u - ph * t1;
    const int mb = v / n;
    place_tile(a, t, nw, ph, mb, v - mb * n);
  }
  __syncthreads();  // s_tab may be reused
}

}  // namespace
}  // namespace moe
