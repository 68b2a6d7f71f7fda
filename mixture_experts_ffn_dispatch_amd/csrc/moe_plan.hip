// Routing and planning kernels of libmoe (gfx950).
//
// The layer's router picks k experts per token and Dispatch groups every token's copies by
// expert (X-Stage paper, Introduction, MoE-layer paragraph); the expert-wave paragraph and
// Section 4.2 (MegaMoE) fix the tile orders that the schedule builder writes.
//
//   route_*        one block per token chunk, one wavefront per token (or one segment of
//                  2^n >= E lanes per token when E <= 64): top-k over the E logits
//                  (descending, ties to the lower expert id), renormalised softmax weights, and
//                  a per-(expert, chunk) count of the routed slots (LDS atomics on integers:
//                  order-free, exact).
//   scan_schedule  one workgroup: per-expert exclusive scans of the count table (one
//                  wavefront per expert row), which give every (expert, chunk) its first row
//                  within the expert and every expert its count; the expert offsets, the
//                  m-block table and zeroed dependency counters; then, on one wavefront when
//                  there are at most 64 expert waves, the per-wave tile counts, the lead and
//                  where each wave's runs start (the wave table, written to the workspace).
//   scatter        one block per chunk, its slots split into 16 consecutive runs, one per
//                  wavefront: per-run expert counts, a per-expert prefix over the runs, then
//                  stable ranks (ballot/match over 64 slots at a time) give perm and pos.
//                  Then every block places its share of the tile list and the group records
//                  from the wave table (each tile independently).
//
// The dispatch gather and the combine are in moe_combine.hip.
#include "moe_plan_dev.h"

namespace moe {
namespace {

// The planner's own kernels: 1024-thread workgroups, one per token chunk (route, scatter) or
// one in all (scan and schedule).
template <int R>
__global__ __launch_bounds__(kPlanThreads) void route_hist_kernel(PlanArgs a) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  route_hist_chunk<R, kPlanThreads>(a, blockIdx.x, cnt);
}

template <int S>
__global__ __launch_bounds__(kPlanThreads) void route_small_kernel(PlanArgs a) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  route_small_chunk<S, kPlanThreads>(a, blockIdx.x, cnt);
}

__global__ __launch_bounds__(kPlanThreads) void scan_schedule_kernel(PlanArgs a) {
  __shared__ int s_tmp[32];
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_tab[kWaveTableLds];
  __shared__ double s_cost[MOE_MAX_EXPERTS];
  scan_schedule_block<kPlanThreads>(a, s_tmp, s_cnt, s_tab, s_cost);
}

__global__ __launch_bounds__(kPlanThreads) void scatter_kernel(PlanArgs a) {
  // 16 rows of running counts (64 KiB), then the wave table in the same space
  __shared__ int run[kPlanThreads / 64 * MOE_MAX_EXPERTS];
  static_assert(kPlanThreads / 64 * MOE_MAX_EXPERTS >= kWaveTableLds, "wave table fits");
  scatter_chunk<kPlanThreads>(a, blockIdx.x, run);
  place_tiles<kPlanThreads>(a, blockIdx.x, min((int)gridDim.x, kPlaceBlocks), run);
}

}  // namespace

hipError_t launch_route_hist(const PlanArgs& a, hipStream_t s) {
  const int R = (a.E + 63) / 64;
  const dim3 grid(a.chunks), block(kPlanThreads);
  if (a.E <= 8) hipLaunchKernelGGL(route_small_kernel<8>, grid, block, 0, s, a);
  else if (a.E <= 16) hipLaunchKernelGGL(route_small_kernel<16>, grid, block, 0, s, a);
  else if (a.E <= 32) hipLaunchKernelGGL(route_small_kernel<32>, grid, block, 0, s, a);
  else if (R <= 1) hipLaunchKernelGGL(route_small_kernel<64>, grid, block, 0, s, a);
  else if (R <= 2) hipLaunchKernelGGL(route_hist_kernel<2>, grid, block, 0, s, a);
  else if (R <= 4) hipLaunchKernelGGL(route_hist_kernel<4>, grid, block, 0, s, a);
  else if (R <= 8) hipLaunchKernelGGL(route_hist_kernel<8>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(route_hist_kernel<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan_schedule(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scan_schedule_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(a.chunks), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
