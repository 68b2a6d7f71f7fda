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
//   plan           all of the above in ONE launch (MOE_FLAG_PLAN_ONE_LAUNCH): a grid of resident
//                  workgroups routes the chunks, the last one to arrive runs the scan and
//                  schedule step while the others wait at a grid barrier, then all scatter
//                  the chunks and place the tile list.
//
// The dispatch gather and the combine are in moe_combine.hip.
#include "moe_plan_dev.h"
#include "moe_sync_dev.h"

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

// The planner in one launch: the route, scan-and-schedule and scatter kernels' steps with a
// grid barrier (moe_sync_dev.h) between routing and the schedule's readers. Every workgroup is
// resident (the grid is capped at the resident capacity) and takes token chunks b, b + G, ...
// The barrier counters live in the workspace (zero between launches; the last workgroup out
// sets them back to zero); a wait that expires skips the scatter and records MOE_ERR_TIMEOUT.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a, int32_t* sync, int spin_limit) {
  // the largest step's LDS: the scatter's 16 rows of running counts (64 KiB); the scan and
  // schedule step needs about 54 KiB of it
  __shared__ __align__(16) int lds[kPlanThreads / 64 * MOE_MAX_EXPERTS];
  __shared__ int bc[2];
  static_assert(4 * (32 + MOE_MAX_EXPERTS + ((kWaveTableLds + 1) & ~1)) + 8 * MOE_MAX_EXPERTS <= sizeof(lds),
                "LDS of the scan and schedule step");
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  for (int c = b; c < a.chunks; c += G) route_chunk<kPlanThreads>(a, c, lds);
  if (layer_count(sync, kSyncArrive, kSyncAll, 1, bc)) {
    // every chunk's counts are in: this workgroup writes the schedule, then opens the barrier
    int* const s_tmp = lds;
    int* const s_cnt = lds + 32;
    int* const s_tab = s_cnt + MOE_MAX_EXPERTS;
    double* const s_cost = reinterpret_cast<double*>(s_tab + ((kWaveTableLds + 1) & ~1));
    scan_schedule_block<kPlanThreads>(a, s_tmp, s_cnt, s_tab, s_cost);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    layer_open(sync, 1);
  }
  // short polls: at most two workgroups per CU wait, with nothing else to do
  if (layer_wait<4>(sync, 1, spin_limit, bc)) {
    for (int c = b; c < a.chunks; c += G) scatter_chunk<kPlanThreads>(a, c, lds);
    place_tiles<kPlanThreads>(a, b, min(G, kPlaceBlocks), lds);
  } else if (threadIdx.x == 0) {
    atomicCAS(sync_line(sync, kSyncErr), 0, (int)MOE_ERR_TIMEOUT);
  }
  if (layer_count(sync, kSyncExit, kSyncAllExit, 1, bc)) {
    if (sync_line(sync, kSyncErr)[0] != 0 && threadIdx.x <= kGroups) {
      // an expired wait left perm, pos and the tile records unwritten: publish an empty tile
      // list, so that a moe_forward on this plan runs no tile (its readers of the routing
      // arrays skip entries out of range)
      a.hdr[HDR_GTASK_OFF + threadIdx.x] = 0;
      a.hdr[HDR_GROUP_OFF + threadIdx.x] = 0;
      if (threadIdx.x == 0) {
        a.hdr[HDR_NTASKS] = 0;
        a.hdr[HDR_NUNITS] = 0;
      }
    }
    __syncthreads();
    layer_sync_reset(sync, a.hdr);
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, int32_t* sync, int spin_limit, hipStream_t s) {
  // resident capacity: the grid never exceeds it, so every workgroup runs at once
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, plan_kernel, kPlanThreads, 0);
  if (err != hipSuccess) return err;
  const int capacity = cus * (per_cu > 0 ? per_cu : 1);
  const int grid = a.chunks < capacity ? a.chunks : capacity;
  hipLaunchKernelGGL(plan_kernel, dim3(grid), dim3(kPlanThreads), 0, s, a, sync, spin_limit);
  return hipGetLastError();
}

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
