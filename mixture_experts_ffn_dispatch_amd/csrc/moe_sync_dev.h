// Grid barriers of libmoe's single-launch kernels (gfx950): the layer kernel (moe_gemm.hip)
// and the one-launch planner (moe_plan.hip). Every workgroup of such a grid is resident at
// once (the grid never exceeds the resident capacity), so a workgroup can wait for all others.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// Barrier n (1, 2, 3, ... within a launch) is hierarchical, like the GEMM's locality groups
// (workgroup w in group w % 8): a workgroup drains its stores, releases at agent scope and
// counts itself on its group's line; the group's last arrival counts the group on the
// all-groups line; the last group's arrival opens barrier n by writing n into every group's
// go word (a caller may first do work that the others wait for, as the planner's schedule
// step). A wait polls its own group's go word (bounded by spin_limit) and acquires. The
// counters (kLayerSyncBytes of the workspace, zero between launches) only grow during a
// launch (barrier n is complete at n arrivals per member), and the last workgroup to exit sets
// them back to zero. bc: two LDS words for the broadcast to the workgroup.

__device__ inline int* sync_line(int32_t* sync, int line) { return sync + line * kSyncLine; }

// Counts this workgroup on `lines` (group arrivals at line lines + g, groups at line `all`)
// for the n-th time; true (on every thread) when it was the last arrival of the whole grid,
// which then holds (acquired) every other arrival's release.
__device__ bool layer_count(int32_t* sync, int lines, int all, int n, int* bc) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = (int)gridDim.x, ng = min(G, kGroups), g = (int)blockIdx.x % kGroups;
    const int members = (G - g + kGroups - 1) / kGroups;
    int last = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int c = __hip_atomic_fetch_add(sync_line(sync, lines + g), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c + 1 == n * members) {  // the group's last: count the group
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      const int d = __hip_atomic_fetch_add(sync_line(sync, all), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d + 1 == n * ng) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        last = 1;
      }
    }
    bc[0] = last;
  }
  __syncthreads();
  return bc[0] != 0;
}

// Opens barrier n for every group (called by the grid's last arrival, one thread enough).
__device__ void layer_open(int32_t* sync, int n) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int ng = min((int)gridDim.x, kGroups);
    for (int h = 0; h < ng; ++h)
      __hip_atomic_store(sync_line(sync, kSyncGo + h), n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Waits until barrier n is open for this workgroup's group; false (on every thread) when the
// bounded wait expired. SLEEP: the pause between polls (s_sleep units of 64 clocks).
template <int SLEEP = 32>
__device__ bool layer_wait(int32_t* sync, int n, int spin_limit, int* bc) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int* go = sync_line(sync, kSyncGo + (int)blockIdx.x % kGroups);
    int ok = 1, spins = 0;
    // by default a poll about every microsecond: up to 64 workgroups share a go word, and the
    // grid's polls should not crowd the memory path of the workgroup that writes the schedule
    while (__hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
      if (++spins > spin_limit) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(SLEEP);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    bc[1] = ok;
  }
  __syncthreads();
  return bc[1] != 0;
}

// A full barrier n: arrive, the grid's last arrival opens it, wait.
__device__ bool layer_barrier(int32_t* sync, int n, int spin_limit, int* bc) {
  if (layer_count(sync, kSyncArrive, kSyncAll, n, bc)) layer_open(sync, n);
  return layer_wait(sync, n, spin_limit, bc);
}

// Run by the grid's last workgroup out (after its layer_count on the exit lines): moves a
// recorded timeout into the workspace's error word and sets every counter back to zero for
// the next launch.
__device__ void layer_sync_reset(int32_t* sync, int32_t* hdr) {
  if (threadIdx.x < kLayerSyncBytes / 4 / kSyncLine) {  // one thread per line
    int* const line = sync_line(sync, threadIdx.x);
    if (threadIdx.x == kSyncErr && line[0]) atomicCAS(hdr + HDR_ERROR, 0, line[0]);
    line[0] = 0;
  }
}

}  // namespace
}  // namespace moe
