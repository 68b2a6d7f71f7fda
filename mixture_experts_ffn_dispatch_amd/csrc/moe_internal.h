// Internal declarations shared by the libmoe translation units (host and device side).
// Not part of the public ABI; the public contract is include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Workspace header slots (int32).
enum : int {
  HDR_ERROR = 0,   // device-side error code (0 or MOE_ERR_TIMEOUT)
  HDR_CURSOR = 1,  // next task index handed to a persistent workgroup
  HDR_NTASKS = 2,  // tasks in the list
  HDR_NMBLK = 3,   // m-blocks in the table
  HDR_TILE_M = 4,
  HDR_N1 = 5,
  HDR_N2 = 6,
  HDR_DONE = 7,    // persistent workgroups that have exited (the last one resets the state)
  HDR_GROUP_CURSOR = 8,   // [8, 16): records of each locality group's tile list handed out
  HDR_NUNITS = 16,        // units in the unit table
  HDR_GROUP_OFF = 17,     // [17, 26): first entry of each group's unit list (9th = end)
  HDR_LEAD = 26,          // interleave lead the plan used (0 for the Expert-Wave order)
  HDR_PLAN_GRID = 27,     // GEMM grid size the plan assumed when it chose the lead
  HDR_SCHED = 28,         // the order the plan wrote (MOE_SCHED_EXPERT_WAVE / _INTERLEAVED)
  HDR_GTASK_OFF = 32,     // [32, 41): first record of each group's tile list (9th = end)
  HDR_SLOTS = 64
};

// Locality groups of the persistent GEMM: workgroup w belongs to group w % kGroups, and all
// workgroups of a group run on one XCD (the hardware deals workgroups to the 8 XCDs
// round-robin; which XCD gets group 0 varies from one dispatch to the next). The list is
// made of units (kUnit consecutive tiles of one run, written in blocks of kBlockM m-blocks x
// kBlockN n-tiles of one expert). Linear-1 units are dealt round-robin to the groups in list
// order, and so are Linear-2 units, so every group gets an even share of both kinds of work;
// the workgroups that share an XCD's L2 work on tiles of one unit, which share operand rows.
// Each group's units, in its order, are also written out as one flat list of tile records
// (task word, expert, first row, rows), kUnit slots per unit, so a workgroup claims a tile
// with one atomic on its group's cursor and one 16-byte load.
constexpr int kGroups = 8;
constexpr int kUnit = 32;
constexpr int kBlockM = 4;
constexpr int kBlockN = 8;
// The planner's wave table (per-wave tile counts, unit prefix sums and run starts, and each
// expert's first m-block and first row): a head of kWaveTableHead ints, then at most
// 10 (E + 1) entries.
constexpr int kWaveTableHead = 24;

// MOE_SCHED_AUTO's model of this kernel on this GPU: sustained MFMA rate of its tiles,
// weight-streaming rate, the last-level cache, and the local memory path's calibration
// (moe_burst_gap on this GPU's own memory).
constexpr double kAutoMfmaFlops = 1.2e15;
constexpr double kAutoStreamBytes = 5.0e12;
constexpr double kAutoCacheBytes = 256.0 * 1024 * 1024;
constexpr double kLocalIssueUs = 0.927;
constexpr double kLocalDrainGBps = 6646.0;
constexpr double kLocalCapacityMiB = 31.2;

constexpr int kTileN2 = 256;         // Linear-2 tile: Yd columns
constexpr int kTileN1 = 128;         // Linear-1 tile: A columns (=> 128 gate + 128 up weight rows)
constexpr int kTileK = 64;           // K step staged through LDS
constexpr int kTaskL2Bit = 31;
constexpr int kTaskMblkShift = 12;
constexpr int kTaskMblkBits = 19;
constexpr int kTaskNtMask = 0xFFF;
constexpr int kDefaultSpinLimit = 1 << 22;
// A Linear-2 tile whose m-block is still not ready after kDeferTicks of the 100 MHz real-time
// counter (1 ms; a healthy wait lasts at most about one Linear-1 tile) is set aside in the
// workgroup's deferral slot, and the workgroup runs tiles that cannot wait until it is ready.
constexpr long long kDeferTicks = 100000;
constexpr int kDeferSlots = 2048;  // workgroups with a deferral slot (others never defer)
constexpr int kReleaseBatch = 2;  // Linear-1 completions a GEMM workgroup releases together
// "no more tiles": all ones. Never a real task because m-block 0x7FFFF is out of range
// (the host rejects plans with 2^19 - 1 or more m-blocks).
constexpr int32_t kNoTask = -1;
// A spare slot of a group record list (units own kUnit slots each; a short unit leaves some
// empty): Linear-1, m-block 0x7FFFF (out of range, as above), n-tile 0xFFE. Claiming one just
// means claiming again.
constexpr int32_t kNopTask = 0x7FFFFFFE;
// Bit of a record's (and the m-block table's) row count that marks a wide m-block: with
// 256-row tiles, an m-block of at most 128 rows runs as tiles of 512 weight rows (two n-tiles,
// the even one named in the task word) by 128 token rows; its odd n-tiles hold no-op records.
constexpr int32_t kRowsWide = 1 << 30;
// Bit of the same words that marks the only m-block of its expert: every weight byte the
// m-block's tiles read is then read by no other tile, so those loads are non-temporal.
constexpr int32_t kRowsOnce = 1 << 29;
constexpr int32_t kRowsFlags = kRowsWide | kRowsOnce;

// Task word: bit 31 = Linear-2, bits 30..12 = m-block, bits 11..0 = n-tile.
__host__ __device__ inline int32_t make_task(int l2, int mblk, int nt) {
  return (int32_t)(((uint32_t)l2 << kTaskL2Bit) | ((uint32_t)mblk << kTaskMblkShift) | (uint32_t)nt);
}

struct PlanArgs {
  const float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  int32_t* hdr;
  int32_t* chunk_counts;  // [E][cstride]: entries [0, chunks) of each row are used
  int32_t* mb_expert;
  int32_t* mb_row0;
  int32_t* mb_rows;
  int32_t* mb_ready;
  int32_t* tasks;
  int32_t* unit_start;  // [max_units + 1]: list position of each unit's first tile
  int32_t* group_units; // [max_units]: each group's units in list order, groups one after another
  int32_t* gtasks;      // [slots][4]: each group's tile records (kUnit slots per unit), groups one after another
  int32_t* wtab;        // the wave table: per-wave tile counts and list positions for the tile placement
  int max_units;
  int T, E, k, chunks, chunk_tokens;
  int cstride;   // row stride of chunk_counts: chunks rounded up to a multiple of 4 (16 B)
  int W;         // experts per wave
  int schedule;  // MOE_SCHED_*
  int lead;      // interleave lead (>= 1), or 0: chosen from the tile counts
  int tile_m, n1, n2;
  int H, I;      // Linear-1 K = H, Linear-2 K = I (tile durations scale with them)
  int grid;      // persistent GEMM workgroups (tiles in flight)
  double xs_issue_s, xs_drain_bps, xs_capacity_b;  // X-Stage calibration for MOE_SCHED_AUTO
  int wide_tails;  // 1: m-blocks of at most tile_m / 2 rows become wide (256-row tiles only)
};

struct GemmArgs {
  const uint16_t* xd;      // dispatched rows [R, H], or unused when gather is set
  const uint16_t* x;       // token rows [T, H] (gather): Linear-1 reads row perm[r] / k for row r
  const int32_t* perm;     // [R] (gather)
  int T, k, gather;
  const uint16_t* w1;
  const uint16_t* w2;
  uint16_t* act;
  uint16_t* yd;
  int32_t* hdr;
  const int32_t* tasks;   // the tile list in schedule order (one shared cursor when ngroups is 1)
  const int32_t* gtasks;  // [slots][4]: each group's tile records (task, expert, row0, rows)
  int ngroups;  // 1: one shared cursor over the list; kGroups: each group takes its own records
  const int32_t* mb_expert;
  const int32_t* mb_row0;
  const int32_t* mb_rows;
  int32_t* mb_ready;
  int R;  // dispatched rows T*k
  int H, I, E;
  int n1;  // Linear-1 n-tiles per m-block (the dependency target)
  int max_tasks, max_mblk;  // capacity of the workspace arrays (guards against a stale plan)
  int max_slots;            // capacity of the group record lists
  int spin_limit;
  int force_timeout;
  int absent_group;      // MOE_FLAG_TEST_ABSENT_GROUP: this group's workgroups take no tile (-1: none)
  int32_t* defer;        // [kDeferSlots][8]: each workgroup's deferred Linear-2 tile
  moe_trace_rec* trace;  // per-tile records (moe_config.trace), or null
};

// The single-launch layer kernel: plan, the persistent GEMM with the dispatch gather, combine.
struct LayerArgs {
  GemmArgs g;      // gather mode: Linear-1 reads token rows of x through perm
  PlanArgs pl;     // the planner's arguments (pl.grid = the launch's grid)
  const float* topk_w;
  const int32_t* pos;
  uint16_t* out;
  int segs;        // column segments per token row in the combine
  int32_t* sync;   // the phase barriers' counters (kLayerSyncBytes, zero between launches)
};

// The single-launch layer's phase barriers: one 128-byte line (32 ints) per counter, so that
// the groups' counters sit on separate cache lines. Lines 0-7: each locality group's
// arrivals; 8: the groups whose every workgroup has arrived; 9-16: each group's "go" word
// (the last barrier the group may pass); 17: a timeout to report; 18-25: each group's exits;
// 26: the groups whose every workgroup has exited.
constexpr int kLayerSyncBytes = 4096;
constexpr int kSyncLine = 32;  // ints per line
constexpr int kSyncArrive = 0, kSyncAll = 8, kSyncGo = 9, kSyncErr = 17, kSyncExit = 18, kSyncAllExit = 26;

// Launchers (return the hipError_t of the launch).
// The planner in one launch (route, scan and schedule, scatter and tile placement); sync: the
// workspace's barrier counters (kLayerSyncBytes, zero between launches).
hipError_t launch_plan(const PlanArgs& a, int32_t* sync, int spin_limit, hipStream_t s);
hipError_t launch_route_hist(const PlanArgs& a, hipStream_t s);
hipError_t launch_scan_schedule(const PlanArgs& a, hipStream_t s);
hipError_t launch_scatter(const PlanArgs& a, hipStream_t s);
hipError_t launch_dispatch(const int32_t* pos, const uint16_t* x, uint16_t* xd, int T, int H, int k,
                           hipStream_t s);
hipError_t launch_combine(const int32_t* pos, const float* w, const uint16_t* yd, uint16_t* out, int T,
                          int H, int k, hipStream_t s);
// Persistent grouped GEMM; grid = num_workgroups (0 = CUs x occupancy).
hipError_t launch_gemm(const GemmArgs& a, int tile_m, bool wide, int num_workgroups, hipStream_t s);
// The grid launch_gemm uses for this tile height and request (every workgroup resident at once).
hipError_t gemm_grid(int tile_m, bool wide, int num_workgroups, int* grid);
// The single-launch layer kernel on the grid gemm_grid gives (la.pl.grid must hold it).
hipError_t launch_layer(const LayerArgs& la, int tile_m, bool wide, int num_workgroups, hipStream_t s);

// Whether moe_plan writes wide last m-blocks, and moe_forward launches the kernel instance that
// runs them: only with 256-row tiles; MOE_FLAG_WIDE_TAILS / MOE_FLAG_NO_WIDE_TAILS force the
// choice, else wide when the average expert fills at most three m-blocks (T * k <= 3 * 256 * E),
// where last blocks are a large share of the tiles. Both calls derive it from the same config.
inline bool plan_wide_tails(const moe_config* c, int tile_m) {
  return tile_m == 256 && (c->flags & MOE_FLAG_WIDE_TAILS) && !(c->flags & MOE_FLAG_NO_WIDE_TAILS);
}
// Column segments per token row: with few tokens, rows are cut into up to 4 segments of at
// least 128 chunks (one step of a wavefront) so that about 4096 wavefronts run.
inline int combine_segments(int T, int H) {
  const int cpr = H / 8;
  int segs = (4096 + T - 1) / T;
  segs = segs < 1 ? 1 : segs > 4 ? 4 : segs;
  while (segs > 1 && cpr / segs < 128) --segs;
  return segs;
}

// Burst-Gap microbenchmark: `producers` workgroups, each storing `bytes` per burst into its own
// `region` of buf, `periods` times, with a busy gap of `gap_ticks` real-time counter ticks.
hipError_t launch_burst_gap(uint8_t* buf, size_t region, int producers, int bytes, int periods,
                            long long gap_ticks, long long* times, hipStream_t s);

}  // namespace moe
