// C ABI of libmoe (declared in include/moe.h): argument validation, workspace layout and
// kernel launches. Host code only; every call validates before it launches anything.
#include <string.h>

#include <mutex>

#include "moe_internal.h"

// The workspace of moe_layer_noalloc: one array per GPU, held until the process ends. In host
// code this name is only a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress (scratch_address below), and only that address is used.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace moe {
namespace {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Rows per GEMM tile for a routing-average of T*k/E rows per expert (the host does not know
// the actual counts). The 256-row tile (eight wavefronts, two per SIMD) is the most efficient
// per flop and wins from about 112 rows per expert on average despite its padding. Below that
// the 128-row tile (one workgroup per CU, weight rows loaded two K steps ahead) streams the
// weights best, and with skewed routing its fewer m-blocks per large expert re-read less; only
// a few rows per expert (under 20) favour the 32-row tile, by a few percent. The 64-row tile
// is still available explicitly (it wins, by ~2%, only for uniform routing near 48 rows).
int auto_tile_m(const moe_config& c) {
  const double avg = (double)c.T * c.k / c.E;
  if (avg >= 112) return 256;
  if (avg >= 20) return 128;
  return 32;
}

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 1 || c->H < 1 || c->I < 1 || c->E < 1 || c->k < 1 || c->k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->experts_per_wave < 1) return MOE_ERR_INVALID_ARG;
  if (c->schedule != MOE_SCHED_EXPERT_WAVE && c->schedule != MOE_SCHED_INTERLEAVED && c->schedule != MOE_SCHED_AUTO)
    return MOE_ERR_INVALID_ARG;
  if (c->lead_waves < 0 || c->num_workgroups < 0 || c->spin_limit < 0) return MOE_ERR_INVALID_ARG;
  if (c->schedule == MOE_SCHED_AUTO && c->lead_waves != 0) return MOE_ERR_INVALID_ARG;
  // calibration: finite and not negative (0 = the local calibration); !(x >= 0) also catches NaN
  if (!(c->xs_issue_us >= 0.f) || !(c->xs_drain_gbps >= 0.f) || !(c->xs_capacity_mib >= 0.f) ||
      c->xs_issue_us > 1e9f || c->xs_drain_gbps > 1e9f || c->xs_capacity_mib > 1e9f)
    return MOE_ERR_INVALID_ARG;
  if (c->flags & ~(MOE_FLAG_FORCE_WAIT_TIMEOUT | MOE_FLAG_NO_WIDE_TAILS | MOE_FLAG_WIDE_TAILS |
                   MOE_FLAG_PLAN_ONE_LAUNCH | MOE_FLAG_TEST_ABSENT_GROUP))
    return MOE_ERR_INVALID_ARG;
  if ((c->flags & MOE_FLAG_NO_WIDE_TAILS) && (c->flags & MOE_FLAG_WIDE_TAILS)) return MOE_ERR_INVALID_ARG;
  if (c->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (c->tile_m != 0 && c->tile_m != 32 && c->tile_m != 64 && c->tile_m != 128 && c->tile_m != 256)
    return MOE_ERR_UNSUPPORTED;
  if (c->E > MOE_MAX_EXPERTS || c->k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (c->H % MOE_DIM_MULTIPLE || c->I % MOE_DIM_MULTIPLE) return MOE_ERR_UNSUPPORTED;
  // 32-bit buffer ranges: dispatched row buffers and one expert's weight slab
  const unsigned long long R = (unsigned long long)c->T * (unsigned long long)c->k;
  const unsigned long long lim = 0xFFFFFFFFull;
  if (R > 0x7FFFFFFFull) return MOE_ERR_UNSUPPORTED;
  if (R * (unsigned long long)c->H * 2ull > lim || R * (unsigned long long)c->I * 2ull > lim) return MOE_ERR_UNSUPPORTED;
  if (4ull * (unsigned long long)c->I * (unsigned long long)c->H > lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status compute_layout(const moe_config* c, moe_ws_layout* L) {
  moe_status st = check_config(c);
  if (st != MOE_OK) return st;
  memset(L, 0, sizeof(*L));
  const long long R = (long long)c->T * c->k;
  const int BM = c->tile_m ? c->tile_m : auto_tile_m(*c);
  const long long n1 = (c->I + kTileN1 - 1) / kTileN1;
  const long long n2 = (c->H + kTileN2 - 1) / kTileN2;
  // routing histogram granularity: at least 16 tokens per chunk, and at most 32K (expert,
  // chunk) counts so the single-workgroup scan stays short
  long long chunk_tokens = ((long long)c->T * c->E + 32767) / 32768;
  chunk_tokens = chunk_tokens < 16 ? 16 : (chunk_tokens + 15) / 16 * 16;
  const long long chunks = ((long long)c->T + chunk_tokens - 1) / chunk_tokens;
  const long long active = R < c->E ? R : c->E;
  const long long max_mblk = (R + active * (BM - 1)) / BM;
  const long long max_tasks = max_mblk * (n1 + n2);
  if (n1 > kTaskNtMask || n2 > kTaskNtMask) return MOE_ERR_UNSUPPORTED;
  if (max_mblk >= (1ll << kTaskMblkBits) - 1) return MOE_ERR_UNSUPPORTED;
  // the planner places tiles with 32-bit arithmetic on unit counts: keep the list below 2^20
  if (max_tasks > (1ll << 20) || chunks * c->E > 0x7FFFFFFFll) return MOE_ERR_UNSUPPORTED;
  L->chunks = (int32_t)chunks;
  L->chunk_tokens = (int32_t)chunk_tokens;
  L->max_mblk = (int32_t)max_mblk;
  L->max_tasks = (int32_t)max_tasks;
  L->tile_m = BM;
  L->tile_n1 = kTileN1;
  L->tile_n2 = kTileN2;
  L->n1_tiles = (int32_t)n1;
  L->n2_tiles = (int32_t)n2;
  size_t off = 0;
  L->header = off;
  off = align_up(off + HDR_SLOTS * 4, 256);
  // the barrier counters of the one-launch planner and of moe_layer sit at the same offset for
  // every config, so a workspace reused across configs (moe_layer_noalloc's array) keeps them
  // zero between launches
  L->layer_sync = off;
  off = align_up(off + (size_t)kLayerSyncBytes, 256);
  L->chunk_counts = off;
  off = align_up(off + (size_t)((chunks + 3) & ~3ll) * c->E * 4, 256);
  L->mblk_expert = off;
  off = align_up(off + (size_t)max_mblk * 4, 256);
  L->mblk_row0 = off;
  off = align_up(off + (size_t)max_mblk * 4, 256);
  L->mblk_rows = off;
  off = align_up(off + (size_t)max_mblk * 4, 256);
  L->mblk_ready = off;
  off = align_up(off + (size_t)max_mblk * 4, 256);
  L->tasks = off;
  off = align_up(off + (size_t)max_tasks * 4, 256);
  L->unit_start = off;
  off = align_up(off + ((size_t)max_tasks + 1) * 4, 256);
  L->group_units = off;
  off = align_up(off + (size_t)max_tasks * 4, 256);
  // group record lists: kUnit slots per unit; a run of t tiles has ceil(t / kUnit) units and
  // there are at most 2 E runs (each wave's Linear-1 and Linear-2 tiles)
  const long long max_slots = (max_tasks + kUnit - 1) / kUnit * kUnit + 2ll * kUnit * c->E;
  L->max_slots = (int32_t)max_slots;
  L->group_tasks = off;
  off = align_up(off + (size_t)max_slots * 16, 256);
  L->defer_slots = off;
  off = align_up(off + (size_t)kDeferSlots * 32, 256);
  L->wave_table = off;
  off = align_up(off + ((size_t)kWaveTableHead + 10 * ((size_t)c->E + 1)) * 4, 256);
  L->total_bytes = off;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_burst_clock_hz(int64_t* hz) {
  if (!hz) return MOE_ERR_INVALID_ARG;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return MOE_ERR_HIP;
  *hz = (int64_t)khz * 1000;
  return MOE_OK;
}

moe_status moe_burst_gap(const moe_burst_cfg* c, void* buf, size_t buf_bytes, int64_t* times, void* stream) {
  if (!c || !buf || !times) return MOE_ERR_INVALID_ARG;
  if (c->reserved0 != 0 || c->periods < 1 || c->periods > 65536) return MOE_ERR_INVALID_ARG;
  if (c->bytes < 4096 || c->bytes % 4096 != 0 || c->bytes > (1 << 30)) return MOE_ERR_INVALID_ARG;
  if (c->gap_ticks < 0 || c->gap_ticks > 1000000) return MOE_ERR_INVALID_ARG;
  if (c->producers < 1) return MOE_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
  if (c->producers > cus) return MOE_ERR_INVALID_ARG;
  const size_t region = buf_bytes / (size_t)c->producers / (size_t)c->bytes * (size_t)c->bytes;
  if (region < (size_t)c->bytes) return MOE_ERR_INVALID_ARG;
  if (launch_burst_gap(static_cast<uint8_t*>(buf), region, c->producers, c->bytes, c->periods, (long long)c->gap_ticks,
                       reinterpret_cast<long long*>(times), static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

const char* moe_strerror(moe_status s) {
  switch (s) {
    case MOE_OK: return "success";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace too small or not filled by moe_plan";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "Linear-2 tile timed out waiting for its Linear-1 rows";
    default: return "unknown status";
  }
}

moe_status moe_workspace_layout(const moe_config* cfg, moe_ws_layout* layout) {
  if (!layout) return MOE_ERR_INVALID_ARG;
  return compute_layout(cfg, layout);
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_ws_layout L;
  moe_status st = compute_layout(cfg, &L);
  if (st == MOE_OK) *bytes = L.total_bytes;
  return st;
}

namespace {
// The planner's arguments for cfg (validated) and a workspace laid out as L.
void fill_plan_args(const moe_config* cfg, const moe_ws_layout& L, const float* logits, const moe_routing* rt,
                    void* ws, PlanArgs& a) {
  a.logits = logits;
  a.topk_ids = rt->topk_ids;
  a.topk_w = rt->topk_w;
  a.counts = rt->counts;
  a.offsets = rt->offsets;
  a.perm = rt->perm;
  a.pos = rt->pos;
  a.hdr = at<int32_t>(ws, L.header);
  a.chunk_counts = at<int32_t>(ws, L.chunk_counts);
  a.mb_expert = at<int32_t>(ws, L.mblk_expert);
  a.mb_row0 = at<int32_t>(ws, L.mblk_row0);
  a.mb_rows = at<int32_t>(ws, L.mblk_rows);
  a.mb_ready = at<int32_t>(ws, L.mblk_ready);
  a.tasks = at<int32_t>(ws, L.tasks);
  a.unit_start = at<int32_t>(ws, L.unit_start);
  a.group_units = at<int32_t>(ws, L.group_units);
  a.gtasks = at<int32_t>(ws, L.group_tasks);
  a.wtab = at<int32_t>(ws, L.wave_table);
  a.max_units = L.max_tasks;
  a.T = cfg->T;
  a.E = cfg->E;
  a.k = cfg->k;
  a.chunks = L.chunks;
  a.cstride = (L.chunks + 3) & ~3;
  a.chunk_tokens = L.chunk_tokens;
  a.W = cfg->experts_per_wave > cfg->E ? cfg->E : cfg->experts_per_wave;
  a.schedule = cfg->schedule;
  a.lead = cfg->lead_waves;
  a.tile_m = L.tile_m;
  a.n1 = L.n1_tiles;
  a.n2 = L.n2_tiles;
  a.H = cfg->H;
  a.I = cfg->I;
  a.wide_tails = plan_wide_tails(cfg, L.tile_m) ? 1 : 0;
  a.xs_issue_s = (cfg->xs_issue_us > 0.f ? (double)cfg->xs_issue_us : kLocalIssueUs) * 1e-6;
  a.xs_drain_bps = (cfg->xs_drain_gbps > 0.f ? (double)cfg->xs_drain_gbps : kLocalDrainGBps) * 1e9;
  a.xs_capacity_b = (cfg->xs_capacity_mib > 0.f ? (double)cfg->xs_capacity_mib : kLocalCapacityMiB) * 1048576.0;
}

moe_status plan_impl(const moe_config* cfg, const float* logits, const moe_routing* rt, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_ws_layout L;
  moe_status st = compute_layout(cfg, &L);
  if (st != MOE_OK) return st;
  if (!logits || !rt || !ws || !rt->topk_ids || !rt->topk_w || !rt->counts || !rt->offsets || !rt->perm ||
      !rt->pos)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total_bytes) return MOE_ERR_WORKSPACE;
  PlanArgs a;
  fill_plan_args(cfg, L, logits, rt, ws, a);
  if (gemm_grid(L.tile_m, a.wide_tails != 0, cfg->num_workgroups, &a.grid) != hipSuccess) return MOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg->flags & MOE_FLAG_PLAN_ONE_LAUNCH) {
    // the grid barrier waits only for resident workgroups to arrive (cfg->spin_limit bounds the
    // Linear-2 tiles' waits): the default bound
    if (launch_plan(a, at<int32_t>(ws, L.layer_sync), kDefaultSpinLimit, s) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
  }
  if (launch_route_hist(a, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_scan_schedule(a, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_scatter(a, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}
}  // namespace

moe_status moe_plan(const moe_config* cfg, const float* logits, const moe_routing* rt, void* ws,
                    size_t ws_bytes, void* stream) {
  return plan_impl(cfg, logits, rt, ws, ws_bytes, stream);
}

moe_status moe_dispatch(const moe_config* cfg, const moe_routing* rt, const uint16_t* x, uint16_t* xd,
                        void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!rt || !rt->pos || !x || !xd) return MOE_ERR_INVALID_ARG;
  if (launch_dispatch(rt->pos, x, xd, cfg->T, cfg->H, cfg->k, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

namespace {
// The persistent GEMM's arguments for cfg (validated) and a workspace laid out as L: rows from
// xd, or (xd NULL) from x through perm.
void fill_gemm_args(const moe_config* cfg, const moe_ws_layout& L, const uint16_t* xd, const uint16_t* x,
                    const int32_t* perm, const uint16_t* w1, const uint16_t* w2, uint16_t* act, uint16_t* yd,
                    void* ws, GemmArgs& g) {
  g.xd = xd;
  g.x = x;
  g.perm = perm;
  g.T = cfg->T;
  g.k = cfg->k;
  g.gather = xd ? 0 : 1;
  g.w1 = w1;
  g.w2 = w2;
  g.act = act;
  g.yd = yd;
  g.hdr = at<int32_t>(ws, L.header);
  g.tasks = at<int32_t>(ws, L.tasks);
  g.gtasks = at<int32_t>(ws, L.group_tasks);
  g.ngroups = 1;  // the launcher picks the group count from the grid it launches
  g.mb_expert = at<int32_t>(ws, L.mblk_expert);
  g.mb_row0 = at<int32_t>(ws, L.mblk_row0);
  g.mb_rows = at<int32_t>(ws, L.mblk_rows);
  g.mb_ready = at<int32_t>(ws, L.mblk_ready);
  g.R = cfg->T * cfg->k;
  g.H = cfg->H;
  g.I = cfg->I;
  g.E = cfg->E;
  g.n1 = L.n1_tiles;
  g.max_tasks = L.max_tasks;
  g.max_slots = L.max_slots;
  g.max_mblk = L.max_mblk;
  g.spin_limit = cfg->spin_limit > 0 ? cfg->spin_limit : kDefaultSpinLimit;
  g.force_timeout = (cfg->flags & MOE_FLAG_FORCE_WAIT_TIMEOUT) ? 1 : 0;
  g.absent_group = (cfg->flags & MOE_FLAG_TEST_ABSENT_GROUP) ? 0 : -1;
  g.defer = at<int32_t>(ws, L.defer_slots);
  g.trace = static_cast<moe_trace_rec*>(cfg->trace);
}
}  // namespace

namespace {
// shared by moe_forward (rows from xd) and moe_forward_gather (rows from x through perm)
moe_status forward_impl(const moe_config* cfg, const uint16_t* xd, const uint16_t* x, const int32_t* perm,
                        const uint16_t* w1, const uint16_t* w2, uint16_t* act, uint16_t* yd, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_ws_layout L;
  moe_status st = compute_layout(cfg, &L);
  if (st != MOE_OK) return st;
  if ((!xd && !(x && perm)) || !w1 || !w2 || !act || !yd || !ws) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total_bytes) return MOE_ERR_WORKSPACE;
  GemmArgs g;
  fill_gemm_args(cfg, L, xd, x, perm, w1, w2, act, yd, ws, g);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_gemm(g, L.tile_m, plan_wide_tails(cfg, L.tile_m), cfg->num_workgroups, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}
}  // namespace

moe_status moe_forward(const moe_config* cfg, const uint16_t* xd, const uint16_t* w1, const uint16_t* w2,
                       uint16_t* act, uint16_t* yd, void* ws, size_t ws_bytes, void* stream) {
  if (!xd) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, xd, nullptr, nullptr, w1, w2, act, yd, ws, ws_bytes, stream);
}

moe_status moe_forward_gather(const moe_config* cfg, const moe_routing* rt, const uint16_t* x, const uint16_t* w1,
                              const uint16_t* w2, uint16_t* act, uint16_t* yd, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!rt || !rt->perm || !x) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, nullptr, x, rt->perm, w1, w2, act, yd, ws, ws_bytes, stream);
}

moe_status moe_layer(const moe_config* cfg, const float* logits, const moe_routing* rt, const uint16_t* x,
                     const uint16_t* w1, const uint16_t* w2, uint16_t* act, uint16_t* yd, uint16_t* out, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_ws_layout L;
  moe_status st = compute_layout(cfg, &L);
  if (st != MOE_OK) return st;
  if (!logits || !rt || !rt->topk_ids || !rt->topk_w || !rt->counts || !rt->offsets || !rt->perm || !rt->pos ||
      !x || !w1 || !w2 || !act || !yd || !out || !ws)
    return MOE_ERR_INVALID_ARG;
  if (cfg->trace) return MOE_ERR_INVALID_ARG;  // the traced instances are the separate forward calls'
  if (ws_bytes < L.total_bytes) return MOE_ERR_WORKSPACE;
  LayerArgs la;
  fill_plan_args(cfg, L, logits, rt, ws, la.pl);
  la.pl.wide_tails = 0;  // the single launch runs regular tiles (the same bytes as wide ones)
  const bool wide = false;
  if (gemm_grid(L.tile_m, wide, cfg->num_workgroups, &la.pl.grid) != hipSuccess) return MOE_ERR_HIP;
  // the schedule step runs on one workgroup of the GEMM's size: with more than 64 expert
  // waves it takes one thread per wave
  const int nw = (cfg->E + la.pl.W - 1) / la.pl.W;
  const int nt = L.tile_m == 256 ? 512 : 256;
  if (nw > 64 && nw > nt) return MOE_ERR_UNSUPPORTED;
  fill_gemm_args(cfg, L, nullptr, x, rt->perm, w1, w2, act, yd, ws, la.g);
  la.topk_w = rt->topk_w;
  la.pos = rt->pos;
  la.out = out;
  la.segs = combine_segments(cfg->T, cfg->H);
  la.sync = at<int32_t>(ws, L.layer_sync);
  if (launch_layer(la, L.tile_m, wide, cfg->num_workgroups, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

namespace {
// Device address of this GPU's scratch array, looked up once per device (with that device
// current) and kept; later calls on the device reuse it.
moe_status scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}
}  // namespace

moe_status moe_layer_noalloc(const moe_config* cfg, const float* logits, const moe_routing* rt,
                             const uint16_t* x, const uint16_t* w1, const uint16_t* w2, uint16_t* act,
                             uint16_t* yd, uint16_t* out, int32_t* status, void* stream) {
  moe_ws_layout L;
  moe_status st = compute_layout(cfg, &L);
  if (st != MOE_OK) return st;
  if (L.total_bytes > (size_t)MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
  // the traced GEMM instances are a measurement aid and may use private (scratch) memory
  if (cfg->trace) return MOE_ERR_INVALID_ARG;
  if (!logits || !rt || !rt->topk_ids || !rt->topk_w || !rt->counts || !rt->offsets || !rt->perm || !rt->pos ||
      !x || !w1 || !w2 || !act || !yd || !out)
    return MOE_ERR_INVALID_ARG;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MOE_OK) return st;
  // moe_plan initialises every part of the workspace the later kernels read (header, cursors,
  // dependency counters, tile lists), so the array's contents from an earlier call do not
  // matter; the GEMM's last workgroup resets its counters again on exit
  if ((st = plan_impl(cfg, logits, rt, ws, MOE_STATIC_WORKSPACE_BYTES, stream)) != MOE_OK) return st;
  if ((st = forward_impl(cfg, nullptr, x, rt->perm, w1, w2, act, yd, ws, MOE_STATIC_WORKSPACE_BYTES, stream)) !=
      MOE_OK)
    return st;
  if ((st = moe_combine(cfg, rt, yd, out, stream)) != MOE_OK) return st;
  // the device-side error word (header slot 0) for the caller, a 4-byte device-to-device copy
  if (status && hipMemcpyAsync(status, at<int32_t>(ws, L.header) + HDR_ERROR, sizeof(int32_t),
                               hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_combine(const moe_config* cfg, const moe_routing* rt, const uint16_t* yd, uint16_t* out,
                       void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!rt || !rt->pos || !rt->topk_w || !yd || !out) return MOE_ERR_INVALID_ARG;
  if (launch_combine(rt->pos, rt->topk_w, yd, out, cfg->T, cfg->H, cfg->k, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_status_read(const void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < HDR_SLOTS * 4) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  int32_t code = 0;
  if (hipMemcpy(&code, ws, sizeof(code), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  return code == 0 ? MOE_OK : (moe_status)code;
}

}  // extern "C"
