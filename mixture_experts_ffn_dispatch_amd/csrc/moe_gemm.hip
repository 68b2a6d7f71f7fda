// Persistent grouped GEMM of libmoe (gfx950): every expert's Linear-1 with a fused SwiGLU
// epilogue and its Linear-2, as one launch that walks the tile list moe_plan wrote.
//
// X-Stage paper, Introduction: each expert evaluates Linear-1 (H -> 2I), SwiGLU, Linear-2
// (I -> H); MegaMoE runs these stages inside one persistent kernel, grouped into expert waves,
// and Section 4.2 reorders independent Linear-1 / Linear-2 tiles across waves. Here:
//
//  * A workgroup (8 wavefronts for 256-row tiles, 4 for smaller ones) takes the next tile of
//    its XCD group's part of the list (one atomic on the group's cursor, then the tile's
//    record), so each group's tiles start in list order whatever the grid size.
//  * Linear-1 tile (expert e, m-block, n-tile): 128 gate rows + the matching 128 up rows of
//    W1[e] against up to tile_m dispatched rows; the epilogue forms
//    A = bf16(silu(gate) * up) for 128 columns; the m-block's ready counter is released (two
//    Linear-1 tiles at a time when the interleave lead is two waves or more, and always before
//    the workgroup takes a Linear-2 tile or exits).
//  * Linear-2 tile: waits (bounded) until all Linear-1 tiles of its m-block have released,
//    then multiplies those A rows by 256 rows of W2[e] and stores Yd in bf16.
//  * Wide last m-blocks (a second instance of the 256-row kernel, when asked for): an m-block of
//    at most 128 rows runs as tiles of twice the weight rows by 128 token rows, so an expert's
//    short last block needs half the tiles and puts no padding rows through the MFMAs.
//  * The MFMA A operand is the weight tile and the B operand the token tile, so one lane
//    ends with four consecutive output columns of one token row; the epilogue stages them in
//    LDS and stores whole row segments (16 bytes per lane).
//  * Operands go from global memory straight into LDS (buffer->LDS loads) in 64-wide K steps,
//    double buffered, the 16-byte chunks of each row XOR-swizzled so that 128-bit fragment
//    reads are free of bank conflicts.
//  * Every output element accumulates its K products in the same order (ascending K steps of
//    16 inside one v_mfma_f32_32x32x16_bf16 chain), so tile order, grid size and tile height
//    never change a result bit.
//  * Loads and stores use buffer resources bounded to the m-block's rows and the expert's
//    weight slab: rows past the end read as zero and are never stored.
//  * With a trace buffer, every tile's claim, wait, main loop, epilogue and release are
//    timed with the real-time counter (Section 5 of the paper instruments its kernel per tile
//    the same way); without one, none of it runs.
#include "moe_combine_dev.h"
#include "moe_internal.h"
#include "moe_plan_dev.h"
#include "moe_sync_dev.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
// cache-policy operand of gfx950 buffer instructions: sc1 (device scope), nt (streaming:
// the lines are not kept for reuse)
constexpr int kCachePolicySC1 = 16;
constexpr int kCachePolicyNT = 2;
// Claim result that tells the workgroup to release the completions it holds and claim again:
// given when its own group's list runs out, so the holds are not kept through the scan of the
// other groups' cursors (one atomic each). Never a task: m-block 0x7FFFF is out of range.
constexpr int32_t kFlushTask = 0x7FFFFFFD;

// The constant-rate real-time counter (its frequency is the device's wall-clock rate).
__device__ inline long long rt_clock() { return (long long)__builtin_amdgcn_s_memrealtime(); }
__device__ inline int hw_xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & 0xFu);
}
__device__ inline int hw_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
  return (int)v;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kRsrcWord3);
}

// 16 bytes per lane from a buffer straight into LDS: lane L's bytes land at lds_dst + 16 L
// (lds_dst is the same for the whole wavefront); voffset and soffset address the buffer only.
// POLICY: the cache policy (0, or kCachePolicyNT for bytes no other load reads).
template <int POLICY = 0>
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voffset, soffset, 0,
                                           POLICY);
}
// The same load as an instruction the compiler does not track: it then inserts no wait for it
// (with the builtin it waits for every such load before each barrier), so loads may stay in
// flight across barriers. The code that issues them waits for them itself (s_waitcnt vmcnt(n):
// loads complete in issue order, so n leaves the n most recent in flight).
template <bool NT = false>
__device__ inline void load_lds16_untracked(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voffset,
                                            uint32_t soffset) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst;
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voffset), "s"(r), "s"(soffset), "{m0}"(m) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voffset), "s"(r), "s"(soffset), "{m0}"(m) : "memory");
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (v_rcp_f32, about 1 ulp) instead of an
// IEEE division: the result is rounded to bf16 right after, and 1 + e^-g is exactly 1 for
// g >= 17, so silu(g) = g exactly there, as with the division. It takes 6 instead of about 14
// vector instructions for each of the 64 outputs a lane forms in a Linear-1 epilogue.
__device__ inline float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// LDS swizzle of a 128-byte operand row: its eight 16-byte chunks are permuted by XOR with
// (row & 7) ^ (bit 3 of row). Any 8 consecutive rows then put one chunk index in 8 distinct
// 16-byte slots of a 128-byte bank window, and any 16 consecutive rows in 16 distinct slots
// of a 256-byte window, so a 128-bit fragment read (32 consecutive rows, one chunk) is free of
// bank conflicts whether the LDS serves 8 or 16 lanes per cycle.
__device__ inline int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Scheduling pattern for one k-step region: NM MFMAs with NV global loads, NR LDS reads and
// NW LDS writes spread evenly between them (each MFMA followed by its share).
// LDS reads go out over the first half of the MFMAs, so they land well before their use.
template <int NM, int NV, int NR, int NW, int I = 0>
struct Interleave {
  static __device__ __forceinline__ void emit() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int NMR = NM > 1 ? NM / 2 : 1;
    constexpr int v = NV * (I + 1) / NM - NV * I / NM;
    constexpr int r = I < NMR ? NR * (I + 1) / NMR - NR * I / NMR : 0;
    constexpr int w = NW * (I + 1) / NM - NW * I / NM;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // global loads
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // LDS reads
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);  // LDS writes
    if constexpr (I + 1 < NM) Interleave<NM, NV, NR, NW, I + 1>::emit();
  }
};

// LDS of a tile shape: two stages of weight rows then token rows (64 K-columns each), and, where
// the two stages already take more than half of a CU's LDS (so one workgroup runs per CU
// anyway) and a third set of weight rows still fits, that third weight stage, so that the
// weight rows can be loaded two K steps ahead of their use (W3).
constexpr int kLdsBytes = 160 * 1024;  // LDS per CU
template <int BM, int WN, int WM, bool WIDE>
struct GemmLds {
  static constexpr bool WIDE_OK = WIDE && BM == 256 && WN == 2 && WM == 4;
  static constexpr int STAGE_BYTES = (WIDE_OK ? 2 * kTileN2 + BM / 2 : kTileN2 + BM) * kTileK * 2;
  static constexpr int WSTAGE_BYTES = kTileN2 * kTileK * 2;
  static constexpr bool W3 = !WIDE_OK && 2 * STAGE_BYTES > kLdsBytes / 2 && 2 * STAGE_BYTES + WSTAGE_BYTES <= kLdsBytes;
  static constexpr int BYTES = 2 * STAGE_BYTES + (W3 ? WSTAGE_BYTES : 0);
};

// The planner's phases of the single-launch layer, on every workgroup of the grid: route the
// token chunks (grid-stride); the last workgroup to arrive scans the counts and writes the
// schedule while the others wait for it; scatter the chunks and place the tile list; then
// all wait until every workgroup is done. lds: the kernel's LDS array (lds_elems bf16); the
// planner uses its first 54 KiB, the barrier broadcasts its last 16 bytes. Returns false when
// a wait expired: the workgroup then runs no later phase, which would read an unfinished plan.
template <int NT>
__device__ bool layer_plan_phases(const LayerArgs& f, uint16_t* lds, int lds_elems) {
  const PlanArgs& a = f.pl;
  int* const il = reinterpret_cast<int*>(lds);
  int* const bc = reinterpret_cast<int*>(lds + lds_elems) - 4;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  for (int c = b; c < a.chunks; c += G) route_chunk<NT>(a, c, il);
  if (layer_count(f.sync, kSyncArrive, kSyncAll, 1, bc)) {
    // every chunk's counts are in: this workgroup writes the schedule, then opens barrier 1
    int* const s_tmp = il;
    int* const s_cnt = il + 32;
    int* const s_tab = s_cnt + MOE_MAX_EXPERTS;
    double* const s_cost = reinterpret_cast<double*>(s_tab + ((kWaveTableLds + 1) & ~1));
    scan_schedule_block<NT>(a, s_tmp, s_cnt, s_tab, s_cost);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    layer_open(f.sync, 1);
  }
  if (!layer_wait(f.sync, 1, f.g.spin_limit, bc)) return false;
  for (int c = b; c < a.chunks; c += G) scatter_chunk<NT>(a, c, il);
  place_tiles<NT>(a, b, min(G, kPlaceBlocks), il);
  return layer_barrier(f.sync, 2, f.g.spin_limit, bc);
}

// Resets the plan's cursors and ready counters (one workgroup of NT threads), so the next
// moe_forward on this plan starts clean without a separate launch.
template <int NT>
__device__ void reset_tile_state(const GemmArgs& p) {
  const int n = min(p.hdr[HDR_NMBLK], p.max_mblk);
  for (int i = threadIdx.x; i < n; i += NT) p.mb_ready[i] = 0;
  if (threadIdx.x == 0) {
    p.hdr[HDR_CURSOR] = 0;
    for (int g = 0; g < kGroups; ++g) p.hdr[HDR_GROUP_CURSOR + g] = 0;
    p.hdr[HDR_DONE] = 0;
  }
}

// After the tile loop of the single-launch layer: wait until every workgroup has finished its
// tiles, combine (grid-stride over tokens and column segments, one wavefront per item), then
// the last workgroup out resets the barriers and the tile state for the next launch and
// reports an expired wait in the error word.
template <int NT>
__device__ void layer_finish_phases(const LayerArgs& f, uint16_t* lds, int lds_elems, bool ok) {
  int* const bc = reinterpret_cast<int*>(lds + lds_elems) - 4;
  const int G = (int)gridDim.x;
  if (ok) ok = layer_barrier(f.sync, 3, f.g.spin_limit, bc);
  if (ok) {
    constexpr int NW = NT / 64;
    combine_items<8>(f.pos, f.topk_w, f.g.yd, f.out, f.g.T, f.g.H, f.g.k, f.g.R, f.segs,
                     (int)blockIdx.x * NW + (int)(threadIdx.x >> 6), G * NW);
  } else if (threadIdx.x == 0) {
    atomicCAS(sync_line(f.sync, kSyncErr), 0, (int)MOE_ERR_TIMEOUT);
  }
  if (layer_count(f.sync, kSyncExit, kSyncAllExit, 1, bc)) {
    reset_tile_state<NT>(f.g);
    layer_sync_reset(f.sync, f.g.hdr);
  }
}

template <bool FUSED>
struct KernelArgsOf {
  using T = GemmArgs;
};
template <>
struct KernelArgsOf<true> {
  using T = LayerArgs;
};
__device__ __forceinline__ const GemmArgs& gemm_args_of(const GemmArgs& a) { return a; }
__device__ __forceinline__ const GemmArgs& gemm_args_of(const LayerArgs& a) { return a.g; }

// FUSED: the single-launch layer (the planner's phases, then the tiles, then the combine);
// otherwise the persistent GEMM alone.
template <int BM, int WN, int WM, int MINW, bool WIDE, bool TRACE, bool FUSED>
__global__ __launch_bounds__(64 * WN * WM, MINW) void gemm_persistent_kernel(typename KernelArgsOf<FUSED>::T ka) {
  const GemmArgs& p = gemm_args_of(ka);
  constexpr int BN = kTileN2;  // weight rows per tile (Linear-1: 128 gate + 128 up)
  constexpr int BK = kTileK;
  constexpr int FN = BN / WN / 32;  // 32x32 MFMA blocks per wave along weight rows
  constexpr int FM = BM / WM / 32;  // ... along token rows
  constexpr int NT = 64 * WN * WM;  // threads
  constexpr int RG = NT / 8;        // operand rows staged per thread-wide step (8 chunks a row)
  // Wide tiles (the WIDE instance of the 256-row variant): an m-block of at most BM / 2 rows is
  // run as one tile of 2 BN weight rows by BM / 2 token rows, the wavefronts arranged
  // 2 WN x WM / 2, so that every wavefront keeps its (BN / WN) x (BM / WM) block, its fragments
  // and its MFMA chain. The capability costs about 1% on regular tiles, so the other instance
  // leaves it out.
  constexpr bool WIDE_OK = WIDE && BM == 256 && WN == 2 && WM == 4;
  constexpr int ROWS = WIDE_OK ? 2 * BN + BM / 2 : BN + BM;  // LDS rows per stage (weights, then tokens)
  constexpr int STAGE = ROWS * BK;  // bf16 elements per stage
  constexpr int LD = ROWS / RG;     // 16-byte chunks a thread may stage per K step
  constexpr int LDN = BN / RG;      // of them weight chunks of a regular tile
  static_assert(FN % 2 == 0 && FN >= 2 && FM >= 1, "tile shape");
  static_assert(BM % RG == 0 && BN % (2 * RG) == 0 && RG % 16 == 0, "staging groups");
  static_assert(BN % 32 == 0 && BM % 32 == 0, "tile shape");
  static_assert(!WIDE_OK || (LD == LDN + BM / RG + 2 && (BM / 2) % RG == 0), "wide staging");
  // W3: weight rows three-buffered. The LDS then holds [W0 T0 W1 T1 W2] (W: BN weight rows, T: BM
  // token rows); token rows keep two stages, K step kt's weight rows sit in W(kt mod 3).
  constexpr bool W3 = GemmLds<BM, WN, WM, WIDE>::W3 && !FUSED;
  constexpr int LDS_ELEMS = W3 ? GemmLds<BM, WN, WM, WIDE>::BYTES / 2 : 2 * STAGE;
  static_assert(GemmLds<BM, WN, WM, WIDE>::STAGE_BYTES == 2 * STAGE && (!W3 || LDN + BM / RG == LD), "LDS layout");

  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  // The tile record, its record slot, the resume and defer flags and the exit flag live at the
  // start of the first LDS stage the mainloop writes after its prologue barrier (stage 1, or
  // W2): every wave passes that barrier after reading them.
  int* const s_task = reinterpret_cast<int*>(&lds[W3 ? 2 * STAGE : STAGE]);
  int* const s_last = s_task + 5;
  // per-tile trace: only the TRACE instances (launched when a trace buffer is given) hold
  // any of its code, so the others are unchanged by it
  constexpr bool tracing = TRACE;
  // the single-launch layer plans first; the tile loop reads the header the plan writes
  bool plan_ok = true;
  if constexpr (FUSED) plan_ok = layer_plan_phases<64 * WN * WM>(ka, lds, LDS_ELEMS);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = tid >> 3, lchunk = tid & 7;  // staging: row within an RG-row group, LDS chunk slot
  const int lds_pchunk = lchunk ^ swz(lrow);    // swizzled chunk (rows RG apart swizzle alike)
  const int fr_row = lane & 31, fr_chunk = lane >> 5;

  const uint32_t yd_bytes = (uint32_t)((size_t)p.R * p.H * 2);
  const uint32_t act_bytes = (uint32_t)((size_t)p.R * p.I * 2);
  const __amdgpu_buffer_rsrc_t r_yd = make_rsrc(p.yd, yd_bytes);
  const __amdgpu_buffer_rsrc_t r_act = make_rsrc(p.act, act_bytes);

  // tile source: one shared cursor over the list, or (with kGroups groups) this workgroup's
  // group list of tile records first, then the other groups' lists in turn. Each group walks
  // its records in list order, so every tile a Linear-2 tile waits for is taken before it by a
  // workgroup that never waits on a later tile. A claim is one atomic on the group's cursor
  // (the list bounds load alongside it) and one 16-byte record load.
  const int my_group = (int)(blockIdx.x % (unsigned)p.ngroups);
  int scan_group = 0;  // thread 0 only: groups whose lists are used up
  // Linear-1 completions are released in batches of kReleaseBatch: one drain of the stores and
  // one agent-scope release (an L2 write-back) for several m-block counters. A workgroup holds
  // completions only while it runs Linear-1 tiles, which never wait; it releases them before
  // any Linear-2 tile (which may wait), before it exits, and when its own group's list runs
  // out, so no wait depends on a held one and none outlasts the scan of the other groups.
  // Holding delays a release by up to one Linear-1 tile, which costs nothing only when the
  // Linear-2 tiles that wait for it lie a whole wave later in the list: an interleaved order
  // with a lead of at least two waves. Otherwise every completion is released at once.
  const int batch = p.hdr[HDR_LEAD] >= 2 ? kReleaseBatch : 1;
  // Progress without every group resident. A Linear-2 tile can wait for Linear-1 tiles in
  // another group's list, which only that group's workgroups take until their own lists run
  // out. If a group has no resident workgroup (a kernel running concurrently keeps its XCD
  // busy), such a wait would last until the bounded wait expires. So a Linear-2 tile whose
  // m-block is not ready after kDeferTicks (far longer than any wait with every group
  // resident) is set aside in the workgroup's deferral slot, and the workgroup then runs only
  // tiles that cannot wait: the first unclaimed record of any group's list if it is a
  // Linear-1 tile or a ready Linear-2 tile (a compare-and-swap on that group's cursor),
  // releasing each Linear-1 completion at once, until the deferred tile is ready. The
  // earliest unfinished tile of the whole list is then always running, or deferred and ready,
  // or first in its group's list and runnable, so a single resident workgroup finishes the
  // list. Only the group lists need it (a shared cursor hands out the list in order).
  bool have_def = false;             // a deferred Linear-2 tile waits in this workgroup's slot
  int npend = 0;                     // completions held (the same value in every lane)
  int pend_mb[kReleaseBatch] = {};  // thread 0: their m-blocks
  int pend_slot[kReleaseBatch] = {};  // thread 0: their trace records
  auto release = [&]() {
    // every wavefront drains its own stores first (a workgroup barrier alone does not wait
    // for them), then one lane releases at agent scope and bumps the counters
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if constexpr (tracing) {
        const long long t = rt_clock();
#pragma unroll
        for (int i = 0; i < kReleaseBatch; ++i)
          if (i < npend) p.trace[pend_slot[i]].t_release = t;
      }
#pragma unroll
      for (int i = 0; i < kReleaseBatch; ++i)
        if (i < npend) __hip_atomic_fetch_add(&p.mb_ready[pend_mb[i]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    npend = 0;
  };
  // MOE_FLAG_TEST_ABSENT_GROUP: this group's workgroups take no tile
  const bool absent = p.ngroups > 1 && my_group == p.absent_group;
  for (;;) {
    if constexpr (FUSED) {
      if (!plan_ok) break;  // a barrier expired: the plan may be unfinished
    }
    if (absent) break;
    long long t_claim = 0;
    if constexpr (tracing) t_claim = rt_clock();
    if (tid == 0) {
      i32x4 rec = {kNoTask, -1, 0, 0};  // task word, expert, first row, rows
      int slot = -1;                    // its trace record: the list position or record slot
      int resumed = 0;                  // 1: the deferred tile, ready; 2: its wait expired
      if (have_def) {
        int* const def = p.defer + 8 * blockIdx.x;
        const i32x4 d = {__hip_atomic_load(def, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         __hip_atomic_load(def + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         __hip_atomic_load(def + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         __hip_atomic_load(def + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
        const int dslot = __hip_atomic_load(def + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // whether a Linear-2 record's m-block has all its Linear-1 releases
        auto ready = [&](const i32x4& r) {
          const int m = (r[0] >> kTaskMblkShift) & ((1 << kTaskMblkBits) - 1);
          if (m >= p.max_mblk) return true;  // malformed: the tile's own checks reject it
          const int need = ((WIDE_OK && (r[3] & kRowsWide)) ? (p.n1 + 1) / 2 : p.n1) + p.force_timeout;
          return __hip_atomic_load(&p.mb_ready[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need;
        };
        for (int spins = 0;; ++spins) {
          if (ready(d)) {
            rec = d;
            slot = dslot;
            resumed = 1;
            break;
          }
          bool got = false;
          for (int h = 0; h < p.ngroups && !got; ++h) {
            const int g = (my_group + h) % p.ngroups;
            int* const cur = &p.hdr[HDR_GROUP_CURSOR + g];
            const int lo = max(p.hdr[HDR_GTASK_OFF + g], 0), hi = min(p.hdr[HDR_GTASK_OFF + g + 1], p.max_slots);
            int c = __hip_atomic_load(cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            while (c >= 0 && c < hi - lo) {
              const i32x4 r = *reinterpret_cast<const i32x4*>(p.gtasks + 4 * (size_t)(lo + c));
              if (r[0] != kNopTask && ((unsigned)r[0] >> kTaskL2Bit) != 0u && !ready(r)) break;
              if (__hip_atomic_compare_exchange_strong(cur, &c, c + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)) {
                if (r[0] == kNopTask) {  // a spare slot: the next record
                  ++c;
                  continue;
                }
                rec = r;
                slot = lo + c;
                got = true;
                break;
              }
              // the cursor moved: c holds its new value
            }
          }
          if (got) break;
          if (spins >= p.spin_limit) {  // run it anyway, as an expired wait does
            atomicCAS(&p.hdr[HDR_ERROR], 0, (int)MOE_ERR_TIMEOUT);
            rec = d;
            slot = dslot;
            resumed = 2;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      } else if (p.ngroups == 1) {
        const int ntasks = min(p.hdr[HDR_NTASKS], p.max_tasks);
        for (;;) {
          const int t = atomicAdd(&p.hdr[HDR_CURSOR], 1);
          if (t < 0 || t >= ntasks) break;
          slot = t;
          rec[0] = p.tasks[t];
          const int mb = (rec[0] >> kTaskMblkShift) & ((1 << kTaskMblkBits) - 1);
          if (mb < p.max_mblk) {  // the m-block record is read only for an index inside the table
            rec[1] = p.mb_expert[mb];
            rec[2] = p.mb_row0[mb];
            rec[3] = p.mb_rows[mb];
          }
          // the odd n-tiles of a wide m-block are covered by the even ones: claim again
          if (!((rec[3] & kRowsWide) && (rec[0] & 1))) break;
          rec = i32x4{kNoTask, -1, 0, 0};
        }
      } else {
        while (scan_group < p.ngroups) {
          const int g = (my_group + scan_group) % p.ngroups;
          const int i = atomicAdd(&p.hdr[HDR_GROUP_CURSOR + g], 1);
          const int lo = max(p.hdr[HDR_GTASK_OFF + g], 0), hi = min(p.hdr[HDR_GTASK_OFF + g + 1], p.max_slots);
          if (i >= 0 && i < hi - lo) {
            slot = lo + i;
            rec = *reinterpret_cast<const i32x4*>(p.gtasks + 4 * (size_t)(lo + i));
            if (rec[0] != kNopTask) break;
            rec = i32x4{kNoTask, -1, 0, 0};  // a spare slot: claim again
            continue;
          }
          ++scan_group;  // this group's list is used up
          if (npend > 0) {  // publish held completions before scanning the other groups
            rec = i32x4{kFlushTask, -1, 0, 0};
            break;
          }
        }
      }
      s_task[0] = rec[0];
      s_task[1] = rec[1];
      s_task[2] = rec[2];
      s_task[3] = rec[3];
      s_task[4] = slot;
      s_task[6] = resumed;
    }
    __syncthreads();
    long long t_claimed = 0;
    if constexpr (tracing) t_claimed = rt_clock();
    // the task and its m-block record are the same for the whole workgroup: keep them scalar
    const int task = __builtin_amdgcn_readfirstlane(s_task[0]);
    if (npend > 0 && (task == kNoTask || ((unsigned)task >> kTaskL2Bit) != 0u)) release();
    if (task == kNoTask) break;
    if (task == kFlushTask) {
      release();
      continue;
    }
    const bool l2 = ((unsigned)task >> kTaskL2Bit) != 0u;
    const int mb = (task >> kTaskMblkShift) & ((1 << kTaskMblkBits) - 1);
    const int nt = task & kTaskNtMask;
    const int e = __builtin_amdgcn_readfirstlane(s_task[1]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_task[2]);
    const int rows_word = __builtin_amdgcn_readfirstlane(s_task[3]);
    const int slot = __builtin_amdgcn_readfirstlane(s_task[4]);
    const int resumed = __builtin_amdgcn_readfirstlane(s_task[6]);
    if (resumed) have_def = false;
    const bool wide = WIDE_OK && (rows_word & kRowsWide) != 0;
    // the expert's only m-block: its weight rows are read by this tile alone
    const bool w_nt = (rows_word & kRowsOnce) != 0;
    const int nrows = rows_word & ~kRowsFlags;
    // a plan this workspace could not have produced: skip the tile, report, never fault
    if (mb >= p.max_mblk || (unsigned)e >= (unsigned)p.E || row0 < 0 || nrows < 1 || row0 > p.R - nrows ||
        nt >= (l2 ? (p.H + kTileN2 - 1) / kTileN2 : p.n1) || (rows_word & kRowsWide && !WIDE_OK) ||
        (wide && (nrows > BM / 2 || (nt & 1)))) {
      if (tid == 0) atomicCAS(&p.hdr[HDR_ERROR], 0, (int)MOE_ERR_WORKSPACE);
      __syncthreads();
      continue;
    }
    const int K = l2 ? p.I : p.H;

    // tile geometry: weight rows and token rows in LDS, and this wavefront's place in the grid
    const int bn = wide ? 2 * BN : BN;
    const int bm = wide ? BM / 2 : BM;
    const int wn = wide ? wave % (2 * WN) : wave % WN;
    const int wm = wide ? wave / (2 * WN) : wave / WN;

    if (l2) {
      if (tid == 0) {
        // every Linear-1 tile of the m-block releases once; a wide m-block has half as many
        const int need = (wide ? (p.n1 + 1) / 2 : p.n1) + p.force_timeout;
        // a tile may be set aside once (not a resumed one, and one at a time)
        const bool may_defer = p.ngroups > 1 && !have_def && resumed == 0 && blockIdx.x < (unsigned)kDeferSlots;
        const long long t_wait = may_defer ? rt_clock() : 0;
        int spins = 0, defer_now = 0;
        while (__hip_atomic_load(&p.mb_ready[mb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++spins > p.spin_limit) {
            atomicCAS(&p.hdr[HDR_ERROR], 0, (int)MOE_ERR_TIMEOUT);
            break;
          }
          if (may_defer && rt_clock() - t_wait > kDeferTicks) {
            int* const def = p.defer + 8 * blockIdx.x;
            *reinterpret_cast<i32x4*>(def) = i32x4{task, e, row0, rows_word};
            def[4] = slot;
            defer_now = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
        s_task[7] = defer_now;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(s_task[7])) {
        have_def = true;
        continue;
      }
    }
    if (tracing && tid == 0 && (unsigned)slot < (unsigned)p.max_slots) {
      // the record's head now, its tail after the epilogue: no reading is kept through the
      // main loop (one lane, vector stores)
      moe_trace_rec* const r = &p.trace[slot];
      *reinterpret_cast<i32x4*>(&r->task) = i32x4{task, (int)blockIdx.x, hw_xcc_id(), hw_id()};
      r->t_claim = t_claim;
      r->t_claimed = t_claimed;
      r->t_start = rt_clock();
    }

    // operand buffers bounded to this expert's weight slab and this m-block's rows
    __amdgpu_buffer_rsrc_t r_w, r_t;
    if (l2) {
      r_w = make_rsrc(p.w2 + (size_t)e * p.H * p.I, (uint32_t)((size_t)p.H * p.I * 2));
      r_t = make_rsrc(p.act + (size_t)row0 * p.I, (uint32_t)((size_t)nrows * p.I * 2));
    } else {
      r_w = make_rsrc(p.w1 + (size_t)e * 2 * p.I * p.H, (uint32_t)((size_t)2 * p.I * p.H * 2));
      r_t = p.gather ? make_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * 2))
                     : make_rsrc(p.xd + (size_t)row0 * p.H, (uint32_t)((size_t)nrows * p.H * 2));
    }
    // staged chunk i of this thread: weight rows for i < BN/RG (per-lane base + wave-uniform
    // row offset), token rows after (one per-lane offset per row group)
    const uint32_t rowb = (uint32_t)K * 2u;  // bytes per operand row
    // the buffer->LDS load puts lane L's 16 bytes at slot L of the wave's 1 KiB, so the global
    // side applies the swizzle: the lane owning LDS chunk slot p of row r loads chunk p ^ swz(r)
    const uint32_t gchunk = (uint32_t)lds_pchunk;
    const uint32_t vbase_w = (uint32_t)((l2 ? nt * kTileN2 : nt * kTileN1) + lrow) * rowb + gchunk * 16u;
    // token rows lrow + RG j: contiguous rows of the m-block, or (Linear-1 with gather) row
    // perm[r] / k of x, the dispatch folded into the load; rows past the m-block, or with a
    // routing entry out of range, get an offset outside the buffer and read as zero
    constexpr int TG = BM / RG;
    uint32_t vtok[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      const int r = lrow + RG * j;
      if (p.gather && !l2) {
        int src = -1;
        if (r < nrows) {
          const int f = p.perm[row0 + r];
          src = (unsigned)f < (unsigned)p.R ? f / p.k : -1;
        }
        vtok[j] = src >= 0 ? (uint32_t)src * rowb + gchunk * 16u : 0x80000000u;
      } else {
        vtok[j] = (uint32_t)r * rowb + gchunk * 16u;
      }
    }
    const uint32_t up_off = l2 ? 0u : (uint32_t)p.I * rowb;  // Linear-1: up rows follow the gate rows
    auto chunk_soff = [&](int i) -> uint32_t {
      if (l2) return (uint32_t)i * RG * rowb;
      const int half = bn / (2 * RG);  // chunks of gate rows
      return i < half ? (uint32_t)i * RG * rowb : up_off + (uint32_t)(i - half) * RG * rowb;
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // LDS row of each weight fragment (Linear-1: first half gate, second half the matching up)
    int wrow[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if (l2) wrow[f] = wn * (BN / WN) + f * 32;
      else
        wrow[f] = (f < FN / 2) ? wn * (BN / 2 / WN) + f * 32 : bn / 2 + wn * (BN / 2 / WN) + (f - FN / 2) * 32;
    }

    // Mainloop, software-pipelined by hand. Per K step of 64 (four MFMA k-steps of 16):
    //   the next K step's operands go straight into the other LDS stage (buffer->LDS loads);
    //   with W3, the next K step's token rows and the weight rows of the one after it
    //   k-step 0 MFMAs | fragments of k-step 1
    //   k-step 1 MFMAs | fragments of k-step 2
    //   k-step 2 MFMAs | fragments of k-step 3
    //   k-step 3 MFMAs
    //   wait for this wave's loads (with W3, all but the weight rows two steps ahead), barrier
    //   (the next K step's operands are complete, this step's stages free), then fragments of
    //   the next K step's k-step 0
    // Fragments alternate between two register sets so that reads for k-step s + 1 are in
    // flight while the MFMAs of k-step s run; the sched_group_barrier patterns keep the
    // compiler from sinking the reads next to their first use.
    bf16x8 fa[2][FN], fb[2][FM];
    const int KT = K / BK;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // K step kt straight into LDS stage st: wave w fills rows 8w + RG i, eight rows (1 KiB) a
    // load. Past the last K step the offsets get bit 31 set, which is outside every buffer
    // range below 2^31 bytes: such loads fetch nothing. (A larger weight slab would read bytes
    // of its own buffer into a stage that is never used.)
    // Weight chunks come first: 0 .. LDN - 1, and LDN .. 2 LDN - 1 of a wide tile; then the
    // token chunks (LDN .. of a regular tile, 2 LDN .. of a wide one).
    auto issue_loads = [&](int kt, int st) {
      const uint32_t past = kt < KT ? 0u : 0x80000000u;
      const uint32_t vw = vbase_w | past;
      const uint32_t ks = (uint32_t)kt * BK * 2u;
      auto dst = [&](int i) -> uint16_t* { return &lds[st * STAGE + (wave_u * 8 + RG * i) * BK]; };
      auto weights = [&](auto policy) {
        constexpr int P = decltype(policy)::value;
#pragma unroll
        for (int i = 0; i < LDN; ++i) load_lds16<P>(r_w, dst(i), vw, chunk_soff(i) + ks);
        if constexpr (WIDE_OK) {
          if (wide) {
#pragma unroll
            for (int i = LDN; i < 2 * LDN; ++i) load_lds16<P>(r_w, dst(i), vw, chunk_soff(i) + ks);
          }
        }
      };
      if (w_nt) weights(std::integral_constant<int, kCachePolicyNT>{});
      else weights(std::integral_constant<int, 0>{});
      if constexpr (WIDE_OK) {
        if (wide) {
#pragma unroll
          for (int i = 2 * LDN; i < LD; ++i) load_lds16(r_t, dst(i), vtok[i - 2 * LDN] | past, ks);
          return;
        }
      }
#pragma unroll
      for (int i = LDN; i < LDN + BM / RG; ++i) load_lds16(r_t, dst(i), vtok[i - LDN] | past, ks);
    };
    // W3 (regular tiles only): K step kt's token rows into stage st, or its weight rows into
    // weight stage ws, with the untracked loads
    auto issue_tokens = [&](int kt, int st) {
      const uint32_t past = kt < KT ? 0u : 0x80000000u;
      const uint32_t ks = (uint32_t)kt * BK * 2u;
#pragma unroll
      for (int i = LDN; i < LD; ++i)
        load_lds16_untracked(r_t, &lds[st * STAGE + (wave_u * 8 + RG * i) * BK], vtok[i - LDN] | past, ks);
    };
    auto issue_weights = [&](int kt, int ws) {
      const uint32_t vw = vbase_w | (kt < KT ? 0u : 0x80000000u);
      const uint32_t ks = (uint32_t)kt * BK * 2u;
      if (w_nt) {
#pragma unroll
        for (int i = 0; i < LDN; ++i)
          load_lds16_untracked<true>(r_w, &lds[ws * STAGE + (wave_u * 8 + RG * i) * BK], vw, chunk_soff(i) + ks);
      } else {
#pragma unroll
        for (int i = 0; i < LDN; ++i)
          load_lds16_untracked(r_w, &lds[ws * STAGE + (wave_u * 8 + RG * i) * BK], vw, chunk_soff(i) + ks);
      }
    };
    // fragments of k-step ks: weight rows from stage ws, token rows from stage st
    auto read_frags = [&](int st, int ws, int ks, int set) {
      const uint16_t* wbase = &lds[ws * STAGE];
      const uint16_t* tbase = &lds[st * STAGE];
      const int pc = ((2 * ks + fr_chunk) ^ swz(fr_row)) * 8;
#pragma unroll
      for (int f = 0; f < FN; ++f) fa[set][f] = *reinterpret_cast<const bf16x8*>(wbase + (wrow[f] + fr_row) * BK + pc);
#pragma unroll
      for (int m = 0; m < FM; ++m)
        fb[set][m] = *reinterpret_cast<const bf16x8*>(tbase + (bn + wm * (BM / WM) + m * 32 + fr_row) * BK + pc);
    };
    auto mfmas = [&](int set) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < FM; ++m)
          acc[f][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][f], fb[set][m], acc[f][m], 0, 0, 0);
    };
    // one K step on LDS stage st (a constant at each call site); K step kt + 1 lands in the
    // other stage meanwhile. W3: the step's weight rows are in stage wr (kt mod 3, a scalar
    // kept across steps), and K step kt + 2's weight rows go to the third one, which held
    // K step kt - 1's; they are left in flight at the step's end (issued last, they are the
    // LDN most recent loads of this wave)
    int wr = 0;
    // A wavefront whose token rows all lie past the m-block (the padding of a partial last
    // m-block) skips its fragment reads and products: it still stages its share of the
    // operands and meets every barrier, and its accumulators stay zero, which the epilogue
    // stages but never stores. Same bytes out; less MFMA and LDS work (dsv3_share +1.8%,
    // small_m_zipf +2% GEMM).
    const bool live = __builtin_amdgcn_readfirstlane(wm * (BM / WM)) < nrows;
    auto step = [&](int st, int kt) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (W3) {
        issue_tokens(kt + 1, st ^ 1);
        issue_weights(kt + 2, wr == 0 ? 2 : wr - 1);
      } else {
        issue_loads(kt + 1, st ^ 1);
      }
      const int ws = W3 ? wr : st;
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
        read_frags(st, ws, 1, 1);
        mfmas(0);
        Interleave<FN * FM, 0, FN + FM, 0>::emit();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(st, ws, 2, 0);
        mfmas(1);
        Interleave<FN * FM, 0, FN + FM, 0>::emit();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(st, ws, 3, 1);
        mfmas(0);
        Interleave<FN * FM, 0, FN + FM, 0>::emit();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (W3) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LDN) : "memory");
        __syncthreads();
        wr = wr == 2 ? 0 : wr + 1;
        read_frags(st ^ 1, wr, 0, 0);
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        read_frags(st ^ 1, st ^ 1, 0, 0);
      }
    };

    if constexpr (W3) {
      issue_weights(0, 0);
      issue_tokens(0, 0);
      issue_weights(1, 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LDN) : "memory");
    } else {
      issue_loads(0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    read_frags(0, 0, 0, 0);
    // two K steps per trip, so the stage index is a constant and the body one basic block
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      step(0, kt);
      step(1, kt + 1);
    }
    if (kt < KT) step(0, kt);
    // W3: the last step's loads past the end (they write zeros) must land before the epilogue
    // reuses the stages
    if constexpr (W3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the epilogue's next task reuses both stages
    if (tracing && tid == 0 && (unsigned)slot < (unsigned)p.max_slots) p.trace[slot].t_epilogue = rt_clock();

    // Epilogue through LDS (both stages are free after the mainloop's last barrier), so that
    // global stores cover whole row segments instead of 8 bytes of 32 rows per instruction.
    // The tile's output is OC columns per token row (Linear-2: 256 of Yd; Linear-1: 128 of A,
    // SwiGLU applied), staged row-major with the 16-byte chunks of row r XOR-swizzled by
    // r mod (chunks per row). A lane holds, for output block (f, m), columns
    // 8g + 4*(lane>>5) + {0..3} of the weight fragment at token row lane & 31.
    {
      const int OC = l2 ? bn : bn / 2;  // output columns of the tile
      const int CPR = OC / 8;           // 16-byte chunks per row (16, 32 or 64)
      uint8_t* const obuf = reinterpret_cast<uint8_t*>(lds);
      auto obuf_off = [&](int row, int chunk) -> int { return row * OC * 2 + ((chunk ^ (row & (CPR - 1))) << 4); };
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        const int tok = wm * (BM / WM) + m * 32 + fr_row;
        if (l2) {
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = wn * (BN / WN) + f * 32 + g * 8;  // + 4 * fr_chunk
              u32x2 v;
              v.x = pack_bf16(acc[f][m][4 * g + 0], acc[f][m][4 * g + 1]);
              v.y = pack_bf16(acc[f][m][4 * g + 2], acc[f][m][4 * g + 3]);
              *reinterpret_cast<u32x2*>(obuf + obuf_off(tok, col >> 3) + fr_chunk * 8) = v;
            }
        } else {
#pragma unroll
          for (int f = 0; f < FN / 2; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = wn * (BN / 2 / WN) + f * 32 + g * 8;
              float a4[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) a4[q] = silu(acc[f][m][4 * g + q]) * acc[f + FN / 2][m][4 * g + q];
              u32x2 v;
              v.x = pack_bf16(a4[0], a4[1]);
              v.y = pack_bf16(a4[2], a4[3]);
              *reinterpret_cast<u32x2*>(obuf + obuf_off(tok, col >> 3) + fr_chunk * 8) = v;
            }
        }
      }
      __syncthreads();
      // thread t stores chunk t % CPR of rows t / CPR, + NT / CPR, ...: a wavefront writes whole
      // row segments; rows past the m-block and columns past the matrix are not stored
      const int ldim = l2 ? p.H : p.I;
      const int col0 = l2 ? nt * kTileN2 : nt * kTileN1;
      const int c = tid & (CPR - 1), col = col0 + c * 8;
      const __amdgpu_buffer_rsrc_t r_out = l2 ? r_yd : r_act;
      if (col < ldim) {  // ldim is a multiple of 64, so a chunk is wholly inside or outside
        for (int r = tid / CPR; r < nrows && r < bm; r += NT / CPR) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(obuf + obuf_off(r, c));
          const int so = (int)(((uint32_t)(row0 + r) * (uint32_t)ldim + (uint32_t)col) * 2u);
          // A is read by Linear-2 tiles on any XCD once the m-block is released: device-scope
          // stores write it through, so the release's L2 write-back has less to do. Yd keeps
          // the default policy, which leaves much of it in the memory-side cache for the
          // combine.
          if (l2) __builtin_amdgcn_raw_buffer_store_b128(v, r_out, so, 0, 0);
          else __builtin_amdgcn_raw_buffer_store_b128(v, r_out, so, 0, kCachePolicySC1);
        }
      }
    }

    if (tracing && tid == 0 && (unsigned)slot < (unsigned)p.max_slots) {
      // the record's tail (a Linear-1 tile's release time follows when it is released)
      p.trace[slot].t_end = rt_clock();
      p.trace[slot].t_release = 0;
    }
    if (!l2) {  // hold this tile's completion; release when the batch is full
      if (tid == 0) {
#pragma unroll
        for (int i = 0; i < kReleaseBatch; ++i)
          if (i == npend) {
            pend_mb[i] = mb;
            pend_slot[i] = (unsigned)slot < (unsigned)p.max_slots ? slot : 0;
          }
      }
      if (++npend >= batch || have_def) release();
    }
    __syncthreads();
  }

  if constexpr (FUSED) {
    layer_finish_phases<NT>(ka, lds, LDS_ELEMS, plan_ok);
  } else {
    // the last workgroup to leave resets the cursor and the ready counters, so the next
    // moe_forward on this plan starts clean without a separate launch
    if (tid == 0) {
      const int done = __hip_atomic_fetch_add(&p.hdr[HDR_DONE], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = done == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (*s_last) {
      const int n = min(p.hdr[HDR_NMBLK], p.max_mblk);
      for (int i = tid; i < n; i += NT) p.mb_ready[i] = 0;
      if (tid == 0) {
        p.hdr[HDR_CURSOR] = 0;
        for (int g = 0; g < kGroups; ++g) p.hdr[HDR_GROUP_CURSOR + g] = 0;
        p.hdr[HDR_DONE] = 0;
      }
    }
  }
}

template <int BM, int WN, int WM, int MINW, bool WIDE>
hipError_t variant_grid(int num_workgroups, int* grid) {
  // the traced and single-launch instances have the same resource limits (launch bounds and
  // LDS): the grid is sized on the plain one
  auto kern = gemm_persistent_kernel<BM, WN, WM, MINW, WIDE, false, false>;
  // resident capacity: the grid never exceeds it, so every workgroup runs at once and each
  // group has workgroups that can take its sublist's tiles
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  constexpr int NT = 64 * WN * WM;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NT, 0);
  if (err != hipSuccess) return err;
  const int capacity = cus * (per_cu > 0 ? per_cu : 1);
  *grid = num_workgroups > 0 && num_workgroups < capacity ? num_workgroups : capacity;
  return hipSuccess;
}

template <int BM, int WN, int WM, int MINW, bool WIDE>
hipError_t launch_variant(const GemmArgs& a, int num_workgroups, hipStream_t s) {
  auto kern = a.trace ? gemm_persistent_kernel<BM, WN, WM, MINW, WIDE, true, false>
                      : gemm_persistent_kernel<BM, WN, WM, MINW, WIDE, false, false>;
  constexpr int NT = 64 * WN * WM;
  int grid = 0;
  hipError_t err = variant_grid<BM, WN, WM, MINW, WIDE>(num_workgroups, &grid);
  if (err != hipSuccess) return err;
  GemmArgs g = a;
  g.ngroups = grid >= kGroups ? kGroups : 1;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

template <int BM, int WN, int WM, int MINW, bool WIDE>
hipError_t launch_layer_variant(const LayerArgs& a, int num_workgroups, hipStream_t s) {
  constexpr int NT = 64 * WN * WM;
  // the planner's phases share the tile loop's LDS (the single-launch instances keep two
  // stages): the scan needs about 54 KiB
  constexpr int kFusedLds = 2 * GemmLds<BM, WN, WM, WIDE>::STAGE_BYTES;
  static_assert(kFusedLds >= 32 * 4 + 4 * MOE_MAX_EXPERTS + 4 * (kWaveTableLds + 1) + 8 * MOE_MAX_EXPERTS + 16,
                "LDS for the planner phases");
  static_assert(kFusedLds >= 4 * (NT / 64) * MOE_MAX_EXPERTS + 16 && kFusedLds >= 4 * kWaveTableLds + 16,
                "LDS for the scatter");
  int grid = 0;
  hipError_t err = variant_grid<BM, WN, WM, MINW, WIDE>(num_workgroups, &grid);
  if (err != hipSuccess) return err;
  if (grid != a.pl.grid) return hipErrorInvalidValue;  // the plan's lead rule assumed this grid
  LayerArgs la = a;
  la.g.ngroups = grid >= kGroups ? kGroups : 1;
  hipLaunchKernelGGL((gemm_persistent_kernel<BM, WN, WM, MINW, WIDE, false, true>), dim3(grid), dim3(NT), 0, s, la);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer(const LayerArgs& a, int tile_m, bool wide, int num_workgroups, hipStream_t s) {
  // the single launch runs regular tiles only: in the wide instance the planner's code pushes
  // the tile loop's scalar registers into scratch memory (moe_layer plans without wide tiles)
  if (wide) return hipErrorInvalidValue;
  switch (tile_m) {
    case 256: return launch_layer_variant<256, 2, 4, 2, false>(a, num_workgroups, s);
    case 128: return launch_layer_variant<128, 2, 2, 1, false>(a, num_workgroups, s);
    case 64: return launch_layer_variant<64, 4, 1, 2, false>(a, num_workgroups, s);
    case 32: return launch_layer_variant<32, 4, 1, 2, false>(a, num_workgroups, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmArgs& a, int tile_m, bool wide, int num_workgroups, hipStream_t s) {
  switch (tile_m) {
    case 256:
      return wide ? launch_variant<256, 2, 4, 2, true>(a, num_workgroups, s)
                  : launch_variant<256, 2, 4, 2, false>(a, num_workgroups, s);
    case 128: return launch_variant<128, 2, 2, 1, false>(a, num_workgroups, s);
    case 64: return launch_variant<64, 4, 1, 2, false>(a, num_workgroups, s);
    case 32: return launch_variant<32, 4, 1, 2, false>(a, num_workgroups, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_grid(int tile_m, bool wide, int num_workgroups, int* grid) {
  switch (tile_m) {
    case 256:
      return wide ? variant_grid<256, 2, 4, 2, true>(num_workgroups, grid)
                  : variant_grid<256, 2, 4, 2, false>(num_workgroups, grid);
    case 128: return variant_grid<128, 2, 2, 1, false>(num_workgroups, grid);
    case 64: return variant_grid<64, 4, 1, 2, false>(num_workgroups, grid);
    case 32: return variant_grid<32, 4, 1, 2, false>(num_workgroups, grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
