/*
 * moe.h - C ABI of libmoe: one GPU's share of an expert-parallel mixture-of-experts FFN layer
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer (X-Stage paper, "X-Stage: An Overlooked Pipeline Stage for Communication-
 * Computation Overlap in DiT Inference", Introduction, MoE-layer paragraph): a router selects
 * k experts per token; Dispatch moves each token to its experts; every expert applies
 * Linear-1 (hidden H -> 2I, gate and up halves), SwiGLU, and Linear-2 (I -> H); Combine sums
 * each token's k expert outputs weighted by the router weights. The same page's expert-wave
 * paragraph groups local experts into waves that order the tile work; Section 4 (the X-Stage
 * design test and the MegaMoE discussion) moves ready Linear-1 tiles of later waves between
 * the Linear-2 tiles of the current wave. Both orders compute identical bytes here.
 *
 * The four calls follow the stages: moe_plan (route + expert histogram + prefix scan +
 * stable scatter + tile schedule), moe_dispatch (gather rows), moe_forward (persistent grouped
 * GEMM: Linear-1 with fused SwiGLU, then Linear-2), moe_combine (router-weighted sum).
 * moe_forward_gather is moe_dispatch + moe_forward in one launch (rows gathered on load);
 * moe_layer runs the whole layer as one launch, and moe_layer_noalloc the layer without a
 * caller workspace. The attention forward of the same paper's second workload is in attn.h.
 *
 * Conventions for every call:
 *   - bfloat16 tensors are passed as uint16_t bit patterns; all tensors are dense row-major.
 *   - Every pointer except `cfg`, `rt` and `bytes`/`layout` outputs is a DEVICE pointer owned
 *     by the caller (for example a torch tensor's data_ptr()). The library never allocates,
 *     frees or retains caller memory and keeps no global state between calls, apart from the
 *     static workspace array of moe_layer_noalloc and its per-device address.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every device call
 *     is asynchronous on that stream and performs no host synchronisation, except
 *     moe_status_read, which synchronises the stream.
 *   - Arguments are validated on the host before anything is launched; an invalid call
 *     returns an error code and launches nothing. No call aborts or throws.
 *   - moe_dispatch / moe_forward / moe_combine must be given the routing buffers and workspace
 *     filled by a moe_plan with the same cfg, earlier on the same stream (or ordered after it).
 *   - Calls on different streams must use different routing buffers and workspaces.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

/* Status codes. */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, k > E, unknown schedule ...   */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement (see limits)      */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_size() reports           */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed                    */
  MOE_ERR_TIMEOUT = -5      /* a Linear-2 tile's bounded wait for its Linear-1 rows expired   */
} moe_status_code;
typedef int32_t moe_status;

/* Tile orders of the persistent grouped GEMM (moe_config.schedule). */
enum {
  /* Expert-Wave order: Linear-1 tiles of wave 0, its Linear-2 tiles, then wave 1, ...
     (X-Stage paper, Introduction, expert-wave paragraph: the original MegaMoE schedule). */
  MOE_SCHED_EXPERT_WAVE = 0,
  /* Cross-wave interleaving: Linear-1 tiles of wave w + lead_waves are spread evenly between
     the Linear-2 tiles of wave w (X-Stage paper, Section 4.1 "reshape injection" and Section
     4.2 on MegaMoE: ready Linear-1 work of later waves is moved between Linear-2 epilogues;
     the lead is the dependency-derived threshold the paper calls D_knee). */
  MOE_SCHED_INTERLEAVED = 1,
  /* moe_plan picks the order and the lead itself, from the routed tile counts and the X-Stage
     calibration in moe_config (X-Stage paper, Discussion, burst-shaping paragraph: a runtime
     compares the predicted X-Stage stall reduction with the locality cost and selects the
     original or the interleaved schedule for the current routing and working set). The rule
     is stated below; lead_waves must be 0. The choice is recorded in the workspace header. */
  MOE_SCHED_AUTO = 2
};

/* The MOE_SCHED_AUTO rule. Per expert wave i: a_i Linear-1 and b_i Linear-2 tiles, A_i bytes of
   activation (rows x I x 2); G persistent workgroups; tile height BM. A tile's main loop over
   K is estimated as t(K) = G * max(2 BM 256 K / P, 512 K / B) (P = 1.2e15 flop/s and
   B = 5.0e12 B/s, the kernel's sustained MFMA and weight-streaming rates on this GPU);
   t1 = t(H), t2 = t(I). Candidates: Expert-Wave, and interleaved with lead D = 1 .. waves. For
   each wave with Linear-2 tiles:
     aligned producers K = max(1, min(G, b_i) * s), s = b_i t2 / (b_i t2 + a_{i+D} t1) the
             Linear-2 share of the work when wave i + D's Linear-1 tiles are spread among wave
             i's Linear-2 tiles (s = 1 in the Expert-Wave order; a_{i+D} = 0 past the last wave),
     burst   V = K * BM * 256 * 2 bytes (their Yd stores, Section 4.2: V = K_act V_t),
     gap     g = t2 (each producer's Linear-2 main loop between its bursts),
     issue   T = max(t_iss0, V / R - g), and at least (V - Q) / R when V - R t_iss0 > Q
             (the max law and the capacity bound of Section 3),
     X-Stage stall   += (b_i / K) * (T - t_iss0),
     dependency stall += t1 / 2 when the wave's Linear-2 tiles can be reached before its
             Linear-1 tiles are done: always in the Expert-Wave order, and in the interleaved
             order when dist_i(D) * (A H + B I) < G * H * (A + B) (the lead rule above).
   Locality cost: the activation bytes kept live while wave i's Linear-2 tiles run (A_i, or
   A_i + ... + A_{i+D} interleaved) above 256 MiB (the last-level cache), the worst wave, divided
   by B, counted only when the GEMM's algorithmic bytes / B exceed its flops / P. The candidate
   with the smallest stall + dependency stall + locality cost wins; ties go to interleaved and
   then to the larger lead. Computed in double precision without fused multiply-adds. */

/* Lead chosen by moe_plan when lead_waves is 0 (interleaved order): a Linear-2 tile of wave w
   should be taken only after the last Linear-1 tile of wave w has finished. With G persistent
   workgroups, list positions are taken at about G per mean tile duration; tile durations scale
   with their K (H for Linear-1, I for Linear-2). With a_j, b_j the Linear-1 / Linear-2 tiles of
   wave j, A, B their totals and PA, PB their prefix sums, the tiles between the last Linear-1
   tile of wave i and its first Linear-2 tile number
     dist_i(D) = PB[i] - PB[max(0, i-D+1)] + PA[min(i+D, nw)] - PA[min(i+1, nw)],
   and D is the smallest lead with dist_i(D) * (A*H + B*I) >= G * H * (A + B) for every wave
   with Linear-2 tiles, else nw. The lead only reorders tiles; results do not depend on it. */

/* Limits of this implementation (violations return MOE_ERR_UNSUPPORTED). */
#define MOE_MAX_EXPERTS 1024 /* E                                        */
#define MOE_MAX_TOPK 32      /* k                                        */
#define MOE_DIM_MULTIPLE 64  /* H and I must be multiples of this        */

typedef struct moe_config {
  int32_t T;                /* tokens on this GPU (>= 1)                                        */
  int32_t H;                /* hidden size (multiple of 64)                                      */
  int32_t I;                /* expert intermediate size (multiple of 64); Linear-1 yields 2*I   */
  int32_t E;                /* local experts (1..1024)                                           */
  int32_t k;                /* experts per token (1..min(E, 32))                                 */
  int32_t experts_per_wave; /* W >= 1; wave w holds experts [w*W, min(E, (w+1)*W))              */
  int32_t schedule;         /* MOE_SCHED_*                                                       */
  int32_t lead_waves;       /* interleaved order only: D >= 1, or 0 = chosen by moe_plan (below);
                               0 with MOE_SCHED_AUTO                                             */
  int32_t num_workgroups;   /* persistent grid; 0 or more than fits at once = every resident slot */
  int32_t tile_m;           /* rows per GEMM tile: 0 = chosen from T*k/E, else 32, 64, 128, 256 */
  int32_t spin_limit;       /* bounded-wait iterations of a Linear-2 tile; 0 = default (~seconds)*/
  int32_t flags;            /* must be 0 except MOE_FLAG_* bits below                            */
  /* X-Stage calibration of the path the Linear-2 stores take, for MOE_SCHED_AUTO (0 = this
     GPU's own memory, as calibrated by moe_burst_gap: 0.927 us, 6646 GB/s, 31.2 MiB) */
  float xs_issue_us;        /* t_iss0: backpressure-free issue time of a burst, microseconds     */
  float xs_drain_gbps;      /* R: effective drain rate, GB/s                                    */
  float xs_capacity_mib;    /* Q: effective outstanding capacity, MiB                           */
  int32_t reserved;         /* must be 0                                                         */
  void* trace;              /* per-tile trace of moe_forward (moe_trace_rec below), NULL = off   */
} moe_config;

/* Per-tile trace (X-Stage paper, Section 5: per-tile instrumentation of the persistent kernel to
 * check which tile order ran and where its time went). When moe_config.trace is not NULL,
 * moe_forward / moe_forward_gather / moe_layer_noalloc write one record per tile they run into
 * that device buffer, which must hold moe_ws_layout.max_slots records. Record i belongs to
 * record slot i of the locality groups' tile lists (moe_ws_layout.group_tasks), or, when the
 * grid has fewer than 8 workgroups (one shared cursor), to list position i of the tile list.
 * Slots no tile ran (no-op slots, the odd n-tiles of wide m-blocks) are left untouched, so
 * callers fill the buffer with a marker first. Times are readings of the constant-rate
 * real-time counter (frequency: moe_burst_clock_hz), taken by the workgroup's waves in step;
 * records are written by one lane with vector stores at the end of each tile. With trace NULL
 * the kernel takes none of these readings. Results never depend on the trace. */
typedef struct moe_trace_rec {
  int32_t task;       /* task word (bit 31 Linear-2, bits 30..12 m-block, bits 11..0 n-tile)      */
  int32_t workgroup;  /* persistent workgroup (block index) that ran the tile                     */
  int32_t xcc;        /* XCC (XCD) it ran on (hardware register XCC_ID)                           */
  int32_t hw_id;      /* raw HW_ID register of its first wavefront (CU, shader engine, SIMD)      */
  int64_t t_claim;    /* before the claim (one atomic on the group cursor, then the record load) */
  int64_t t_claimed;  /* the tile's record in hand                                               */
  int64_t t_start;    /* main loop starts (Linear-2: after its dependency wait)                   */
  int64_t t_epilogue; /* main loop done, epilogue starts                                         */
  int64_t t_end;      /* epilogue stores issued                                                  */
  int64_t t_release;  /* Linear-1: its completion released (after the agent-scope release fence,
                         before the m-block counter is bumped); Linear-2: 0                      */
} moe_trace_rec;

/* Test hook: make every Linear-2 tile wait for one Linear-1 completion that never comes, so the
   bounded wait expires (after spin_limit iterations) and the kernel exits normally with
   MOE_ERR_TIMEOUT recorded. Results are then undefined. Never set in production. */
#define MOE_FLAG_FORCE_WAIT_TIMEOUT 0x1

/* Wide last m-blocks. With 256-row tiles, moe_plan can run an m-block of at most 128 rows (an
   expert's last, partial block) as tiles of 128 token rows by 512 weight rows: half as many
   tiles as 256 x 256 ones, with no token rows of padding. moe_forward then launches the kernel
   instance that runs them. It is off by default: the regular instance keeps weight rows two K
   steps ahead and skips the products of wavefronts that hold only padding rows, which measured
   as fast or faster on every workload where 256-row tiles are picked. MOE_FLAG_WIDE_TAILS turns
   it on (MOE_FLAG_NO_WIDE_TAILS, off, is the default; setting both is MOE_ERR_INVALID_ARG).
   Outputs are bit-identical either way: every element keeps its K order. moe_plan and
   moe_forward must receive the same flags. */
#define MOE_FLAG_NO_WIDE_TAILS 0x2
#define MOE_FLAG_WIDE_TAILS 0x4

/* moe_plan runs its steps in one launch with a grid barrier instead of three launches (route,
   scan and schedule, scatter); the results are the same bytes. On MI355X the barrier's
   cross-XCD atomics cost more than the two launch boundaries it replaces (the plan takes 3 to
   15 us longer), so this is for comparison. */
#define MOE_FLAG_PLAN_ONE_LAUNCH 0x8

/* Test hook: the persistent GEMM's workgroups of locality group 0 take no tile, as if a kernel
   running concurrently kept their XCD busy for the whole launch; the other groups must run
   every tile (see the progress note on moe_forward). Never set in production. */
#define MOE_FLAG_TEST_ABSENT_GROUP 0x10

/* Routing buffers, written by moe_plan and read by the later calls (device pointers). */
typedef struct moe_routing {
  int32_t* topk_ids; /* [T, k]   expert of slot (t, j); j ascending = descending router logit  */
  float* topk_w;     /* [T, k]   renormalised router weight of slot (t, j)                      */
  int32_t* counts;   /* [E]      rows routed to each expert                                     */
  int32_t* offsets;  /* [E + 1]  first dispatched row of each expert; offsets[E] = T*k          */
  int32_t* perm;     /* [T*k]    perm[r] = flat slot t*k + j held by dispatched row r           */
  int32_t* pos;      /* [T*k]    pos[t*k + j] = dispatched row of slot (t, j)                   */
} moe_routing;

/* Where moe_plan keeps its schedule inside the workspace (byte offsets from the workspace
   base; all int32 arrays). Filled on the host by moe_workspace_layout. */
typedef struct moe_ws_layout {
  size_t total_bytes;   /* = moe_workspace_size                                     */
  size_t header;        /* int32[64]: [0] error code, [1] task cursor, [2] task count,
                           [3] m-block count, [4] tile_m, [5] L1 n-tiles per m-block,
                           [6] L2 n-tiles per m-block, [7] exited workgroups,
                           [8..15] records handed out from each locality group's list,
                           [16] units in the unit table, [17..25] group unit lists,
                           [26] interleave lead used (0: Expert-Wave order), [27] GEMM grid
                           the plan assumed, [28] the order used (MOE_SCHED_EXPERT_WAVE or
                           MOE_SCHED_INTERLEAVED),
                           [32..40] group record lists (first record of group g, 9th = end) */
  size_t chunk_counts;  /* int32[E * ((chunks + 3) & ~3)]: per-(expert, token chunk) counts, then each
                           chunk's first row among its expert's rows */
  size_t mblk_expert;   /* int32[max_mblk]                                        */
  size_t mblk_row0;     /* int32[max_mblk]                                        */
  size_t mblk_rows;     /* int32[max_mblk]                                        */
  size_t mblk_ready;    /* int32[max_mblk]: Linear-1 tiles finished per m-block   */
  size_t tasks;         /* int32[max_tasks]: the tile list in schedule order; bit 31 = Linear-2,
                           bits 30..12 m-block, bits 11..0 n-tile                    */
  size_t unit_start;    /* int32[max_tasks + 1]: list position of each unit's first tile
                           (a unit: up to 32 consecutive tiles of one wave's Linear-1 or
                           Linear-2 run; header[16] holds the unit count)           */
  size_t group_units;   /* int32[max_tasks]: the units of locality group 0 in list order,
                           then those of group 1, ... (group g: entries
                           [header[17+g], header[18+g]))                           */
  size_t group_tasks;   /* int32[max_slots][4]: each group's units in its order, 32 record
                           slots per unit holding its tiles as (task word, expert, first
                           dispatched row, rows), spare slots 0x7FFFFFFE (no-op);
                           group g: slots [header[32+g], header[33+g])             */
  size_t wave_table;    /* int32[24 + 10 (E + 1)] at most: per expert wave its tile counts,
                           unit prefix sums and list positions, and each expert's first
                           m-block and first row, from which moe_plan places the tiles */
  size_t layer_sync;    /* 4 KiB right after the header, at the same offset for every config:
                           the grid-barrier counters of moe_plan and moe_layer, one per
                           128-byte line (zero before the first call on a workspace; every
                           launch leaves them zero) */
  size_t defer_slots;   /* int32[2048][8]: each persistent workgroup's deferred Linear-2 tile
                           (its record and record slot), written before it is read */
  int32_t chunks;       /* token chunks of the routing histogram                  */
  int32_t chunk_tokens; /* tokens per chunk (the last chunk may hold fewer)       */
  int32_t max_mblk;
  int32_t max_tasks;
  int32_t max_slots;    /* record slots of the group lists                        */
  int32_t tile_m;       /* rows per tile                                          */
  int32_t tile_n1;      /* Linear-1 tile: output columns of A per tile (gate+up = 2x weight rows) */
  int32_t tile_n2;      /* Linear-2 tile: output columns of Yd per tile            */
  int32_t n1_tiles;     /* ceil(I / tile_n1)                                        */
  int32_t n2_tiles;     /* ceil(H / tile_n2)                                        */
} moe_ws_layout;

/* ABI version of the loaded library (MOE_ABI_VERSION). Host only. */
int32_t moe_abi_version(void);

/* Static description of a status code. Never NULL. Host only. */
const char* moe_strerror(moe_status status);

/* Bytes of device workspace that moe_plan / moe_forward need for `cfg` (host only, no GPU
   access). The workspace holds the routing histogram, the m-block table, the dependency
   counters and the tile list. Errors: MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as for
   moe_plan. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Host-side description of the workspace layout for `cfg` (no GPU access). */
moe_status moe_workspace_layout(const moe_config* cfg, moe_ws_layout* layout);

/* Route and plan (X-Stage paper, Introduction, MoE-layer and expert-wave paragraphs).
 *   logits [T, E] float32: router logits of this GPU's tokens over its E local experts.
 * Writes every array of `rt` and the schedule in `ws`:
 *   topk_ids/topk_w: per token the k largest logits in descending order (equal logits: lower
 *     expert id first; -0 equals +0); weights = softmax restricted to the k kept logits
 *     (the full softmax renormalised over them), float32. NaN logits are not supported.
 *   counts/offsets/perm/pos: a stable counting sort of slots f = t*k + j by expert, so the
 *     dispatched rows are expert-contiguous and, within an expert, in slot order.
 *   ws: m-block table, zeroed dependency counters, and the Linear-1/Linear-2 tile list in
 *     the order cfg->schedule asks for.
 * Three kernel launches (route, scan and schedule, scatter and tile placement), no host
 * synchronisation. With MOE_FLAG_PLAN_ONE_LAUNCH one launch instead: its grid of resident
 * workgroups routes the token chunks; the last workgroup to arrive writes the schedule while
 * the others wait at a grid barrier, then all scatter and place the tile list. Its barrier
 * counters (moe_ws_layout.layer_sync) must then be zero before the call (a zero-filled
 * workspace; every launch leaves them zero). That wait is bounded: if a kernel running
 * concurrently keeps workgroups of the grid from starting until it expires, MOE_ERR_TIMEOUT
 * is recorded (moe_status_read), the routing outputs are undefined and the tile list is left
 * empty, so a later moe_forward runs no tile. */
moe_status moe_plan(const moe_config* cfg, const float* logits, const moe_routing* rt, void* ws,
                    size_t ws_bytes, void* stream);

/* Dispatch: xd[r, :] = x[perm[r] / k, :] for r < T*k (bit copy). Implemented token-major
 * (each token row is read once and written to its k rows pos[t*k + j]), so it reads rt->pos.
 *   x [T, H] bf16 in; xd [T*k, H] bf16 out (caller-allocated). */
moe_status moe_dispatch(const moe_config* cfg, const moe_routing* rt, const uint16_t* x,
                        uint16_t* xd, void* stream);

/* Expert FFN over all dispatched rows in one persistent launch (its last workgroup resets the
 * plan's counters, so moe_forward may be repeated on one plan).
 * Progress: each of the 8 locality groups (workgroup index mod 8, one XCD each) walks its own
 * part of the tile list first and takes the other groups' parts once its own is used up. A
 * Linear-2 tile waits for Linear-1 tiles that may sit in another group's part; if that group
 * has no resident workgroup (a kernel running concurrently keeps its XCD busy), a wait that
 * lasts 1 ms sets the tile aside and its workgroup runs only tiles that cannot wait (the
 * first unclaimed record of any group's part that is a Linear-1 tile or a ready Linear-2
 * tile) until it is ready. So the launch finishes as long as at least one workgroup of the
 * grid runs; what remains required is that workgroups which have started keep running. The
 * grid is sized to the resident capacity; a wait that still exceeds spin_limit records
 * MOE_ERR_TIMEOUT (outputs undefined; no hang). MOE_FLAG_TEST_ABSENT_GROUP forces an absent
 * group for tests.
 *   xd  [T*k, H] bf16 dispatched rows (from moe_dispatch)
 *   w1  [E, 2I, H] bf16: rows [0, I) gate, rows [I, 2I) up (out x in, like nn.Linear.weight)
 *   w2  [E, H, I] bf16
 *   act [T*k, I] bf16 out: A = bf16(silu(xd W_gate^T) * (xd W_up^T)), fp32 accumulation
 *   yd  [T*k, H] bf16 out: Yd = bf16(A W2^T), fp32 accumulation
 * Tiles run in the order moe_plan stored; every order gives the same bytes (each output
 * element accumulates over k in the same fixed order). Experts with no rows read no weights.
 * A Linear-2 tile that waits longer than the bounded spin records MOE_ERR_TIMEOUT in the
 * workspace (read it with moe_status_read) and the kernel still exits. */
moe_status moe_forward(const moe_config* cfg, const uint16_t* xd, const uint16_t* w1,
                       const uint16_t* w2, uint16_t* act, uint16_t* yd, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_forward with the dispatch folded into Linear-1's operand loads (the MegaMoE kernel of the
 * X-Stage paper's Introduction fuses dispatch into its persistent kernel): a Linear-1 tile
 * reads token row perm[r] / k of x for dispatched row r, so no xd buffer is written or read.
 *   rt  routing from moe_plan (reads rt->perm); x [T, H] bf16 token rows
 *   w1, w2, act, yd, ws as for moe_forward.
 * act, yd (and so the combined output) are byte-identical to moe_dispatch + moe_forward.
 * MOE_ERR_INVALID_ARG if rt, rt->perm or x is NULL; otherwise as moe_forward. */
moe_status moe_forward_gather(const moe_config* cfg, const moe_routing* rt, const uint16_t* x,
                              const uint16_t* w1, const uint16_t* w2, uint16_t* act, uint16_t* yd,
                              void* ws, size_t ws_bytes, void* stream);

/* Combine: out[t, :] = bf16( sum_{j=0..k-1} topk_w[t, j] * yd[pos[t*k + j], :] ), fp32 sum in
 * ascending j (fixed order, no atomics, deterministic).
 *   yd [T*k, H] bf16 in; out [T, H] bf16 out. */
moe_status moe_combine(const moe_config* cfg, const moe_routing* rt, const uint16_t* yd,
                       uint16_t* out, void* stream);

/* The whole layer in ONE kernel launch (X-Stage paper, Introduction, MegaMoE paragraph: one
 * persistent kernel runs every stage of the layer). The persistent grid first routes the token
 * chunks, then its last workgroup to arrive writes the schedule while the others wait, then
 * all scatter the chunks and place the tile list; after a grid-wide barrier they run the tiles
 * (Linear-1 gathering token rows from x through perm, SwiGLU, Linear-2), and after another
 * one the combine. Same kernels' arithmetic as moe_plan + moe_forward_gather + moe_combine:
 * rt, act, yd and out are byte-identical to them.
 *   logits, rt, x, w1, w2, act, yd, out, ws: as for those calls.
 * The workspace's phase counters (moe_ws_layout.layer_sync) must be zero before its first
 * moe_layer (a zero-filled workspace); every launch leaves them zero. The grid's workgroups
 * wait for one another at the phase barriers, so they must all be resident at once: the grid
 * is sized to the resident capacity, and a kernel running concurrently on another stream can
 * keep some from starting; every wait is bounded (spin_limit), and an expired one records
 * MOE_ERR_TIMEOUT (moe_status_read) with the outputs undefined, and never hangs or faults. After moe_layer the workspace holds its plan, ready
 * for moe_forward / moe_forward_gather as after moe_plan. It always runs regular tiles (no
 * wide last m-blocks, whatever the flags say; the bytes are the same), so a later
 * moe_forward on that plan must not be given MOE_FLAG_WIDE_TAILS.
 * Errors: as moe_plan; MOE_ERR_INVALID_ARG for a non-NULL cfg->trace (trace the separate
 * calls); MOE_ERR_UNSUPPORTED with more than 64 expert waves when they also exceed the
 * workgroup's threads (512 for 256-row tiles, else 256). */
moe_status moe_layer(const moe_config* cfg, const float* logits, const moe_routing* rt, const uint16_t* x,
                     const uint16_t* w1, const uint16_t* w2, uint16_t* act, uint16_t* yd, uint16_t* out, void* ws,
                     size_t ws_bytes, void* stream);

/* ---- Layer without caller-provided workspace ----
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. moe_layer_noalloc runs moe_plan, moe_forward_gather
 * and moe_combine (the same kernels, so the same bytes) with the workspace in a static device
 * array of MOE_STATIC_WORKSPACE_BYTES inside the library instead of a caller buffer. It calls
 * no hipMalloc, hipFree or other allocating routine. Each GPU the library runs on holds its own
 * array until the process ends; its device address is looked up with hipGetSymbolAddress on
 * the first call on that device (made with that device current) and kept.
 *   logits, rt, x, w1, w2, act, yd, out: as for moe_plan / moe_forward_gather / moe_combine
 *     (caller-owned device buffers; rt's arrays are written).
 *   status: device int32 or NULL; receives the device-side error word (MOE_OK or
 *     MOE_ERR_TIMEOUT, as moe_status_read reports it) by a 4-byte device-to-device copy
 *     ordered after the layer on `stream`.
 * Every call on one GPU shares that GPU's array, and each call's moe_plan rewrites every part
 * of it that the later kernels read: calls on one GPU must be ordered (one stream, or events);
 * calls that overlap on one GPU race and give undefined results.
 * cfg->trace must be NULL (MOE_ERR_INVALID_ARG otherwise): the traced kernel instances are a
 * measurement aid and may use private memory.
 * Errors: as moe_plan; MOE_ERR_WORKSPACE when moe_workspace_size(cfg) exceeds
 * MOE_STATIC_WORKSPACE_BYTES (checked before anything is launched); MOE_ERR_HIP if the array's
 * address cannot be obtained or a launch fails. */
#define MOE_STATIC_WORKSPACE_BYTES (8u << 20)
moe_status moe_layer_noalloc(const moe_config* cfg, const float* logits, const moe_routing* rt,
                             const uint16_t* x, const uint16_t* w1, const uint16_t* w2, uint16_t* act,
                             uint16_t* yd, uint16_t* out, int32_t* status, void* stream);

/* ---- Burst-Gap calibration (X-Stage paper, Section 3: the Burst-Gap microbenchmarks) ----
 * K producers each store a burst of B bytes, then compute for a gap G, for P periods; the
 * page measures the sender-visible issue time and the period to fit the backpressure-free
 * issue time, the effective drain rate and the effective outstanding capacity. This runs the
 * benchmark against the GPU's own memory (the page's local-memory control). */
typedef struct moe_burst_cfg {
  int32_t producers;  /* K: concurrent producer workgroups, 1 .. number of CUs (one per CU)   */
  int32_t bytes;      /* B: bytes each producer stores per burst, a multiple of 4096, <= 2^30  */
  int32_t periods;    /* P: bursts per producer, 1 .. 65536                                     */
  int32_t reserved0;  /* must be 0                                                              */
  int64_t gap_ticks;  /* G in ticks of the real-time counter (moe_burst_clock_hz), 0 .. 10^6   */
} moe_burst_cfg;

/* Runs the benchmark on `stream` (asynchronous). The buffer is split into K equal regions; each
 * producer's bursts rotate through its region (a region far larger than the caches makes the
 * stores drain to memory). times[(w * P + p) * 2 + 0] / [+ 1] receive, for producer w and
 * period p, the real-time counter when the producer starts the burst and when all of its
 * wavefronts have issued their last store (nothing waits for the stores); the gap is a busy wait
 * from the second reading.
 *   buf   device buffer of buf_bytes >= K * B bytes (its contents are overwritten)
 *   times device int64 [K * P * 2]
 * MOE_ERR_INVALID_ARG for a NULL pointer, a field outside its range or a buffer too small;
 * MOE_ERR_HIP if the device query or the launch fails. */
moe_status moe_burst_gap(const moe_burst_cfg* cfg, void* buf, size_t buf_bytes, int64_t* times,
                         void* stream);

/* Frequency of the real-time counter used by moe_burst_gap, in Hz (a device attribute). */
moe_status moe_burst_clock_hz(int64_t* hz);

/* Synchronises `stream`, then returns the device-side error recorded in the workspace since
 * the last moe_plan: MOE_OK, MOE_ERR_TIMEOUT (a bounded wait expired), or
 * MOE_ERR_WORKSPACE (moe_forward found a tile that no moe_plan for this cfg could have written
 * and skipped it); MOE_ERR_HIP if the stream reports a failure. */
moe_status moe_status_read(const void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
