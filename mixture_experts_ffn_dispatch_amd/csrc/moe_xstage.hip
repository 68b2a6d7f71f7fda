// Burst-Gap microbenchmark of libmoe (gfx950): the X-Stage paper's Section 3 characterisation,
// run against this GPU's own memory (the page's local-memory control) instead of a peer's.
//
// K producer workgroups (one per CU) each issue a burst of B bytes of stores, then compute for
// a gap G, for P periods. The aggregate burst volume is V = K * B. Per producer and period the
// kernel records two readings of the constant-rate real-time counter (s_memrealtime):
//   t_start   all of the producer's wavefronts are about to issue the burst
//   t_issued  every wavefront has issued its last store of the burst (the sender-visible end
//             of issue: nothing waits for the stores to complete)
// The issue time is t_issued - t_start and the period the distance between consecutive
// t_start. The gap is a busy wait from t_issued on the same counter. Bursts rotate through the
// producer's region of the buffer, so a large region keeps the data from settling in cache and
// the stores must drain to memory.
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBurstThreads = 256;
constexpr int kBurstChunk = kBurstThreads * 16;  // bytes one store instruction per thread covers

struct BurstArgs {
  uint8_t* buf;
  size_t region;   // bytes of buf per producer (a multiple of bytes)
  int bytes;       // per producer per burst (a multiple of kBurstChunk)
  int periods;
  long long gap_ticks;
  long long* times;  // [producers][periods][2]
};

__global__ __launch_bounds__(kBurstThreads) void burst_gap_kernel(BurstArgs a) {
  const int tid = threadIdx.x, w = blockIdx.x;
  uint8_t* const base = a.buf + (size_t)w * a.region;
  const int slots = (int)(a.region / (size_t)a.bytes);
  const int n = a.bytes / kBurstChunk;
  const u32x4 val = {(unsigned)w, (unsigned)tid, 0x5A5A5A5Au, 0xA5A5A5A5u};
  long long* const out = a.times + (size_t)w * a.periods * 2;
  for (int p = 0; p < a.periods; ++p) {
    u32x4* const dst = reinterpret_cast<u32x4*>(base + (size_t)(p % slots) * a.bytes);
    __builtin_amdgcn_s_barrier();  // the workgroup starts the burst together (no memory fence)
    const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < n; ++i) dst[(size_t)i * kBurstThreads + tid] = val;
    __builtin_amdgcn_s_barrier();  // every wavefront has issued its stores (none waited for)
    const long long t1 = (long long)__builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
      out[2 * p] = t0;
      out[2 * p + 1] = t1;
    }
    // the producer's compute gap: spin on the same counter
    while ((long long)__builtin_amdgcn_s_memrealtime() - t1 < a.gap_ticks) __builtin_amdgcn_s_sleep(1);
  }
}

}  // namespace

hipError_t launch_burst_gap(uint8_t* buf, size_t region, int producers, int bytes, int periods,
                            long long gap_ticks, long long* times, hipStream_t s) {
  BurstArgs a{buf, region, bytes, periods, gap_ticks, times};
  hipLaunchKernelGGL(burst_gap_kernel, dim3(producers), dim3(kBurstThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
