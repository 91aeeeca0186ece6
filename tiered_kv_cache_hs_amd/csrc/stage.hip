// Staging the inputs of a decode step inside its graph.
//
// HiSparse summary (marsggbo.github.io, 2026-09-23), section 5: the resolve
// is part of the decode step's graph and runs with no host synchronisation,
// so it reads the indexer's selection from a fixed device buffer that the
// step's own earlier kernels write. hs_k_stage stands in for those
// producers (the indexer, the query projection, the new token's record):
// for step t it copies entry t % ring of each region's source ring into the
// region's fixed destination, then advances t, all on the device. A graph
// that captured one launch stages a new step on every replay.
//
// The step counter advances once per launch: every workgroup reads it
// first, copies its share, and arrives on a counter; the last to arrive
// (all others have read the step by then) writes step + 1 and clears the
// arrivals, so the control words need no clearing between launches.
#include "hs_device.h"

namespace hs {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int STAGE_THREADS = 1024;

// The regions' chunks form one index space (region 0's first, then region
// 1's, ...); each thread copies chunk c = its global index, then c + the
// grid's thread count, and so on (one chunk per thread at the usual sizes).
// The region table is a kernel argument. The control word packs the step
// (high half) and the arrivals of the running launch (low half): thread 0 of
// each workgroup reads it and hands the step to the workgroup through LDS,
// so the only device access before the copy is that read; after its own
// chunk, thread 0 arrives with one atomic add, and the workgroup that
// arrives last (every other one has read its step by then) writes
// (step + 1, 0), so the control word needs no clearing between launches.
// Against taking the step from the arrival's own atomic before the copy
// (every workgroup's first access contending on one word): stage 7.7-8.0
// against 8.6-8.8 us for 328 workgroups, no change for 41.
__global__ __launch_bounds__(STAGE_THREADS) void hs_k_stage(const StageTable tab,
                                                            uint64_t total16, uint64_t *ctl,
                                                            uint32_t ring) {
  __shared__ uint32_t s_step;
  if (threadIdx.x == 0)
    s_step = (uint32_t)(__hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
  lds_barrier();
  const uint32_t t = s_step;
  const uint64_t e = t % ring;
  const uint64_t stride = (uint64_t)gridDim.x * STAGE_THREADS;
  for (uint64_t c = (uint64_t)blockIdx.x * STAGE_THREADS + threadIdx.x; c < total16; c += stride) {
    // the chunk's region: the first whose running end exceeds c
    int i = 0;
#pragma unroll
    for (int j = 0; j + 1 < STAGE_MAX_REGIONS; ++j)
      i += (j + 1 < tab.n && c >= tab.end16[j]) ? 1 : 0;
    const uint64_t off = c - (i ? tab.end16[i - 1] : 0);
    const StageRegion &r = tab.r[i];
    ((HS_GLOBAL v4u *)r.dst)[off] = ((const HS_GLOBAL v4u *)r.src)[e * r.stride16 + off];
  }
  // the arrival, after this thread's step read (same word, program order)
  // and off the copy's path
  if (threadIdx.x == 0) {
    const uint64_t before = __hip_atomic_fetch_add(ctl, (uint64_t)1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)before == gridDim.x - 1)
      __hip_atomic_store(ctl, (uint64_t)(t + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void hs_k_stage_set(uint64_t *ctl, uint32_t step) {
  if (threadIdx.x == 0) *ctl = (uint64_t)step << 32;
}

}  // namespace

hipError_t launch_stage(const StageTable &table, uint64_t total16, uint32_t *d_ctl,
                        uint32_t ring, hipStream_t stream) {
  // one 16-byte chunk per thread, at most 1024 workgroups
  uint64_t blocks = (total16 + STAGE_THREADS - 1) / STAGE_THREADS;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  return launch_k(HS_TRACE_STAGE, hs_k_stage, dim3((unsigned)blocks), dim3(STAGE_THREADS), 0,
                  stream, table, total16, (uint64_t *)d_ctl, ring);
}

hipError_t launch_stage_set(uint32_t *d_ctl, uint32_t step, hipStream_t stream) {
  hipLaunchKernelGGL(hs_k_stage_set, dim3(1), dim3(64), 0, stream, (uint64_t *)d_ctl, step);
  return hipGetLastError();
}

}  // namespace hs
