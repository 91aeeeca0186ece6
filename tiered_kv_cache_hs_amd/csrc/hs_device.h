// Internal definitions shared by the HIP sources of libhisparse (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hs {

// Device view of one (request, layer) unit of a batch. 128 bytes.
struct __attribute__((aligned(128))) UnitDesc {
  uint8_t *rows;        // B rows of rec_bytes (device memory)
  int32_t *pos;         // page table: slot -> logical position, -1 empty
  uint32_t *stamp;      // LRU stamps, 0 = never used
  int2 *work;           // last resolve's fetch list: (slot, position), B entries
  int32_t *fsrc;        // last resolve, per selection index: its position if it
                        // was a miss (fetched from the pool), else -1; B entries
  uint32_t *ctl;        // [CTL_CLOCK], [CTL_ERR], [CTL_FETCH]
  const uint8_t *pool;  // device-visible address of the unit's host records
  const int64_t *len;   // the unit's pool length (device memory)
  int32_t B;
  int32_t pad[5];
};

constexpr int CTL_CLOCK = 0;  // resolve steps done
constexpr int CTL_ERR = 1;    // sticky HS_ERR_* bits
constexpr int CTL_FETCH = 2;  // records the last resolve must fetch
constexpr int CTL_WORDS = 64; // control block size in words (256 bytes)

// Workgroup barrier that orders LDS accesses only. A plain __syncthreads()
// also waits for every outstanding global load and store of the wave
// (s_waitcnt vmcnt(0)); where threads exchange data only through LDS, this
// one lets global traffic stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Byte layout of a buffer's caller-owned memory.
struct BufferLayout {
  size_t rows, pos, stamp, work, fsrc, ctl, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline BufferLayout buffer_layout(size_t rec_bytes, int B) {
  BufferLayout l;
  l.rows = 0;
  l.pos = align_up((size_t)B * rec_bytes, 256);
  l.stamp = l.pos + align_up((size_t)B * 4, 256);
  l.work = l.stamp + align_up((size_t)B * 4, 256);
  l.fsrc = l.work + align_up((size_t)B * 8, 256);
  l.ctl = l.fsrc + align_up((size_t)B * 4, 256);
  l.total = l.ctl + CTL_WORDS * 4;
  return l;
}

// ----------------------------------------------------------------- tracing
// Event pairs around kernel launches while hs_trace_enable(1) is in effect
// (no-ops otherwise). Defined in runtime.hip.
void trace_begin(int cls, hipStream_t stream);
void trace_end(hipStream_t stream);

// ---------------------------------------------------------------- launches
// Declared here, defined in the .hip files; all enqueue on `stream` and
// return the hipError_t of the launch.
hipError_t launch_buffer_init(int32_t *pos, uint32_t *stamp, int32_t *fsrc, uint32_t *ctl,
                              int B, hipStream_t stream);
hipError_t launch_resolve(const UnitDesc *d_units, int n_units, int max_B,
                          const int32_t *d_topk, int k, int32_t *d_slots,
                          int32_t *d_miss, int gather_wgs, int rec_bytes,
                          hipStream_t stream);
size_t resolve_lds_bytes(int k);
hipError_t launch_regather(const UnitDesc *d_unit, int B, int rec_bytes,
                           hipStream_t stream);
hipError_t launch_append(uint8_t *dst_dev, const uint8_t *src, int64_t bytes,
                         int64_t *d_len, int64_t new_len, hipStream_t stream);

struct AttnMhaArgs {
  const UnitDesc *units;
  const void *q;
  const int32_t *slots;
  int n_units, k, Hq, Hkv, D, dtype, splits, chunk, rec_bytes;
  int fetch;  // fused resolve: read just-resolved misses from the host pool
  float scale_log2;
  float *ws_o, *ws_ml, *out;
};
hipError_t launch_attn_mha(const AttnMhaArgs &a, hipStream_t stream);

struct AttnLatentArgs {
  const UnitDesc *units;
  const uint16_t *q;
  const int32_t *slots;
  int n_units, k, Hq, splits, chunk;
  int fetch;  // fused resolve: read just-resolved misses from the host pool
  float scale_log2;
  float *ws_o, *ws_ml, *out;
};
hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream);

hipError_t launch_combine(const float *ws_o, const float *ws_ml, int rows,
                          int splits, int dv, float *out, hipStream_t stream);

}  // namespace hs
