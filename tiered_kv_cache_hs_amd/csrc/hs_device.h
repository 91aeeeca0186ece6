// Internal definitions shared by the HIP sources of libhisparse (gfx950).
#pragma once

#include <hip/hip_ext.h>
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
  const uint64_t *pages;  // the unit's pool page table (device memory): entry i
                          // is the device-visible address of records
                          // [i << page_shift, (i + 1) << page_shift) in host memory
  const int64_t *len;   // the unit's pool length (device memory)
  int32_t *inv;         // inverse page table: position -> slot, -1 when the
                        // position is not resident; inv_len entries
  int32_t B;
  int32_t page_shift;   // log2 of the records per pool page
  int32_t n_pages;      // entries of the page table
  int32_t inv_len;      // the request's most positions
};

#define HS_GLOBAL __attribute__((address_space(1)))

// (slot, position) pair of a fetch list entry
typedef int32_t int2v __attribute__((ext_vector_type(2)));


// The same unit as seen by a kernel: every pointer in the global address
// space, so accesses compile to global_* instructions. Generic (flat)
// accesses are counted by the LDS wait counter as well as the vector-memory
// one, so a flat load in flight makes every LDS wait, and every barrier
// that orders LDS, wait for it too.
struct UnitG {
  HS_GLOBAL uint8_t *rows;
  HS_GLOBAL int32_t *pos;
  HS_GLOBAL uint32_t *stamp;
  HS_GLOBAL int2v *work;
  HS_GLOBAL int32_t *fsrc;
  HS_GLOBAL uint32_t *ctl;
  HS_GLOBAL const uint64_t *pages;
  HS_GLOBAL const int64_t *len;
  HS_GLOBAL int32_t *inv;
  int32_t B;
  int32_t page_shift;
  int32_t n_pages;
  int32_t inv_len;
};

__device__ __forceinline__ UnitG unit_g(const UnitDesc &d) {
  UnitG g;
  g.rows = (HS_GLOBAL uint8_t *)d.rows;
  g.pos = (HS_GLOBAL int32_t *)d.pos;
  g.stamp = (HS_GLOBAL uint32_t *)d.stamp;
  g.work = (HS_GLOBAL int2v *)d.work;
  g.fsrc = (HS_GLOBAL int32_t *)d.fsrc;
  g.ctl = (HS_GLOBAL uint32_t *)d.ctl;
  g.pages = (HS_GLOBAL const uint64_t *)d.pages;
  g.len = (HS_GLOBAL const int64_t *)d.len;
  g.inv = (HS_GLOBAL int32_t *)d.inv;
  g.B = d.B;
  g.page_shift = d.page_shift;
  g.n_pages = d.n_pages;
  g.inv_len = d.inv_len;
  return g;
}

// Host record p of a unit, through its pool page table (global address space).
__device__ __forceinline__ const HS_GLOBAL uint8_t *pool_record(const UnitG &d, uint32_t p,
                                                               size_t rec_bytes) {
  const uint64_t page = d.pages[p >> d.page_shift];
  const uint32_t in_page = p & ((1u << d.page_shift) - 1u);
  return (const HS_GLOBAL uint8_t *)page + (size_t)in_page * rec_bytes;
}

// A generic pointer taken as a global one (kernel arguments and workspace).
template <class T>
__device__ __forceinline__ HS_GLOBAL T *glb(T *p) {
  return (HS_GLOBAL T *)p;
}

constexpr int CTL_CLOCK = 0;  // resolve steps done
constexpr int CTL_ERR = 1;    // sticky HS_ERR_* bits
constexpr int CTL_FETCH = 2;  // records the last resolve fetched (or left to fetch)
constexpr int CTL_WORDS = 64; // control block size in words (256 bytes)

// Sticky error bits of a unit (device scope).
__device__ __forceinline__ void set_error(HS_GLOBAL uint32_t *ctl, uint32_t bits) {
  __hip_atomic_fetch_or(ctl + CTL_ERR, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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
// While hs_trace_enable(1) is in effect, a launch of class cls takes the
// next pair of the tracer's events (defined in runtime.hip); false when
// tracing is off or the record is full.
bool trace_claim(int cls, hipEvent_t *start, hipEvent_t *stop);

// Every kernel is launched through this. With tracing on, the start and
// stop events are those of the dispatch itself (hipExtLaunchKernelGGL):
// their elapsed time is the kernel's execution, the interval a kernel
// tracer reports, without the marker packets around it.
template <typename F, typename... Args>
inline hipError_t launch_k(int cls, F kernel, dim3 grid, dim3 block, uint32_t lds,
                           hipStream_t stream, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  if (trace_claim(cls, &start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launches
// Declared here, defined in the .hip files; all enqueue on `stream` and
// return the hipError_t of the launch.
// Slots [0, B) empty; the control words cleared too unless ctl is null.
hipError_t launch_buffer_init(int32_t *pos, uint32_t *stamp, int32_t *fsrc, uint32_t *ctl,
                              int B, hipStream_t stream);
// How a resolve fetches its misses: not at all (the attention kernels read
// them from the host pool), inside the resolve kernel (its first host reads
// overlap the victim selection; one workgroup per unit), or with a second
// kernel of many workgroups per unit (enough host reads in flight when the
// batch has few units).
constexpr int FETCH_NONE = 0, FETCH_INLINE = 1, FETCH_KERNEL = 2;
// gb: the fetch's host-read chunks of 16 bytes per lane per batch (1, 2, 4
// or 8; 0 = the default for the buffer size).
hipError_t launch_resolve(const UnitDesc *d_units, int n_units, int max_B,
                          const int32_t *d_topk, int k, int32_t *d_slots,
                          int32_t *d_miss, int fetch, int gb, int rec_bytes,
                          hipStream_t stream);
size_t resolve_lds_bytes(int k);
// Fetch every unit's share of its state's last fetch list (about `workgroups`
// workgroups in total, 0 = 64; `batch` host reads in flight per lane, 1-8).
hipError_t launch_prefetch(const UnitDesc *d_units, int n, int rec_bytes, int workgroups,
                           int batch, hipStream_t stream);
hipError_t launch_regather(const UnitDesc *d_unit, int B, int rec_bytes,
                           hipStream_t stream);
// Inverse page table upkeep: every entry -1; then (rebuild) entry pos[s] = s
// for every occupied slot s < B.
hipError_t launch_inv_clear(int32_t *inv, int64_t n, hipStream_t stream);
hipError_t launch_inv_rebuild(int32_t *inv, int64_t n, const int32_t *pos, int B,
                              hipStream_t stream);
// Records [pos, pos + n) of a unit's pool (page table d_pages) from device
// memory, then its length raised to new_len.
hipError_t launch_append(const uint64_t *d_pages, int page_shift, int64_t pos, int64_t n,
                         int rec_bytes, const uint8_t *src, int64_t *d_len, int64_t new_len,
                         hipStream_t stream);
// One record per unit, from src[u] (device, [n][rec_bytes]) to position
// *len of the unit's pool, then *len + 1; HS_ERR_APPEND where no page is
// allocated there. One workgroup per unit.
hipError_t launch_append_batch(const UnitDesc *d_units, int n, int rec_bytes, const uint8_t *src,
                               hipStream_t stream);

// A stage region: n16 16-byte chunks from src + (t % ring) * stride16 chunks
// to dst. 32 bytes.
struct StageRegion {
  const uint8_t *src;
  uint8_t *dst;
  uint64_t n16;
  uint64_t stride16;
};
// At most this many regions per stage; the table travels in the kernel's
// arguments (no device reads before the copy).
constexpr int STAGE_MAX_REGIONS = 8;
struct StageTable {
  StageRegion r[STAGE_MAX_REGIONS];
  uint64_t end16[STAGE_MAX_REGIONS];  // running sum of n16 up to and including region i
  int n;
};
// Stage control words (device memory, 8-byte aligned): one 64-bit word with
// the step counter in its high half and the arrivals of the running launch
// in its low half (0 between launches).
constexpr int STAGE_CTL_WORDS = 64;
// Copies entry step % ring of every region, then advances the step.
hipError_t launch_stage(const StageTable &table, uint64_t total16, uint32_t *d_ctl,
                        uint32_t ring, hipStream_t stream);
// Sets the step (arrivals 0).
hipError_t launch_stage_set(uint32_t *d_ctl, uint32_t step, hipStream_t stream);

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

// Most selection entries one latent attention workgroup covers (its slot
// ids are staged in LDS).
constexpr int LAT_MAX_CHUNK = 2048;

struct AttnLatentArgs {
  const UnitDesc *units;
  const uint16_t *q;
  const int32_t *slots;
  int n_units, k, Hq, splits, chunk;  // chunk: a multiple of 64, at most LAT_MAX_CHUNK
  int hpw;                            // query heads per workgroup: 32 or 64
  float scale_log2;
  uint16_t *ws_o;  // split partials, bf16
  float *ws_ml, *out;
};
hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream);

// Split-k combine over [rows][splits][dv] partials, fp32 (partial_bf16 = 0)
// or bf16 (1), and [rows][splits] (m, l) pairs.
hipError_t launch_combine(const void *ws_o, int partial_bf16, const float *ws_ml, int rows,
                          int splits, int dv, float *out, hipStream_t stream);

}  // namespace hs
