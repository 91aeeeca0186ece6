// Host runtime of libhisparse: the C ABI declared in include/hisparse.h.
//
// Owns the pinned host pool (HiSparse summary, marsggbo.github.io
// 2026-09-23, section 3: the host copy is authoritative and holds every
// record), validates arguments, lays out caller-owned device buffers, uploads
// batch descriptor tables and enqueues the kernels of resolve.hip,
// attn_mha.hip and attn_latent.hip. Nothing on the enqueue paths allocates
// or synchronises, so hs_resolve and hs_sparse_attn can be captured in a
// hipGraph (section 5: the resolve step lives inside the decode graph).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "hs_device.h"

using hs::UnitDesc;

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hs_status hip_fail(hipError_t e, const char *what) {
  return fail(HS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HS_HIP(call)                              \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

hs_tuning g_tuning = {0, 0, 0, 0, 0, 0, {0, 0}};

inline hipStream_t S(void *s) { return (hipStream_t)s; }

// Event pairs of the kernel tracer.
constexpr int TRACE_CAP = 4096;
struct TraceState {
  bool on = false;
  std::vector<hipEvent_t> begin, end;
  std::vector<int> cls;
  int n = 0;        // pairs handed to launches
  int64_t dropped = 0;
};
TraceState g_trace;

}  // namespace

namespace hs {

bool trace_claim(int cls, hipEvent_t *start, hipEvent_t *stop) {
  if (!g_trace.on) return false;
  if (g_trace.n >= TRACE_CAP) {
    ++g_trace.dropped;
    return false;
  }
  *start = g_trace.begin[g_trace.n];
  *stop = g_trace.end[g_trace.n];
  g_trace.cls[g_trace.n] = cls;
  ++g_trace.n;
  return true;
}

}  // namespace hs

struct hs_pool_s {
  int32_t R = 0, L = 0, kind = 0, dtype = 0, Hkv = 0, D = 0, Dl = 0, Dr = 0;
  size_t rec = 0;
  int32_t page_shift = 0;      // records per page: 1 << page_shift
  std::vector<int64_t> cap;    // records allocated per request (whole pages)
  std::vector<int64_t> max_cap;
  // per request, per page: one pinned allocation holding that page of every
  // layer, layer-major (layer l's records at l * page_records * rec)
  std::vector<std::vector<uint8_t *>> host, dev;
  std::vector<int64_t> max_pages;   // page-table entries per unit of request r
  std::vector<size_t> table_off;    // entry offset of request r's tables
  uint64_t *d_pages = nullptr;      // device page tables of every unit
  int64_t *d_len = nullptr;         // [R * L]
  std::vector<int64_t> shadow;      // lengths as of the calls made so far
  std::vector<uint8_t> shadow_known; // 0 once a device-position append (whose
                                     // count of replays the host cannot know) ran
  std::vector<uint64_t> gen;         // per request: bumped when its pages are released
  uint64_t epoch = 0;               // bumped when a buffer of the pool moves (grows)
  int device = 0;
  int64_t page_records() const { return (int64_t)1 << page_shift; }
};

struct hs_buffer_s {
  hs_pool_t pool = nullptr;
  int32_t req = 0, layer = 0, B = 0;
  hs_buffer_s *base = nullptr;  // owner of the shared state, if not this one
  int32_t n_members = 0;        // live buffers sharing this one's state
  uint8_t *mem = nullptr;
  hs::BufferLayout lay{};
  UnitDesc desc{};
  UnitDesc *d_desc = nullptr;  // single-unit table (state restore)
  int32_t *d_inv = nullptr;    // inverse page table this buffer owns (not for a
                               // buffer sharing another's state)
  uint64_t gen = 0;            // the request's generation when the state was
                               // last made empty or restored (state owner only)
  hs_buffer_s *owner() { return base ? base : this; }
};

struct hs_batch_s {
  hs_pool_t pool = nullptr;
  int32_t n = 0, min_B = 0, max_B = 0;
  bool shared_twice = false;  // two units share one state (not resolvable)
  bool unit_twice = false;    // two units of one (request, layer) (no batch append)
  std::vector<hs_buffer_s *> bufs;
  uint64_t epoch = 0;         // the pool's epoch when the table was made
  UnitDesc *d_units = nullptr;
};

extern "C" {

const char *hs_status_str(hs_status s) {
  switch (s) {
    case HS_OK: return "ok";
    case HS_E_INVAL: return "invalid argument";
    case HS_E_RANGE: return "out of range";
    case HS_E_NOMEM: return "out of memory";
    case HS_E_HIP: return "HIP runtime error";
    case HS_E_DEVICE: return "data error reported by the device";
    case HS_E_STATE: return "invalid buffer state";
    default: return "unknown status";
  }
}

const char *hs_last_error(void) { return g_last_error.c_str(); }

hs_status hs_set_tuning(const hs_tuning *t) {
  if (!t) return fail(HS_E_INVAL, "null tuning");
  if (t->attn_splits < 0 || t->attn_splits > 4096)
    return fail(HS_E_INVAL, "tuning value out of range");
  const int hpw = t->latent_heads_per_wg;
  if (hpw != 0 && hpw != 32 && hpw != 64)
    return fail(HS_E_INVAL, "latent_heads_per_wg must be 0, 32 or 64");
  if (t->prefetch_workgroups < 0 || t->prefetch_workgroups > 65536)
    return fail(HS_E_INVAL, "prefetch_workgroups outside [0, 65536]");
  const int pb = t->prefetch_batch;
  if (pb != 0 && pb != 1 && pb != 2 && pb != 4 && pb != 8)
    return fail(HS_E_INVAL, "prefetch_batch must be 0, 1, 2, 4 or 8");
  const int gb = t->gather_bytes_per_lane;
  if (gb != 0 && gb != 16 && gb != 32 && gb != 64 && gb != 128)
    return fail(HS_E_INVAL, "gather_bytes_per_lane must be 0, 16, 32, 64 or 128");
  if (t->resolve_fetch < 0 || t->resolve_fetch > 2)
    return fail(HS_E_INVAL, "resolve_fetch must be 0, 1 or 2");
  g_tuning = *t;
  return HS_OK;
}

hs_status hs_get_tuning(hs_tuning *t) {
  if (!t) return fail(HS_E_INVAL, "null tuning");
  *t = g_tuning;
  return HS_OK;
}

// ------------------------------------------------------------------- pool

static hs_status check_unit(hs_pool_t p, int32_t req, int32_t layer) {
  if (!p) return fail(HS_E_INVAL, "null pool");
  if (req < 0 || req >= p->R || layer < 0 || layer >= p->L)
    return fail(HS_E_RANGE, "unit (%d, %d) outside %d x %d", req, layer, p->R, p->L);
  return HS_OK;
}

// Page table of unit (req, layer) in device memory.
static uint64_t *unit_table(hs_pool_t p, int32_t req, int32_t layer) {
  return p->d_pages + p->table_off[req] + (size_t)layer * p->max_pages[req];
}

static size_t page_bytes(hs_pool_t p) { return (size_t)p->page_records() * p->rec; }

// Host address of record pos of unit (req, layer); pos < cap[req].
static uint8_t *record_host(hs_pool_t p, int32_t req, int32_t layer, int64_t pos) {
  const int64_t pg = pos >> p->page_shift, in = pos & (p->page_records() - 1);
  return p->host[req][pg] + ((size_t)layer * p->page_records() + (size_t)in) * p->rec;
}

// Allocates request req's pages up to `records` (whole pages) and enters
// them in its units' device page tables. Synchronous. All or nothing: on a
// failure the pages of this call are freed and the pool is as before (the
// table entries past the capacity are never read: positions are checked
// against lengths <= the capacity).
static hs_status reserve_pages(hs_pool_t p, int32_t req, int64_t records) {
  const int64_t need = (records + p->page_records() - 1) >> p->page_shift;
  const int64_t have = (int64_t)p->host[req].size();
  if (need <= have) return HS_OK;
  const size_t pb = page_bytes(p);
  std::vector<uint8_t *> nh, nd;  // this call's pages: host and device addresses
  auto undo = [&nh]() {
    for (auto h : nh) (void)hipHostFree(h);
  };
  for (int64_t g = have; g < need; ++g) {
    void *h = nullptr;
    hipError_t e = hipHostMalloc(&h, pb * p->L, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess || !h) {
      undo();
      return fail(HS_E_NOMEM, "hipHostMalloc(%zu bytes) for request %d: %s", pb * p->L, req,
                  hipGetErrorString(e));
    }
    nh.push_back((uint8_t *)h);
    void *dp = nullptr;
    e = hipHostGetDevicePointer(&dp, h, 0);
    if (e != hipSuccess) {
      undo();
      return hip_fail(e, "hipHostGetDevicePointer");
    }
    nd.push_back((uint8_t *)dp);
  }
  std::vector<uint64_t> entries((size_t)(need - have));
  for (int l = 0; l < p->L; ++l) {
    for (int64_t g = 0; g < need - have; ++g)
      entries[(size_t)g] = (uint64_t)(uintptr_t)(nd[(size_t)g] + (size_t)l * pb);
    hipError_t e = hipMemcpy(unit_table(p, req, l) + have, entries.data(),
                             sizeof(uint64_t) * entries.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      undo();
      return hip_fail(e, "page table upload");
    }
  }
  p->host[req].insert(p->host[req].end(), nh.begin(), nh.end());
  p->dev[req].insert(p->dev[req].end(), nd.begin(), nd.end());
  p->cap[req] = need << p->page_shift;
  return HS_OK;
}

static void pool_free(hs_pool_t p) {
  for (auto &v : p->host)
    for (auto h : v)
      if (h) (void)hipHostFree(h);
  if (p->d_pages) (void)hipFree(p->d_pages);
  if (p->d_len) (void)hipFree(p->d_len);
  delete p;
}

hs_status hs_pool_create(const hs_pool_desc *d, hs_pool_t *out) {
  if (!d || !out) return fail(HS_E_INVAL, "null argument");
  *out = nullptr;
  if (d->n_requests < 1 || d->n_layers < 1 || !d->capacity_tokens)
    return fail(HS_E_INVAL, "need n_requests, n_layers >= 1 and capacities");
  if (d->dtype != HS_F32 && d->dtype != HS_BF16) return fail(HS_E_INVAL, "bad dtype");
  const size_t es = d->dtype == HS_F32 ? 4 : 2;
  size_t rec;
  if (d->kind == HS_KV_MHA) {
    if (d->n_kv_heads < 1 || d->head_dim < 1) return fail(HS_E_INVAL, "bad MHA shape");
    rec = 2 * (size_t)d->n_kv_heads * d->head_dim * es;
  } else if (d->kind == HS_KV_LATENT) {
    if (d->latent_dim < 1 || d->rope_dim < 0) return fail(HS_E_INVAL, "bad latent shape");
    rec = ((size_t)d->latent_dim + d->rope_dim) * es;
  } else {
    return fail(HS_E_INVAL, "bad kind");
  }
  if (rec % 16) return fail(HS_E_INVAL, "record bytes %zu not a multiple of 16", rec);
  int64_t largest = 1;
  for (int r = 0; r < d->n_requests; ++r) {
    const int64_t c = d->capacity_tokens[r];
    const int64_t m = d->max_tokens ? d->max_tokens[r] : c;
    if (c < 1 || m < c || m > 0x7FFFFFFF)
      return fail(HS_E_INVAL, "request %d: need 1 <= capacity <= max < 2^31", r);
    largest = std::max(largest, m);
  }
  int shift = 0;
  if (d->page_tokens > 0) {
    if (d->page_tokens & (d->page_tokens - 1))
      return fail(HS_E_INVAL, "page_tokens %d is not a power of two", d->page_tokens);
    while ((1 << shift) < d->page_tokens) ++shift;
  } else {  // 65536 records, or the largest request rounded up to a power of two
    while (shift < 16 && ((int64_t)1 << shift) < largest) ++shift;
  }
  if ((size_t)1 << shift > ((size_t)1 << 40) / rec)
    return fail(HS_E_INVAL, "page of %lld records too large", (long long)1 << shift);

  hs_pool_s *p = new (std::nothrow) hs_pool_s;
  if (!p) return fail(HS_E_NOMEM, "pool handle");
  p->R = d->n_requests;
  p->L = d->n_layers;
  p->kind = d->kind;
  p->dtype = d->dtype;
  p->Hkv = d->n_kv_heads;
  p->D = d->head_dim;
  p->Dl = d->latent_dim;
  p->Dr = d->rope_dim;
  p->rec = rec;
  p->page_shift = shift;
  p->cap.assign(p->R, 0);
  p->max_cap.resize(p->R);
  p->host.resize(p->R);
  p->dev.resize(p->R);
  p->max_pages.resize(p->R);
  p->table_off.resize(p->R);
  p->shadow.assign((size_t)p->R * p->L, 0);
  p->shadow_known.assign((size_t)p->R * p->L, 1);
  p->gen.assign(p->R, 0);
  (void)hipGetDevice(&p->device);
  size_t entries = 0;
  for (int r = 0; r < p->R; ++r) {
    p->max_cap[r] = d->max_tokens ? d->max_tokens[r] : d->capacity_tokens[r];
    p->max_pages[r] = (p->max_cap[r] + p->page_records() - 1) >> shift;
    p->table_off[r] = entries;
    entries += (size_t)p->L * p->max_pages[r];
  }
  hipError_t e = hipMalloc(&p->d_pages, sizeof(uint64_t) * entries);
  if (e == hipSuccess) e = hipMemset(p->d_pages, 0, sizeof(uint64_t) * entries);
  if (e == hipSuccess) e = hipMalloc(&p->d_len, sizeof(int64_t) * p->R * p->L);
  if (e == hipSuccess) e = hipMemset(p->d_len, 0, sizeof(int64_t) * p->R * p->L);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    pool_free(p);
    return fail(HS_E_NOMEM, "pool tables: %s", hipGetErrorString(e));
  }
  for (int r = 0; r < p->R; ++r) {
    hs_status s = reserve_pages(p, r, d->capacity_tokens[r]);
    if (s) {
      pool_free(p);
      return s;
    }
  }
  *out = p;
  return HS_OK;
}

hs_status hs_pool_destroy(hs_pool_t p) {
  if (!p) return fail(HS_E_INVAL, "null pool");
  pool_free(p);
  return HS_OK;
}

hs_status hs_pool_record_bytes(hs_pool_t p, size_t *rec) {
  if (!p || !rec) return fail(HS_E_INVAL, "null argument");
  *rec = p->rec;
  return HS_OK;
}

hs_status hs_pool_capacity(hs_pool_t p, int32_t req, int64_t *capacity, int64_t *max_tokens,
                           int64_t *page_tokens) {
  hs_status s = check_unit(p, req, 0);
  if (s) return s;
  if (capacity) *capacity = p->cap[req];
  if (max_tokens) *max_tokens = p->max_cap[req];
  if (page_tokens) *page_tokens = p->page_records();
  return HS_OK;
}

hs_status hs_pool_reserve(hs_pool_t p, int32_t req, int64_t records) {
  hs_status s = check_unit(p, req, 0);
  if (s) return s;
  if (records < 0 || records > p->max_cap[req])
    return fail(HS_E_RANGE, "request %d: %lld records above its maximum %lld", req,
                (long long)records, (long long)p->max_cap[req]);
  return reserve_pages(p, req, records);
}

hs_status hs_pool_release(hs_pool_t p, int32_t req) {
  hs_status s = check_unit(p, req, 0);
  if (s) return s;
  HS_HIP(hipDeviceSynchronize());  // no kernel may still read these pages
  // lengths first (every later access is checked against them), then the
  // page-table entries, then the memory
  for (int l = 0; l < p->L; ++l) {
    const size_t ui = (size_t)req * p->L + l;
    HS_HIP(hipMemset(p->d_len + ui, 0, sizeof(int64_t)));
    p->shadow[ui] = 0;
    p->shadow_known[ui] = 1;
  }
  ++p->gen[req];  // the request's buffers must be reset before they resolve again
  HS_HIP(hipMemset(unit_table(p, req, 0), 0,
                   sizeof(uint64_t) * (size_t)p->L * (size_t)p->max_pages[req]));
  HS_HIP(hipDeviceSynchronize());
  for (auto h : p->host[req]) (void)hipHostFree(h);
  p->host[req].clear();
  p->dev[req].clear();
  p->cap[req] = 0;
  return HS_OK;
}

hs_status hs_pool_record_ptr(hs_pool_t p, int32_t req, int32_t layer, int64_t pos,
                             void **host_ptr, size_t *rec_bytes) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (pos < 0 || pos >= p->cap[req])
    return fail(HS_E_RANGE, "position %lld outside the capacity %lld", (long long)pos,
                (long long)p->cap[req]);
  if (host_ptr) *host_ptr = record_host(p, req, layer, pos);
  if (rec_bytes) *rec_bytes = p->rec;
  return HS_OK;
}

hs_status hs_pool_page_ptr(hs_pool_t p, int32_t req, int32_t layer, int64_t page,
                           void **host_ptr) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (page < 0 || page >= (int64_t)p->host[req].size())
    return fail(HS_E_RANGE, "page %lld of request %d not allocated", (long long)page, req);
  if (host_ptr) *host_ptr = record_host(p, req, layer, page << p->page_shift);
  return HS_OK;
}

hs_status hs_pool_length(hs_pool_t p, int32_t req, int32_t layer, int64_t *len) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (!len) return fail(HS_E_INVAL, "null len");
  HS_HIP(hipDeviceSynchronize());
  HS_HIP(hipMemcpy(len, p->d_len + (size_t)req * p->L + layer, sizeof(int64_t),
                   hipMemcpyDeviceToHost));
  const size_t ui = (size_t)req * p->L + layer;
  p->shadow[ui] = *len;
  p->shadow_known[ui] = 1;
  return HS_OK;
}

hs_status hs_pool_set_length(hs_pool_t p, int32_t req, int32_t layer, int64_t len) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (len < 0 || len > p->cap[req])
    return fail(HS_E_RANGE, "length %lld outside [0, %lld]", (long long)len,
                (long long)p->cap[req]);
  HS_HIP(hipDeviceSynchronize());
  HS_HIP(hipMemcpy(p->d_len + (size_t)req * p->L + layer, &len, sizeof(int64_t),
                   hipMemcpyHostToDevice));
  HS_HIP(hipDeviceSynchronize());
  p->shadow[(size_t)req * p->L + layer] = len;
  p->shadow_known[(size_t)req * p->L + layer] = 1;
  return HS_OK;
}

hs_status hs_pool_append(hs_pool_t p, int32_t req, int32_t layer, int64_t pos, int64_t n,
                         const void *src, int32_t src_on_device, void *stream) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (n < 0 || (n > 0 && !src)) return fail(HS_E_INVAL, "bad source");
  const size_t ui = (size_t)req * p->L + layer;
  if (!p->shadow_known[ui]) {
    // device-position appends ran: read the length the device has now
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HS_HIP(hipStreamIsCapturing(S(stream), &cs));
    if (cs != hipStreamCaptureStatusNone)
      return fail(HS_E_INVAL, "unit (%d, %d): length unknown after device-position appends; "
                              "read it (hs_pool_length) before capture", req, layer);
    HS_HIP(hipStreamSynchronize(S(stream)));
    int64_t len = 0;
    hs_status ls = hs_pool_length(p, req, layer, &len);
    if (ls) return ls;
  }
  if (pos < 0 || pos > p->shadow[ui] || n > p->cap[req] || pos + n > p->cap[req])
    return fail(HS_E_RANGE, "append [%lld, %lld) with length %lld, capacity %lld",
                (long long)pos, (long long)(pos + n), (long long)p->shadow[ui],
                (long long)p->cap[req]);
  if (n == 0) return HS_OK;
  const int64_t new_len = std::max(p->shadow[ui], pos + n);
  if (src_on_device) {
    if ((uintptr_t)src % 16) return fail(HS_E_INVAL, "device source must be 16-byte aligned");
    hipError_t e = hs::launch_append(unit_table(p, req, layer), p->page_shift, pos, n,
                                     (int)p->rec, (const uint8_t *)src, p->d_len + ui, new_len,
                                     S(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
  } else {
    HS_HIP(hipStreamSynchronize(S(stream)));
    const uint8_t *in = (const uint8_t *)src;
    for (int64_t q = pos; q < pos + n;) {  // one run per page
      const int64_t end = std::min(pos + n, ((q >> p->page_shift) + 1) << p->page_shift);
      memcpy(record_host(p, req, layer, q), in, (size_t)(end - q) * p->rec);
      in += (size_t)(end - q) * p->rec;
      q = end;
    }
    HS_HIP(hipMemcpyAsync(p->d_len + ui, &new_len, sizeof(int64_t), hipMemcpyHostToDevice,
                          S(stream)));
    HS_HIP(hipStreamSynchronize(S(stream)));
  }
  p->shadow[ui] = new_len;
  return HS_OK;
}

hs_status hs_pool_append_batch(hs_batch_t b, const void *d_src, void *stream) {
  if (!b || !d_src) return fail(HS_E_INVAL, "null argument");
  if (b->epoch != b->pool->epoch)
    return fail(HS_E_INVAL, "a buffer of the pool grew after this batch was made");
  if (b->unit_twice) return fail(HS_E_INVAL, "the batch holds two buffers of one unit");
  if ((uintptr_t)d_src % 16) return fail(HS_E_INVAL, "source must be 16-byte aligned");
  hs_pool_t p = b->pool;
  hipError_t e = hs::launch_append_batch(b->d_units, b->n, (int)p->rec, (const uint8_t *)d_src,
                                         S(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  for (int i = 0; i < b->n; ++i)
    p->shadow_known[(size_t)b->bufs[i]->req * p->L + b->bufs[i]->layer] = 0;
  return HS_OK;
}

// ----------------------------------------------------------------- buffers

size_t hs_buffer_bytes(hs_pool_t p, int32_t B) {
  if (!p || B < 1) return 0;
  return hs::buffer_layout(p->rec, B).total;
}

hs_status hs_buffer_create(hs_pool_t p, int32_t req, int32_t layer, int32_t B, void *d_mem,
                           size_t bytes, void *stream, hs_buffer_t *out) {
  hs_status s = check_unit(p, req, layer);
  if (s) return s;
  if (!out || !d_mem) return fail(HS_E_INVAL, "null argument");
  *out = nullptr;
  if (B < 1) return fail(HS_E_INVAL, "B must be >= 1");
  if ((uintptr_t)d_mem % 256) return fail(HS_E_INVAL, "buffer memory must be 256-byte aligned");
  const hs::BufferLayout lay = hs::buffer_layout(p->rec, B);
  if (bytes < lay.total)
    return fail(HS_E_INVAL, "buffer needs %zu bytes, got %zu", lay.total, bytes);
  hs_buffer_s *b = new (std::nothrow) hs_buffer_s;
  if (!b) return fail(HS_E_NOMEM, "buffer handle");
  b->pool = p;
  b->req = req;
  b->layer = layer;
  b->B = B;
  b->mem = (uint8_t *)d_mem;
  b->lay = lay;
  b->gen = p->gen[req];
  UnitDesc &d = b->desc;
  d.rows = b->mem + lay.rows;
  d.pos = (int32_t *)(b->mem + lay.pos);
  d.stamp = (uint32_t *)(b->mem + lay.stamp);
  d.work = (int2 *)(b->mem + lay.work);
  d.fsrc = (int32_t *)(b->mem + lay.fsrc);
  d.ctl = (uint32_t *)(b->mem + lay.ctl);
  d.pages = unit_table(p, req, layer);
  d.len = p->d_len + (size_t)req * p->L + layer;
  d.B = B;
  d.page_shift = p->page_shift;
  d.n_pages = (int32_t)p->max_pages[req];
  // the inverse page table covers every position the request can reach
  d.inv_len = (int32_t)std::max<int64_t>(1, p->max_cap[req]);
  hipError_t e = hipMalloc(&b->d_inv, sizeof(int32_t) * (size_t)d.inv_len);
  d.inv = b->d_inv;
  if (e == hipSuccess) e = hipMalloc(&b->d_desc, sizeof(UnitDesc));
  if (e == hipSuccess)
    e = hipMemcpy(b->d_desc, &b->desc, sizeof(UnitDesc), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hs::launch_buffer_init(d.pos, d.stamp, d.fsrc, d.ctl, B, S(stream));
  if (e == hipSuccess) e = hs::launch_inv_clear(d.inv, d.inv_len, S(stream));
  if (e != hipSuccess) {
    if (b->d_desc) (void)hipFree(b->d_desc);
    if (b->d_inv) (void)hipFree(b->d_inv);
    delete b;
    return hip_fail(e, "buffer create");
  }
  *out = b;
  return HS_OK;
}

size_t hs_buffer_shared_bytes(hs_pool_t p, int32_t B) {
  if (!p || B < 1) return 0;
  return hs::align_up((size_t)B * p->rec, 256);
}

hs_status hs_buffer_create_shared(hs_buffer_t base, int32_t layer, void *d_mem, size_t bytes,
                                  hs_buffer_t *out) {
  if (!base || !out || !d_mem) return fail(HS_E_INVAL, "null argument");
  *out = nullptr;
  hs_pool_t p = base->pool;
  hs_status s = check_unit(p, base->req, layer);
  if (s) return s;
  if ((uintptr_t)d_mem % 256) return fail(HS_E_INVAL, "buffer memory must be 256-byte aligned");
  const size_t need = hs_buffer_shared_bytes(p, base->B);
  if (bytes < need) return fail(HS_E_INVAL, "shared buffer needs %zu bytes, got %zu", need, bytes);
  hs_buffer_s *b = new (std::nothrow) hs_buffer_s;
  if (!b) return fail(HS_E_NOMEM, "buffer handle");
  b->pool = p;
  b->req = base->req;
  b->layer = layer;
  b->B = base->B;
  b->mem = (uint8_t *)d_mem;
  b->lay = base->lay;
  // the group's state (page table, stamps, fetch list, control words) is
  // base's; rows, pool records and length are this layer's
  b->base = base->base ? base->base : base;
  b->desc = base->desc;
  b->desc.rows = b->mem;
  b->desc.pages = unit_table(p, b->req, layer);
  b->desc.len = p->d_len + (size_t)b->req * p->L + layer;
  hipError_t e = hipMalloc(&b->d_desc, sizeof(UnitDesc));
  if (e == hipSuccess)
    e = hipMemcpy(b->d_desc, &b->desc, sizeof(UnitDesc), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (b->d_desc) (void)hipFree(b->d_desc);
    delete b;
    return hip_fail(e, "shared buffer create");
  }
  ++b->base->n_members;
  *out = b;
  return HS_OK;
}

hs_status hs_buffer_destroy(hs_buffer_t b) {
  if (!b) return fail(HS_E_INVAL, "null buffer");
  if (b->n_members > 0)
    return fail(HS_E_INVAL, "%d shared buffers still use this buffer's state", b->n_members);
  if (b->base) --b->base->n_members;
  if (b->d_desc) (void)hipFree(b->d_desc);
  if (b->d_inv) (void)hipFree(b->d_inv);
  delete b;
  return HS_OK;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uint8_t *a0 = (const uint8_t *)a, *b0 = (const uint8_t *)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Checks new memory for a buffer that grows to new_B (full state when rows_only
// is false, rows only for a member of a layer group).
static hs_status check_grow_mem(const hs_buffer_s *b, int32_t new_B, const void *d_mem,
                                size_t bytes, bool rows_only) {
  if (!d_mem) return fail(HS_E_INVAL, "null memory");
  if ((uintptr_t)d_mem % 256) return fail(HS_E_INVAL, "buffer memory must be 256-byte aligned");
  const size_t need = rows_only ? hs_buffer_shared_bytes(b->pool, new_B)
                                : hs::buffer_layout(b->pool->rec, new_B).total;
  if (bytes < need) return fail(HS_E_INVAL, "buffer needs %zu bytes, got %zu", need, bytes);
  const size_t old = rows_only ? hs_buffer_shared_bytes(b->pool, b->B) : b->lay.total;
  if (overlaps(d_mem, need, b->mem, old))
    return fail(HS_E_INVAL, "new memory overlaps the buffer's");
  return HS_OK;
}

// Enqueues the move of b's rows [0, B) to nm, and unless rows_only, of its
// metadata into the layout for new_B, with slots [B, new_B) made empty.
static hs_status enqueue_move(const hs_buffer_s *b, int32_t new_B, uint8_t *nm, bool rows_only,
                              hipStream_t st) {
  const size_t rec = b->pool->rec, B = (size_t)b->B;
  HS_HIP(hipMemcpyAsync(nm, b->desc.rows, B * rec, hipMemcpyDeviceToDevice, st));
  if (rows_only) return HS_OK;
  const hs::BufferLayout lay = hs::buffer_layout(rec, new_B);
  HS_HIP(hipMemcpyAsync(nm + lay.pos, b->mem + b->lay.pos, B * 4, hipMemcpyDeviceToDevice, st));
  HS_HIP(hipMemcpyAsync(nm + lay.stamp, b->mem + b->lay.stamp, B * 4, hipMemcpyDeviceToDevice, st));
  HS_HIP(hipMemcpyAsync(nm + lay.work, b->mem + b->lay.work, B * 8, hipMemcpyDeviceToDevice, st));
  HS_HIP(hipMemcpyAsync(nm + lay.fsrc, b->mem + b->lay.fsrc, B * 4, hipMemcpyDeviceToDevice, st));
  HS_HIP(hipMemcpyAsync(nm + lay.ctl, b->mem + b->lay.ctl, hs::CTL_WORDS * 4,
                        hipMemcpyDeviceToDevice, st));
  if ((size_t)new_B > B) {
    hipError_t e = hs::launch_buffer_init((int32_t *)(nm + lay.pos) + B,
                                          (uint32_t *)(nm + lay.stamp) + B,
                                          (int32_t *)(nm + lay.fsrc) + B, nullptr,
                                          new_B - (int32_t)B, st);
    if (e != hipSuccess) return hip_fail(e, "grow init");
  }
  return HS_OK;
}

// Points base (full state in nm) and its members (rows in member_mem[i]) at
// their new memory and uploads their descriptors.
static hs_status commit_move(hs_buffer_s *base, int32_t new_B, uint8_t *nm,
                             hs_buffer_s *const *members, void *const *member_mem, int32_t n) {
  const hs::BufferLayout lay = hs::buffer_layout(base->pool->rec, new_B);
  UnitDesc d = base->desc;
  d.rows = nm + lay.rows;
  d.pos = (int32_t *)(nm + lay.pos);
  d.stamp = (uint32_t *)(nm + lay.stamp);
  d.work = (int2 *)(nm + lay.work);
  d.fsrc = (int32_t *)(nm + lay.fsrc);
  d.ctl = (uint32_t *)(nm + lay.ctl);
  d.B = new_B;
  HS_HIP(hipMemcpy(base->d_desc, &d, sizeof(UnitDesc), hipMemcpyHostToDevice));
  base->desc = d;
  base->mem = nm;
  base->lay = lay;
  base->B = new_B;
  for (int32_t i = 0; i < n; ++i) {
    hs_buffer_s *m = members[i];
    UnitDesc md = d;  // the group's state, this member's rows and pool records
    md.rows = (uint8_t *)member_mem[i];
    md.pages = m->desc.pages;
    md.len = m->desc.len;
    HS_HIP(hipMemcpy(m->d_desc, &md, sizeof(UnitDesc), hipMemcpyHostToDevice));
    m->desc = md;
    m->mem = (uint8_t *)member_mem[i];
    m->lay = lay;
    m->B = new_B;
  }
  ++base->pool->epoch;  // batch tables made before describe the old memory
  return HS_OK;
}

hs_status hs_buffer_grow(hs_buffer_t b, int32_t new_B, void *d_mem, size_t bytes,
                         void *stream) {
  if (!b || !d_mem) return fail(HS_E_INVAL, "null argument");
  if (b->base || b->n_members > 0)
    return fail(HS_E_INVAL, "a buffer whose state is shared grows with hs_buffer_grow_group");
  if (new_B < b->B || new_B > HS_MAX_B)
    return fail(HS_E_INVAL, "new B = %d outside [%d, %d]", new_B, b->B, HS_MAX_B);
  hs_status s = check_grow_mem(b, new_B, d_mem, bytes, false);
  if (s) return s;
  hipStream_t st = S(stream);
  s = enqueue_move(b, new_B, (uint8_t *)d_mem, false, st);
  if (s) return s;
  HS_HIP(hipStreamSynchronize(st));
  return commit_move(b, new_B, (uint8_t *)d_mem, nullptr, nullptr, 0);
}

hs_status hs_buffer_grow_group(hs_buffer_t base, const hs_buffer_t *members,
                               int32_t n_members, int32_t new_B, void *d_mem, size_t bytes,
                               void *const *member_mem, const size_t *member_bytes,
                               void *stream) {
  if (!base || !d_mem || (n_members > 0 && (!members || !member_mem || !member_bytes)))
    return fail(HS_E_INVAL, "null argument");
  if (base->base) return fail(HS_E_INVAL, "base is itself a member of a group");
  if (n_members != base->n_members)
    return fail(HS_E_INVAL, "the group has %d members, %d given", base->n_members, n_members);
  if (new_B < base->B || new_B > HS_MAX_B)
    return fail(HS_E_INVAL, "new B = %d outside [%d, %d]", new_B, base->B, HS_MAX_B);
  hs_status s = check_grow_mem(base, new_B, d_mem, bytes, false);
  if (s) return s;
  const size_t full = hs::buffer_layout(base->pool->rec, new_B).total;
  const size_t rows = hs_buffer_shared_bytes(base->pool, new_B);
  for (int32_t i = 0; i < n_members; ++i) {
    const hs_buffer_s *m = members[i];
    if (!m || m->base != base) return fail(HS_E_INVAL, "member %d is not in base's group", i);
    for (int32_t j = 0; j < i; ++j)
      if (members[j] == m) return fail(HS_E_INVAL, "member %d is listed twice", i);
    s = check_grow_mem(m, new_B, member_mem[i], member_bytes[i], true);
    if (s) return s;
    // new regions must not overlap one another or any memory the move reads
    if (overlaps(member_mem[i], rows, d_mem, full) ||
        overlaps(member_mem[i], rows, base->mem, base->lay.total))
      return fail(HS_E_INVAL, "member %d's new memory overlaps the group's", i);
    for (int32_t j = 0; j < n_members; ++j) {
      const size_t old_j = hs_buffer_shared_bytes(base->pool, members[j]->B);
      if ((j != i && overlaps(member_mem[i], rows, members[j]->mem, old_j)) ||
          (j < i && overlaps(member_mem[i], rows, member_mem[j], rows)))
        return fail(HS_E_INVAL, "member %d's new memory overlaps another member's", i);
    }
  }
  for (int32_t i = 0; i < n_members; ++i) {
    const size_t old_i = hs_buffer_shared_bytes(base->pool, members[i]->B);
    if (overlaps(d_mem, full, members[i]->mem, old_i))
      return fail(HS_E_INVAL, "new memory overlaps member %d's rows", i);
  }
  hipStream_t st = S(stream);
  s = enqueue_move(base, new_B, (uint8_t *)d_mem, false, st);
  for (int32_t i = 0; !s && i < n_members; ++i)
    s = enqueue_move(members[i], new_B, (uint8_t *)member_mem[i], true, st);
  HS_HIP(hipStreamSynchronize(st));
  if (s) return s;
  return commit_move(base, new_B, (uint8_t *)d_mem, members, member_mem, n_members);
}

hs_status hs_buffer_reset(hs_buffer_t b, void *stream) {
  if (!b) return fail(HS_E_INVAL, "null buffer");
  hipError_t e = hs::launch_buffer_init(b->desc.pos, b->desc.stamp, b->desc.fsrc, b->desc.ctl, b->B,
                                         S(stream));
  if (e == hipSuccess) e = hs::launch_inv_clear(b->desc.inv, b->desc.inv_len, S(stream));
  if (e != hipSuccess) return hip_fail(e, "buffer reset");
  b->owner()->gen = b->pool->gen[b->req];
  return HS_OK;
}

hs_status hs_buffer_rows(hs_buffer_t b, void **d_rows, size_t *rec_bytes) {
  if (!b) return fail(HS_E_INVAL, "null buffer");
  if (d_rows) *d_rows = b->desc.rows;
  if (rec_bytes) *rec_bytes = b->pool->rec;
  return HS_OK;
}

hs_status hs_buffer_state_get(hs_buffer_t b, int32_t *pos, uint32_t *stamp, uint32_t *clock,
                              int32_t *err, void *stream) {
  if (!b) return fail(HS_E_INVAL, "null buffer");
  uint32_t ctl[4];
  if (pos)
    HS_HIP(hipMemcpyAsync(pos, b->desc.pos, sizeof(int32_t) * b->B, hipMemcpyDeviceToHost,
                          S(stream)));
  if (stamp)
    HS_HIP(hipMemcpyAsync(stamp, b->desc.stamp, sizeof(uint32_t) * b->B, hipMemcpyDeviceToHost,
                          S(stream)));
  HS_HIP(hipMemcpyAsync(ctl, b->desc.ctl, sizeof ctl, hipMemcpyDeviceToHost, S(stream)));
  HS_HIP(hipStreamSynchronize(S(stream)));
  if (clock) *clock = ctl[hs::CTL_CLOCK];
  if (err) *err = (int32_t)ctl[hs::CTL_ERR];
  return HS_OK;
}

hs_status hs_buffer_state_set(hs_buffer_t b, const int32_t *pos, const uint32_t *stamp,
                              uint32_t clock, int32_t err, void *stream) {
  if (!b || !pos || !stamp) return fail(HS_E_INVAL, "null argument");
  int64_t len = 0;
  hs_status s = hs_pool_length(b->pool, b->req, b->layer, &len);
  if (s) return s;
  if (clock >= 0x7FFFFFFFu) return fail(HS_E_STATE, "clock %u exhausted", clock);
  std::vector<int32_t> seen;
  seen.reserve(b->B);
  for (int32_t i = 0; i < b->B; ++i) {
    if (pos[i] < -1 || (int64_t)pos[i] >= len)
      return fail(HS_E_STATE, "slot %d: position %d outside [-1, %lld)", i, pos[i],
                  (long long)len);
    if ((pos[i] < 0) != (stamp[i] == 0))
      return fail(HS_E_STATE, "slot %d: stamp must be 0 exactly when empty", i);
    if ((uint64_t)stamp[i] > 2ull * clock)
      return fail(HS_E_STATE, "slot %d: stamp %u newer than clock %u", i, stamp[i], clock);
    if (pos[i] >= 0) seen.push_back(pos[i]);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(HS_E_STATE, "a position is held by two slots");
  uint32_t ctl[hs::CTL_WORDS] = {0};
  ctl[hs::CTL_CLOCK] = clock;
  ctl[hs::CTL_ERR] = (uint32_t)err;
  HS_HIP(hipMemcpyAsync(b->desc.pos, pos, sizeof(int32_t) * b->B, hipMemcpyHostToDevice,
                        S(stream)));
  HS_HIP(hipMemcpyAsync(b->desc.stamp, stamp, sizeof(uint32_t) * b->B, hipMemcpyHostToDevice,
                        S(stream)));
  HS_HIP(hipMemcpyAsync(b->desc.ctl, ctl, sizeof ctl, hipMemcpyHostToDevice, S(stream)));
  hipError_t e = hs::launch_inv_rebuild(b->desc.inv, b->desc.inv_len, b->desc.pos, b->B,
                                        S(stream));
  if (e == hipSuccess) e = hs::launch_regather(b->d_desc, b->B, (int)b->pool->rec, S(stream));
  if (e != hipSuccess) return hip_fail(e, "regather");
  HS_HIP(hipStreamSynchronize(S(stream)));
  b->owner()->gen = b->pool->gen[b->req];
  return HS_OK;
}

// ----------------------------------------------------------------- batches

hs_status hs_batch_create(const hs_buffer_t *bufs, int32_t n, hs_batch_t *out) {
  if (!bufs || !out || n < 1) return fail(HS_E_INVAL, "need n >= 1 buffers");
  *out = nullptr;
  std::vector<UnitDesc> h(n);
  hs_pool_t pool = bufs[0] ? bufs[0]->pool : nullptr;
  int min_B = 0x7FFFFFFF, max_B = 0;
  for (int i = 0; i < n; ++i) {
    if (!bufs[i]) return fail(HS_E_INVAL, "null buffer %d", i);
    if (bufs[i]->pool != pool) return fail(HS_E_INVAL, "buffers of different pools");
    h[i] = bufs[i]->desc;
    min_B = std::min(min_B, bufs[i]->B);
    max_B = std::max(max_B, bufs[i]->B);
  }
  // a state (page table) named twice cannot be resolved by one launch
  std::vector<uintptr_t> states(n);
  for (int i = 0; i < n; ++i) states[i] = (uintptr_t)h[i].pos;
  std::sort(states.begin(), states.end());
  const bool shared_twice = std::adjacent_find(states.begin(), states.end()) != states.end();
  std::vector<int64_t> ids(n);
  for (int i = 0; i < n; ++i) ids[i] = (int64_t)bufs[i]->req * pool->L + bufs[i]->layer;
  std::sort(ids.begin(), ids.end());
  const bool unit_twice = std::adjacent_find(ids.begin(), ids.end()) != ids.end();
  hs_batch_s *bt = new (std::nothrow) hs_batch_s;
  if (!bt) return fail(HS_E_NOMEM, "batch handle");
  bt->pool = pool;
  bt->n = n;
  bt->min_B = min_B;
  bt->max_B = max_B;
  bt->shared_twice = shared_twice;
  bt->unit_twice = unit_twice;
  bt->bufs.assign(bufs, bufs + n);
  bt->epoch = pool->epoch;
  hipError_t e = hipMalloc(&bt->d_units, sizeof(UnitDesc) * n);
  if (e == hipSuccess)
    e = hipMemcpy(bt->d_units, h.data(), sizeof(UnitDesc) * n, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (bt->d_units) (void)hipFree(bt->d_units);
    delete bt;
    return hip_fail(e, "batch table");
  }
  *out = bt;
  return HS_OK;
}

hs_status hs_batch_destroy(hs_batch_t b) {
  if (!b) return fail(HS_E_INVAL, "null batch");
  if (b->d_units) (void)hipFree(b->d_units);
  delete b;
  return HS_OK;
}

// A batch made before a buffer of its pool moved describes freed memory; a
// buffer of a request whose pages were released since its state was last
// made empty (or restored) holds positions of the finished request.
static hs_status check_epoch(hs_batch_t b) {
  if (b->epoch != b->pool->epoch)
    return fail(HS_E_INVAL, "a buffer of the pool grew after this batch was made: create the "
                            "batch again");
  for (int i = 0; i < b->n; ++i) {
    hs_buffer_s *x = b->bufs[i];
    if (x->owner()->gen != b->pool->gen[x->req])
      return fail(HS_E_INVAL, "unit %d: request %d was released after its buffer's state was "
                              "set; reset the buffer (hs_buffer_reset) first", i, x->req);
  }
  return HS_OK;
}

hs_status hs_batch_status(hs_batch_t b, int32_t *errs, void *stream) {
  if (!b) return fail(HS_E_INVAL, "null batch");
  if (b->epoch != b->pool->epoch)
    return fail(HS_E_INVAL, "a buffer of the pool grew after this batch was made");
  HS_HIP(hipStreamSynchronize(S(stream)));
  bool any = false;
  for (int i = 0; i < b->n; ++i) {
    uint32_t e = 0;
    HS_HIP(hipMemcpy(&e, b->bufs[i]->desc.ctl + hs::CTL_ERR, sizeof e, hipMemcpyDeviceToHost));
    if (errs) errs[i] = (int32_t)e;
    any |= e != 0;
  }
  if (any) return fail(HS_E_DEVICE, "a unit of the batch has error bits set");
  return HS_OK;
}

// ----------------------------------------------------------------- resolve

static hs_status check_resolve(hs_batch_t b, const int32_t *d_topk, int32_t k,
                               const int32_t *d_slots) {
  if (!b || !d_topk || !d_slots) return fail(HS_E_INVAL, "null argument");
  if (check_epoch(b)) return HS_E_INVAL;
  if (b->shared_twice)
    return fail(HS_E_INVAL, "the batch holds two buffers of one shared state");
  if (k < 1 || k > HS_MAX_K || k > b->min_B)
    return fail(HS_E_INVAL, "k = %d outside [1, min(%d, smallest B = %d)]", k, HS_MAX_K,
                b->min_B);
  if (b->max_B > HS_MAX_B) return fail(HS_E_INVAL, "B = %d above %d", b->max_B, HS_MAX_B);
  static int lds_limit = -1;
  if (lds_limit < 0) {
    int dev = 0, v = 0;
    HS_HIP(hipGetDevice(&dev));
    HS_HIP(hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    lds_limit = v;
  }
  if (hs::resolve_lds_bytes(k) + 2048 > (size_t)lds_limit)
    return fail(HS_E_INVAL, "k = %d needs %zu bytes of LDS; the device allows %d", k,
                hs::resolve_lds_bytes(k) + 2048, lds_limit);
  return HS_OK;
}

hs_status hs_resolve(hs_batch_t b, const int32_t *d_topk, int32_t k, int32_t *d_slots,
                     int32_t *d_miss, void *stream) {
  hs_status s = check_resolve(b, d_topk, k, d_slots);
  if (s) return s;
  // one workgroup per unit cannot keep enough host reads in flight for the
  // link when the batch is small: fetch with a second, wider kernel there
  const int fetch = g_tuning.resolve_fetch == 1   ? hs::FETCH_INLINE
                    : g_tuning.resolve_fetch == 2 ? hs::FETCH_KERNEL
                    : b->n >= 4                   ? hs::FETCH_INLINE
                                                  : hs::FETCH_KERNEL;
  hipError_t e = hs::launch_resolve(b->d_units, b->n, b->max_B, d_topk, k, d_slots, d_miss,
                                    fetch, g_tuning.gather_bytes_per_lane / 16,
                                    (int)b->pool->rec, S(stream));
  if (e != hipSuccess) return hip_fail(e, "resolve launch");
  return HS_OK;
}

// --------------------------------------------------------------- attention

struct AttnPlan {
  int splits, chunk, dv;
  int hpw;  // latent: query heads per workgroup
  size_t ws_o_bytes, ws_ml_floats, ws_bytes;
};

static hs_status plan_attn(hs_batch_t b, int32_t Hq, int32_t k, AttnPlan *pl) {
  const hs_pool_s *p = b->pool;
  if (k < 1 || k > HS_MAX_K) return fail(HS_E_INVAL, "k = %d outside [1, %d]", k, HS_MAX_K);
  int base, min_chunk, target;
  if (p->kind == HS_KV_MHA) {
    if (p->D != 64 && p->D != 128) return fail(HS_E_INVAL, "head_dim %d unsupported", p->D);
    if (Hq < p->Hkv || Hq % p->Hkv) return fail(HS_E_INVAL, "n_q_heads %% n_kv_heads != 0");
    const int gq = Hq / p->Hkv;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8)
      return fail(HS_E_INVAL, "GQA group %d unsupported", gq);
    // splits until the grid reaches 512 workgroups (two per compute unit)
    // or a split would hold fewer than 64 slots; on the 32-request GQA
    // workload (256 (unit, KV head) pairs) 2 splits of 1024 slots measured
    // 2.4% faster per layer than 4 of 512
    base = b->n * p->Hkv;
    min_chunk = 64;
    target = 512;
    pl->dv = p->D;
  } else {
    if (p->dtype != HS_BF16 || p->Dl != 512 || p->Dr != 64)
      return fail(HS_E_INVAL, "latent attention needs bf16, 512 + 64");
    if (Hq != 16 && Hq != 32 && Hq != 64)
      return fail(HS_E_INVAL, "latent attention supports 16, 32 or 64 query heads");
    // A workgroup covers hpw = 32 or 64 heads (16 pad to 32) of a (unit,
    // split) and holds a compute unit. With 64 each row is copied once per
    // (unit, split); with 32 the two head groups copy it apart (the second
    // time mostly from L2), but a workgroup's epilogue writes half as many
    // partial bytes and the unit's work spreads over twice the workgroups,
    // which measured faster on both MLA workloads (batch 8: 21.5 against
    // 25.7 us with the combine; batch 64: 48.3 against 50.0), so 32 is the
    // default. Every split writes a 1 KB bf16 partial per head, which the
    // split-k combine reads back, so splits keep at least 128 rows and are
    // added until the grid reaches 256 workgroups (batch 8: 32 heads x 16
    // splits; batch 64: 32 x 2; 32 requests at k = 512: 32 x 4). Against 256
    // rows at least (8 and 2 splits on the first and last), attention plus
    // combine measured 18.6-19.5 against 20.0-20.6 us at batch 8 and 19.6
    // against 20.9-21.3 us on the 32 requests. With bf16 partials 64 heads x
    // 4 splits beat 32 x 2 at batch 64 when the same step's attention is
    // timed alone (44.0 against 46.3-47.7 us) but not inside the decode step
    // (47.7 against 47.6, the resolve having just written 45 MB of rows), and
    // lost at 8, 16 and 32 requests, so 32 stays the default.
    const int n8 = (b->n + 7) / 8 * 8;
    int hpw = g_tuning.latent_heads_per_wg;
    if (hpw <= 0 || Hq <= 32) hpw = 32;
    pl->hpw = hpw;
    base = n8 * ((Hq + hpw - 1) / hpw);
    min_chunk = 128;
    target = 256;
    pl->dv = p->Dl;
  }
  int splits = g_tuning.attn_splits > 0 ? g_tuning.attn_splits : (target + base - 1) / base;
  const int max_splits = std::max(1, k / min_chunk);
  if (g_tuning.attn_splits <= 0) splits = std::min(splits, max_splits);
  splits = std::max(1, std::min(std::min(splits, k), 64));  // the combine merges <= 64
  if (p->kind == HS_KV_LATENT)
    splits = std::max(splits, (k + hs::LAT_MAX_CHUNK - 1) / hs::LAT_MAX_CHUNK);
  int chunk = (k + splits - 1) / splits;
  if (p->kind == HS_KV_LATENT) chunk = (chunk + 63) / 64 * 64;  // whole pairs of 32-row tiles
  splits = (k + chunk - 1) / chunk;  // every split has at least one slot
  pl->splits = splits;
  pl->chunk = chunk;
  if (splits == 1) {
    pl->ws_o_bytes = pl->ws_ml_floats = 0;
    pl->ws_bytes = 0;
  } else {
    const size_t rows = (size_t)b->n * Hq;
    // partials: fp32 for MHA records, bf16 for latent ones (a latent split
    // writes 512 values per head, as many bytes in fp32 as two of its rows)
    pl->ws_o_bytes = rows * splits * pl->dv * (p->kind == HS_KV_LATENT ? 2 : 4);
    pl->ws_ml_floats = rows * splits * 2;
    pl->ws_bytes = hs::align_up(pl->ws_o_bytes, 256) + pl->ws_ml_floats * 4;
  }
  return HS_OK;
}

size_t hs_sparse_attn_workspace(hs_batch_t b, int32_t n_q_heads, int32_t k) {
  AttnPlan pl;
  if (!b || plan_attn(b, n_q_heads, k, &pl) != HS_OK) return 0;
  return pl.ws_bytes;
}

static hs_status check_attn(hs_batch_t b, const void *d_q, int32_t Hq, const int32_t *d_slots,
                            int32_t k, float sm_scale, float *d_out, void *d_ws, size_t ws_bytes,
                            AttnPlan *pl) {
  if (!b || !d_q || !d_slots || !d_out) return fail(HS_E_INVAL, "null argument");
  if (check_epoch(b)) return HS_E_INVAL;
  if (k > b->min_B) return fail(HS_E_INVAL, "k = %d above smallest B = %d", k, b->min_B);
  if (!(sm_scale > 0.f) || sm_scale == __builtin_huge_valf())
    return fail(HS_E_INVAL, "sm_scale must be positive and finite");
  if ((uintptr_t)d_q % 16 || (uintptr_t)d_out % 16)
    return fail(HS_E_INVAL, "q and out must be 16-byte aligned");
  hs_status s = plan_attn(b, Hq, k, pl);
  if (s) return s;
  if (pl->ws_bytes > 0 && (!d_ws || ws_bytes < pl->ws_bytes))
    return fail(HS_E_INVAL, "workspace needs %zu bytes, got %zu", pl->ws_bytes, ws_bytes);
  if (d_ws && (uintptr_t)d_ws % 256) return fail(HS_E_INVAL, "workspace must be 256-byte aligned");
  return HS_OK;
}

static hs_status enqueue_attn(hs_batch_t b, const void *d_q, int32_t Hq, const int32_t *d_slots,
                              int32_t k, float sm_scale, float *d_out, void *d_ws,
                              const AttnPlan &pl, int fetch, void *stream) {
  float *ws_ml = pl.ws_bytes ? (float *)((uint8_t *)d_ws + hs::align_up(pl.ws_o_bytes, 256))
                             : nullptr;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const hs_pool_s *p = b->pool;
  hipError_t e;
  if (p->kind == HS_KV_MHA) {
    hs::AttnMhaArgs a;
    a.units = b->d_units;
    a.q = d_q;
    a.slots = d_slots;
    a.n_units = b->n;
    a.k = k;
    a.Hq = Hq;
    a.Hkv = p->Hkv;
    a.D = p->D;
    a.dtype = p->dtype;
    a.splits = pl.splits;
    a.chunk = pl.chunk;
    a.rec_bytes = (int)p->rec;
    a.fetch = fetch;
    a.scale_log2 = scale_log2;
    a.ws_o = (float *)d_ws;
    a.ws_ml = ws_ml;
    a.out = d_out;
    e = hs::launch_attn_mha(a, S(stream));
  } else {
    hs::AttnLatentArgs a;
    a.units = b->d_units;
    a.q = (const uint16_t *)d_q;
    a.slots = d_slots;
    a.n_units = b->n;
    a.k = k;
    a.Hq = Hq;
    a.splits = pl.splits;
    a.chunk = pl.chunk;
    a.hpw = pl.hpw;
    a.scale_log2 = scale_log2;
    a.ws_o = (uint16_t *)d_ws;
    a.ws_ml = ws_ml;
    a.out = d_out;
    e = hs::launch_attn_latent(a, S(stream));
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return HS_OK;
}

hs_status hs_sparse_attn(hs_batch_t b, const void *d_q, int32_t Hq, const int32_t *d_slots,
                         int32_t k, float sm_scale, float *d_out, void *d_ws, size_t ws_bytes,
                         void *stream) {
  AttnPlan pl;
  hs_status s = check_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, d_ws, ws_bytes, &pl);
  if (s) return s;
  return enqueue_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, d_ws, pl, 0, stream);
}

}  // extern "C"

// ---------------------------------------------------- allocation-free attention
namespace {

// The split-k partials of hs_sparse_attn_noalloc: one array per GPU (each
// device holds its own copy of a __device__ variable). In host code the
// name is a host-side stand-in, never a device address: kernels get the
// address hipGetSymbolAddress returns for the current device.
__device__ __attribute__((aligned(256))) uint8_t scratch[HS_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[SCRATCH_MAX_DEVICES] = {};

// The current device's address of `scratch`, looked up once per device.
hs_status scratch_address(void **out) {
  int dev = 0;
  HS_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(HS_E_INVAL, "device %d beyond the %d this library serves", dev,
                SCRATCH_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HS_E_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_sparse_attn_noalloc(hs_batch_t b, const void *d_q, int32_t Hq,
                                 const int32_t *d_slots, int32_t k, float sm_scale, float *d_out,
                                 void *stream) {
  AttnPlan pl;
  if (!b) return fail(HS_E_INVAL, "null batch");
  // the plan alone first: its workspace size is checked against the scratch
  hs_status s = plan_attn(b, Hq, k, &pl);
  if (s) return s;
  if (pl.ws_bytes > HS_NOALLOC_SCRATCH_BYTES)
    return fail(HS_E_INVAL, "this attention needs %zu bytes of split-k scratch; the "
                            "allocation-free form holds %zu (use hs_sparse_attn with a workspace)",
                pl.ws_bytes, (size_t)HS_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (pl.ws_bytes > 0) {
    s = scratch_address(&ws);
    if (s) return s;
  }
  s = check_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, ws, HS_NOALLOC_SCRATCH_BYTES, &pl);
  if (s) return s;
  return enqueue_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, ws, pl, 0, stream);
}

hs_status hs_resolve_attn(hs_batch_t b, const int32_t *d_topk, int32_t k, int32_t *d_slots,
                          int32_t *d_miss, const void *d_q, int32_t Hq, float sm_scale,
                          float *d_out, void *d_ws, size_t ws_bytes, void *stream) {
  hs_status s = check_resolve(b, d_topk, k, d_slots);
  if (s) return s;
  AttnPlan pl;
  s = check_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, d_ws, ws_bytes, &pl);
  if (s) return s;
  if (b->pool->kind == HS_KV_LATENT) {
    // latent records: the resolve moves the misses (its first host reads
    // overlap the victim selection) and attention reads resident rows only
    s = hs_resolve(b, d_topk, k, d_slots, d_miss, stream);
    if (s) return s;
    return enqueue_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, d_ws, pl, 0, stream);
  }
  // resolve without the gather: the attention kernels fetch the misses
  hipError_t e = hs::launch_resolve(b->d_units, b->n, b->max_B, d_topk, k, d_slots, d_miss,
                                    hs::FETCH_NONE, 0, (int)b->pool->rec, S(stream));
  if (e != hipSuccess) return hip_fail(e, "resolve launch");
  return enqueue_attn(b, d_q, Hq, d_slots, k, sm_scale, d_out, d_ws, pl, 1, stream);
}

// ---------------------------------------------------------------- prefetch

hs_status hs_prefetch(hs_batch_t b, void *stream) {
  if (!b) return fail(HS_E_INVAL, "null batch");
  if (check_epoch(b)) return HS_E_INVAL;
  hipError_t e = hs::launch_prefetch(b->d_units, b->n, (int)b->pool->rec,
                                     g_tuning.prefetch_workgroups,
                                     g_tuning.prefetch_batch > 0 ? g_tuning.prefetch_batch : 1,
                                     S(stream));
  if (e != hipSuccess) return hip_fail(e, "prefetch launch");
  return HS_OK;
}

// ------------------------------------------------------------------- stage

struct hs_stage_s {
  uint32_t ring = 1;
  uint64_t total16 = 0;
  hs::StageTable table{};
  uint32_t *d_ctl = nullptr;
};

hs_status hs_stage_create(const hs_stage_region *regions, int32_t n, int32_t ring,
                          hs_stage_t *out) {
  if (!regions || !out || n < 1 || n > hs::STAGE_MAX_REGIONS || ring < 1)
    return fail(HS_E_INVAL, "need 1 to %d regions and ring >= 1", hs::STAGE_MAX_REGIONS);
  *out = nullptr;
  std::vector<hs::StageRegion> h(n);
  uint64_t total = 0;
  for (int i = 0; i < n; ++i) {
    const hs_stage_region &r = regions[i];
    if (!r.d_src || !r.d_dst || r.bytes == 0)
      return fail(HS_E_INVAL, "region %d: null pointer or no bytes", i);
    if (r.bytes % 16 || r.src_stride % 16 || (uintptr_t)r.d_src % 16 || (uintptr_t)r.d_dst % 16)
      return fail(HS_E_INVAL, "region %d: sizes and pointers must be multiples of 16", i);
    const size_t span = (size_t)(ring - 1) * r.src_stride + r.bytes;
    for (int j = 0; j <= i; ++j) {
      const hs_stage_region &o = regions[j];
      const size_t ospan = (size_t)(ring - 1) * o.src_stride + o.bytes;
      if (overlaps(r.d_dst, r.bytes, o.d_src, ospan) || (j < i && overlaps(o.d_dst, o.bytes, r.d_src, span)) ||
          (j < i && overlaps(r.d_dst, r.bytes, o.d_dst, o.bytes)))
        return fail(HS_E_INVAL, "region %d overlaps region %d", i, j);
    }
    h[i].src = (const uint8_t *)r.d_src;
    h[i].dst = (uint8_t *)r.d_dst;
    h[i].n16 = r.bytes / 16;
    h[i].stride16 = r.src_stride / 16;
    total += h[i].n16;
  }
  hs_stage_s *st = new (std::nothrow) hs_stage_s;
  if (!st) return fail(HS_E_NOMEM, "stage handle");
  st->ring = (uint32_t)ring;
  st->total16 = total;
  st->table.n = n;
  uint64_t run = 0;
  for (int i = 0; i < n; ++i) {
    st->table.r[i] = h[i];
    run += h[i].n16;
    st->table.end16[i] = run;
  }
  hipError_t e = hipMalloc(&st->d_ctl, sizeof(uint32_t) * hs::STAGE_CTL_WORDS);
  if (e == hipSuccess) e = hs::launch_stage_set(st->d_ctl, 0u, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (st->d_ctl) (void)hipFree(st->d_ctl);
    delete st;
    return hip_fail(e, "stage create");
  }
  *out = st;
  return HS_OK;
}

hs_status hs_stage_destroy(hs_stage_t st) {
  if (!st) return fail(HS_E_INVAL, "null stage");
  (void)hipFree(st->d_ctl);
  delete st;
  return HS_OK;
}

hs_status hs_stage_run(hs_stage_t st, void *stream) {
  if (!st) return fail(HS_E_INVAL, "null stage");
  hipError_t e = hs::launch_stage(st->table, st->total16, st->d_ctl, st->ring, S(stream));
  if (e != hipSuccess) return hip_fail(e, "stage launch");
  return HS_OK;
}

hs_status hs_stage_set_step(hs_stage_t st, uint32_t step, void *stream) {
  if (!st) return fail(HS_E_INVAL, "null stage");
  hipError_t e = hs::launch_stage_set(st->d_ctl, step, S(stream));
  if (e != hipSuccess) return hip_fail(e, "stage set");
  return HS_OK;
}

hs_status hs_stage_get_step(hs_stage_t st, uint32_t *step) {
  if (!st || !step) return fail(HS_E_INVAL, "null argument");
  HS_HIP(hipDeviceSynchronize());
  uint64_t w = 0;  // step in the high half, arrivals (0 between launches) in the low
  HS_HIP(hipMemcpy(&w, st->d_ctl, sizeof(uint64_t), hipMemcpyDeviceToHost));
  *step = (uint32_t)(w >> 32);
  return HS_OK;
}

// ------------------------------------------------------------------ tracing

hs_status hs_trace_enable(int32_t on) {
  if (on && g_trace.begin.empty()) {
    g_trace.begin.resize(TRACE_CAP);
    g_trace.end.resize(TRACE_CAP);
    g_trace.cls.assign(TRACE_CAP, 0);
    for (int i = 0; i < TRACE_CAP; ++i) {
      HS_HIP(hipEventCreate(&g_trace.begin[i]));
      HS_HIP(hipEventCreate(&g_trace.end[i]));
    }
  }
  g_trace.on = on != 0;
  return HS_OK;
}

hs_status hs_trace_read(hs_trace *out) {
  if (!out) return fail(HS_E_INVAL, "null trace");
  memset(out, 0, sizeof *out);
  if (g_trace.n > 0) HS_HIP(hipDeviceSynchronize());
  for (int i = 0; i < g_trace.n; ++i) {
    float ms = 0.f;
    HS_HIP(hipEventElapsedTime(&ms, g_trace.begin[i], g_trace.end[i]));
    const int c = g_trace.cls[i];
    if (c >= 0 && c < HS_TRACE_CLASSES) {
      out->total_us[c] += 1000.0 * ms;
      ++out->launches[c];
    }
  }
  out->dropped = g_trace.dropped;
  g_trace.n = 0;
  g_trace.dropped = 0;
  return HS_OK;
}

}  // extern "C"
