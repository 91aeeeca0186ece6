/* hisparse.h - C ABI of the HiSparse decode hot path on AMD Instinct MI355X
 * (gfx950): a pinned host KV pool, per-(request, layer) device buffers, the
 * fused RESOLVE step and top-k sparse attention over the resolved slots.
 *
 * Source of the operations: "HiSparse: Scaling Sparse-Attention Decoding
 * with Hierarchical KV Cache Management", as summarised on the
 * marsggbo.github.io page of 2026-09-23 ("HiSparse | 稀疏注意力省了算力却没省
 * 显存…"), cited below as "HiSparse summary" with the page's own section
 * numbers:
 *   section 3 - the architecture: the host pool is the authoritative copy of
 *     every record; each request and layer owns a fixed B-slot device buffer
 *     with a page table and LRU metadata; per decode step the indexer's k
 *     selected positions are resolved against the buffer (hits used in
 *     place, misses swapped in from host in one batch, LRU victims evicted);
 *     the physical slots feed the sparse-attention backend; the new token's
 *     record is written through to the host pool. The result is exact.
 *   section 4 - the LRU state is kept and updated in place across steps.
 *   section 5 - the fused resolve: an on-chip hash table of the selection,
 *     a parallel probe of every buffer slot, a parallel scan that picks the
 *     victims (hits to most-recently-used, misses right after the hits),
 *     GPU threads loading the missing records straight from pinned host
 *     memory, and a published slot vector aligned with the selection; the
 *     whole step is capturable in a graph (no host synchronisation).
 *   section 6 - exact cross-layer prefetch: when a group of layers reuses
 *     one indexer selection (IndexShare), the group's fetch plan is known as
 *     soon as that selection is resolved, so the records the later layers
 *     miss can be fetched while earlier layers compute.
 *   section 8 - the knobs: top_k (k per call) and device_buffer_size (B).
 *
 * Conventions
 *   - Every call returns hs_status. HS_OK is 0; errors are negative.
 *     hs_last_error() gives a message for the last failing call on the
 *     calling thread.
 *   - Handles are opaque and not thread-safe. A stream argument is a
 *     hipStream_t passed as void* (NULL is the default stream).
 *   - "Enqueue only" calls validate their arguments on the host, enqueue
 *     GPU work on the stream and return; they never synchronise and are
 *     safe inside hipStreamBeginCapture/EndCapture. Calls marked
 *     "synchronous" block until their work is done and must not be called
 *     while the stream is being captured.
 *   - Device pointers (d_*) are caller-owned HIP device memory. Host
 *     pointers are plain host memory.
 *   - Units: a batch is an ordered list of n buffers ("units"); per-unit
 *     arrays are unit-major: topk/slots [n][k], miss [n], queries
 *     [n][n_q_heads][q_dim], outputs [n][n_q_heads][v_dim].
 *
 * Data errors found on the device (a selection or slot that the host cannot
 * check without synchronising) are reported in the unit's sticky error word
 * (read with hs_buffer_state_get): bits accumulate and are cleared only by
 * hs_buffer_reset or hs_buffer_state_set.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hs_status;
#define HS_OK 0
#define HS_E_INVAL (-1)  /* malformed argument (null, size, shape, k vs B) */
#define HS_E_RANGE (-2)  /* request/layer/position outside the pool */
#define HS_E_NOMEM (-3)  /* host or device allocation failed */
#define HS_E_HIP (-4)    /* a HIP runtime call failed */
#define HS_E_DEVICE (-5) /* the device reported a data error (hs_batch_status) */
#define HS_E_STATE (-6)  /* state given to hs_buffer_state_set is not valid */

/* Bits of a unit's device error word. */
#define HS_ERR_RANGE 1u  /* a selected position was outside [0, pool length) */
#define HS_ERR_DUP 2u    /* an in-range position was selected twice */
#define HS_ERR_CLOCK 4u  /* the buffer's clock is exhausted (2^31 - 1 steps) */
#define HS_ERR_SLOT 8u   /* attention got a slot outside [0, B) */
#define HS_ERR_INTERNAL 16u /* resolve found its victim count inconsistent with
                               the miss count (never expected; state untouched) */
#define HS_ERR_APPEND 32u /* hs_pool_append_batch found the unit's pool full
                             (no page allocated at its length); nothing written */

/* Record layouts. HS_KV_MHA: one record per token holds
 * [K: n_kv_heads x head_dim][V: n_kv_heads x head_dim]. HS_KV_LATENT
 * (MLA-style shared latent): [latent: latent_dim][rope: rope_dim]; the key is
 * the whole record and the value is the latent part. */
#define HS_KV_MHA 0
#define HS_KV_LATENT 1

#define HS_F32 0
#define HS_BF16 1

/* Limits of this implementation. */
#define HS_MAX_K 4096          /* selected positions per unit and call */
#define HS_MAX_B 16384         /* slots of a buffer that hs_resolve accepts */

typedef struct hs_pool_s *hs_pool_t;
typedef struct hs_buffer_s *hs_buffer_t;
typedef struct hs_batch_s *hs_batch_t;

typedef struct hs_pool_desc {
  int32_t n_requests;             /* >= 1 */
  int32_t n_layers;               /* >= 1 */
  int32_t kind;                   /* HS_KV_MHA or HS_KV_LATENT */
  int32_t dtype;                  /* HS_F32 or HS_BF16 (records) */
  int32_t n_kv_heads;             /* HS_KV_MHA */
  int32_t head_dim;               /* HS_KV_MHA */
  int32_t latent_dim;             /* HS_KV_LATENT: value part */
  int32_t rope_dim;               /* HS_KV_LATENT: key-only part */
  const int64_t *capacity_tokens; /* [n_requests] records per layer allocated
                                     at creation, host */
  const int64_t *max_tokens;      /* [n_requests] the most records per layer a
                                     request may reserve later (hs_pool_reserve),
                                     host; NULL = capacity_tokens */
  int32_t page_tokens;            /* records per pool page, a power of two;
                                     0 = 65536, or less when every request's
                                     maximum fits in a smaller power of two */
} hs_pool_desc;

/* Tuning knobs (library-wide; 0 = choose automatically). */
typedef struct hs_tuning {
  int32_t attn_splits;          /* split-k factor of sparse attention */
  int32_t latent_heads_per_wg;  /* latent attention: query heads per workgroup
                                   (32 or 64; 0 = by batch size) */
  int32_t prefetch_workgroups;  /* hs_prefetch: workgroups per launch
                                   (0 = 64; 1 to 65536) */
  int32_t prefetch_batch;       /* hs_prefetch: host reads in flight per lane
                                   (0 = 1; 1, 2, 4 or 8) */
  int32_t gather_bytes_per_lane; /* hs_resolve's miss fetch (the swap-in transfer
                                   block of HiSparse summary, sections 5 and 8):
                                   bytes of host reads each lane keeps in flight
                                   per batch, 16 x {1, 2, 4, 8}; 0 = 64 */
  int32_t resolve_fetch;        /* where hs_resolve moves the misses: 0 = by
                                   batch size (the resolve kernel for 4 or more
                                   units, else a gather kernel of its own);
                                   1 = the resolve kernel; 2 = a gather kernel
                                   of its own (many workgroups per unit) */
  int32_t reserved[2];
} hs_tuning;

const char *hs_status_str(hs_status s);
const char *hs_last_error(void);

hs_status hs_set_tuning(const hs_tuning *t);
hs_status hs_get_tuning(hs_tuning *t);

/* ---------------- host KV pool (HiSparse summary, sections 3, 8) -----------
 * The pool is the authoritative copy of every record (section 3), kept in
 * pinned host memory mapped into the current device's address space
 * (hipHostMalloc) and allocated in pages as requests grow (section 8: the
 * host pool is allocated in pages). A page holds page_tokens consecutive
 * records of every layer of one request; each (request, layer) unit has a
 * device page table (entry i: the device-visible address of its records
 * [i * page_tokens, (i + 1) * page_tokens)) through which the kernels reach
 * host records, so records of one unit need not be contiguous and adding
 * pages never moves existing records or invalidates buffers or batches.
 * hs_pool_create allocates each request's pages up to capacity_tokens and
 * page tables sized for max_tokens, plus a device table of per-unit lengths
 * (all 0). The library owns that memory until hs_pool_destroy. Synchronous.
 * Errors: HS_E_INVAL (bad descriptor), HS_E_NOMEM (allocation failed). */
hs_status hs_pool_create(const hs_pool_desc *desc, hs_pool_t *out);
/* The caller must have synchronised every stream that used the pool. */
hs_status hs_pool_destroy(hs_pool_t pool);
/* Bytes of one record. */
hs_status hs_pool_record_bytes(hs_pool_t pool, size_t *rec_bytes);
/* Records allocated for request req (whole pages), its maximum and the page
 * size (any pointer may be NULL). HS_E_RANGE for a bad req. */
hs_status hs_pool_capacity(hs_pool_t pool, int32_t req, int64_t *capacity,
                           int64_t *max_tokens, int64_t *page_tokens);
/* Allocates request req's pages so that at least `records` records per
 * layer exist (no-op if they do); existing records stay where they are.
 * Synchronous; not while a stream is being captured. HS_E_RANGE above the
 * request's max_tokens, HS_E_NOMEM if an allocation fails. */
hs_status hs_pool_reserve(hs_pool_t pool, int32_t req, int64_t records);
/* Returns all of request req's pages (the request finished): its units'
 * lengths become 0 and its capacity 0; hs_pool_reserve gives the request
 * index pages again (for a new request, up to the same maximum). Buffers of
 * the request keep positions that no longer exist: reset them
 * (hs_buffer_reset) before resolving for the new request (until then a
 * resolve reports HS_ERR_RANGE and reads nothing). Synchronous (waits for
 * the device). HS_E_RANGE for a bad req. */
hs_status hs_pool_release(hs_pool_t pool, int32_t req);
/* Host pointer of record pos of unit (req, layer), for writing prefill
 * records directly and for reading them back. HS_E_RANGE for a bad
 * req/layer or pos outside [0, capacity). */
hs_status hs_pool_record_ptr(hs_pool_t pool, int32_t req, int32_t layer,
                             int64_t pos, void **host_ptr, size_t *rec_bytes);
/* Host pointer of page `page` of unit (req, layer): records
 * [page * page_tokens, (page + 1) * page_tokens) lie contiguously from it.
 * HS_E_RANGE for a bad req/layer or a page not allocated. */
hs_status hs_pool_page_ptr(hs_pool_t pool, int32_t req, int32_t layer,
                           int64_t page, void **host_ptr);
/* Current length (records valid for selection) of unit (req, layer).
 * Synchronous (reads the device table). */
hs_status hs_pool_length(hs_pool_t pool, int32_t req, int32_t layer,
                         int64_t *len);
/* Declare that records [0, len) of the unit were written through
 * hs_pool_record_ptr / hs_pool_page_ptr (prefill). Synchronous. HS_E_RANGE if
 * len > the allocated capacity. */
hs_status hs_pool_set_length(hs_pool_t pool, int32_t req, int32_t layer,
                             int64_t len);
/* Write-through append (HiSparse summary, section 3, arrow 5): write n
 * records from src to positions [pos, pos + n) of unit (req, layer) and set
 * its length to max(length, pos + n). The pool stays contiguous: pos must
 * not exceed the length as of the calls made so far (appends enqueued but
 * not yet run count). Only the pool is written; device buffers see the new
 * records only through later misses.
 * src_on_device = 0: src is host memory; copied synchronously.
 * src_on_device = 1: src is device memory; enqueued on stream (capture-safe).
 * Errors: HS_E_RANGE (pos > length or pos + n > the allocated capacity:
 * reserve first), HS_E_INVAL. */
hs_status hs_pool_append(hs_pool_t pool, int32_t req, int32_t layer,
                         int64_t pos, int64_t n, const void *src,
                         int32_t src_on_device, void *stream);
/* Write-through append at the end, for a decode graph replayed every step
 * (HiSparse summary, section 3, arrow 5; section 5: the step runs inside the
 * graph with no host synchronisation). For every unit u of the batch, the
 * record d_src[u] (device memory, [n][rec_bytes], 16-byte aligned) is
 * written to position len of u's (request, layer) pool, where len is the
 * unit's length when the kernel runs, and the length becomes len + 1. The
 * position is read on the device, so one captured call appends at the next
 * position on every replay. A unit whose pool has no page allocated at len
 * is not written and gets HS_ERR_APPEND in its error word (reserve pages
 * before capture). Only the pool is written. After this call the host no
 * longer knows the lengths without reading them: a later hs_pool_append of
 * such a unit synchronises its stream to read the length (and is refused,
 * HS_E_INVAL, while that stream is being captured). A batch holding two
 * buffers of one (request, layer) is refused (HS_E_INVAL).
 * Enqueue only; capture-safe. */
hs_status hs_pool_append_batch(hs_batch_t batch, const void *d_src,
                               void *stream);

/* ------------- hot device buffer (HiSparse summary, sections 3-4) ----------
 * A buffer of B record slots for unit (req, layer) with its page table
 * (slot -> logical position, -1 when empty), LRU stamps, clock and error
 * word. The memory is caller-owned device memory of at least
 * hs_buffer_bytes(pool, B) bytes, 256-byte aligned; the library only writes
 * into it and never frees it. Beside it the library keeps the inverse page
 * table (position -> slot, -1 when not resident; 4 bytes per position the
 * request can reach, max_tokens), allocated by hs_buffer_create and freed by
 * hs_buffer_destroy, which lets the resolve classify a selected position
 * with one read. */
size_t hs_buffer_bytes(hs_pool_t pool, int32_t B);
/* Enqueues the empty state (every slot empty, clock 0, error 0) on stream.
 * HS_E_INVAL for B < 1, too few bytes or misaligned memory; HS_E_RANGE for
 * a bad req/layer; HS_E_HIP if the inverse page table cannot be allocated. */
hs_status hs_buffer_create(hs_pool_t pool, int32_t req, int32_t layer,
                           int32_t B, void *d_mem, size_t bytes, void *stream,
                           hs_buffer_t *out);
/* Frees the handle only (not d_mem). HS_E_INVAL while shared buffers made
 * from it (hs_buffer_create_shared) still exist: destroy those first. */
hs_status hs_buffer_destroy(hs_buffer_t buf);
/* On-demand growth (HiSparse summary, section 8: the per-request, per-layer
 * device cache is allocated and grown as needed). Moves the buffer into new
 * caller-owned memory of at least hs_buffer_bytes(pool, new_B) bytes
 * (256-byte aligned, not overlapping the current memory), with
 * B <= new_B <= HS_MAX_B: slots [0, B) keep their positions, stamps and
 * rows, slots [B, new_B) are empty; clock, error word and the last fetch list
 * carry over. From then on the handle uses the new memory and the old memory
 * is no longer read (the caller may free it). Batches of the pool made
 * before describe the old memory: the resolve, attention and prefetch calls
 * refuse them (HS_E_INVAL) until they are created again, and graphs captured
 * before must be captured again. Refused (HS_E_INVAL) for a buffer whose
 * state is shared with others (either side of hs_buffer_create_shared):
 * such a group grows as a whole with hs_buffer_grow_group.
 * Synchronous (waits for stream). */
hs_status hs_buffer_grow(hs_buffer_t buf, int32_t new_B, void *d_mem, size_t bytes,
                         void *stream);
/* Enqueues the empty state again (also clears the error word). */
hs_status hs_buffer_reset(hs_buffer_t buf, void *stream);
/* Device pointer and size of the rows region: row s (the record held by
 * slot s) is at *d_rows + s * rec_bytes. */
hs_status hs_buffer_rows(hs_buffer_t buf, void **d_rows, size_t *rec_bytes);
/* Copies the buffer's metadata to host arrays pos[B], stamp[B] and scalars
 * (any pointer may be NULL). Synchronises stream. */
hs_status hs_buffer_state_get(hs_buffer_t buf, int32_t *pos, uint32_t *stamp,
                              uint32_t *clock, int32_t *err, void *stream);
/* Replaces the metadata (checkpoint restore) and re-gathers every occupied
 * row from the host pool; the error word is set to err. The state must be
 * valid: every pos in [-1, pool length), occupied positions distinct,
 * stamp 0 exactly for empty slots, stamps <= 2 * clock, clock < 2^31 - 1;
 * otherwise HS_E_STATE and nothing changes. Synchronous. */
hs_status hs_buffer_state_set(hs_buffer_t buf, const int32_t *pos,
                              const uint32_t *stamp, uint32_t clock,
                              int32_t err, void *stream);

/* -------- buffers of layers sharing one selection (HiSparse summary, §6) ---
 * When a group of layers of a request reuses one selection every step, their
 * buffers see the same requests and would hold identical page tables, stamps
 * and clocks; only the rows differ (each layer's own records). A shared
 * buffer is the rows of one more layer attached to the state of an existing
 * buffer `base` of the same request: page table, stamps, clock, error word
 * and the last resolve's fetch list live in base's memory and are the
 * group's; d_mem (caller-owned, 256-byte aligned, at least
 * hs_buffer_shared_bytes(pool, B) bytes with B = base's) holds the rows.
 * Resolving any one member (hs_resolve) advances the group's state and
 * fetches that member's misses; hs_prefetch then fetches the same misses
 * for the other members from their own layers' records. Attention works on
 * every member as on any buffer, with the group's slot vector.
 * Rules: resolve one member of a group per step (a batch holding two members
 * of one group is refused by the resolve calls); hs_buffer_reset and
 * hs_buffer_state_set on a member act on the group's state, and state_set
 * re-gathers the rows of that member only (restore a group by calling it on
 * every member with the same state); base's memory must outlive every
 * member. No GPU work is enqueued; the rows start undefined, like those of
 * empty slots. HS_E_INVAL for a null or misaligned argument, too few bytes,
 * or base of another pool or request; HS_E_RANGE for a bad layer. */
size_t hs_buffer_shared_bytes(hs_pool_t pool, int32_t B);
hs_status hs_buffer_create_shared(hs_buffer_t base, int32_t layer, void *d_mem,
                                  size_t bytes, hs_buffer_t *out);
/* Growth of a layer group (HiSparse summary, sections 6 and 8): the group's
 * state moves with base into d_mem (as hs_buffer_grow, at least
 * hs_buffer_bytes(pool, new_B) bytes) and the rows of members[i] into
 * member_mem[i] (at least hs_buffer_shared_bytes(pool, new_B) bytes,
 * member_bytes[i] given), all 256-byte aligned, with B <= new_B <= HS_MAX_B.
 * members lists every live buffer made from base or its members by
 * hs_buffer_create_shared, each once, in any order (n_members of them; 0 when
 * base has none). Slots [0, B) keep position, stamp and each layer's rows;
 * slots [B, new_B) are empty; clock, error word and fetch list carry over.
 * No new region may overlap another or any current region of the group; the
 * old memory is no longer read afterwards. Batches and graphs made before
 * must be made again, as after hs_buffer_grow. HS_E_INVAL for a null or
 * misaligned argument, too few bytes, overlapping memory, a base that is a
 * member, or a member list that is not exactly the group; nothing changes
 * then. Synchronous (waits for stream). */
hs_status hs_buffer_grow_group(hs_buffer_t base, const hs_buffer_t *members,
                               int32_t n_members, int32_t new_B, void *d_mem,
                               size_t bytes, void *const *member_mem,
                               const size_t *member_bytes, void *stream);

/* ------------------------------- batches -----------------------------------
 * An ordered list of n units (buffers of one pool; buffer sizes may
 * differ). Uploads a device descriptor table. Synchronous; create batches
 * before graph capture. The buffers must outlive the batch. */
hs_status hs_batch_create(const hs_buffer_t *bufs, int32_t n,
                          hs_batch_t *out);
hs_status hs_batch_destroy(hs_batch_t batch);
/* Error words of the batch's units after the work enqueued so far: errs[u]
 * (host array of n, may be NULL) receives unit u's sticky HS_ERR_* bits.
 * Returns HS_E_DEVICE if any unit has a bit set, else HS_OK. Synchronises
 * stream; not while it is being captured. */
hs_status hs_batch_status(hs_batch_t batch, int32_t *errs, void *stream);

/* --------------- RESOLVE (HiSparse summary, sections 4-5) ------------------
 * For every unit u, resolves the selection d_topk[u][0..k) (logical
 * positions) against u's buffer in place, and writes d_slots[u][i], the
 * slot that now holds position d_topk[u][i] (aligned with the selection),
 * and d_miss[u], the number of positions fetched from the host pool
 * (d_miss may be NULL). Semantics, per unit, with c = clock + 1:
 *   hits   - slots whose position is selected; their stamp becomes 2c;
 *   misses - selected positions held by no slot, in selection order;
 *   victims- the m = #misses non-hit slots with the smallest key
 *            (stamp, position, slot) (empty slots: stamp 0, position -1,
 *            so they are used first, lowest slot first; equal stamps leave
 *            in ascending position), sorted by ascending slot; the j-th miss
 *            goes into the j-th victim with stamp 2c - 1, and its record is
 *            copied from the host pool into the slot's row;
 *   clock  - becomes c.
 * Host checks (HS_E_INVAL): 1 <= k <= min B, k <= HS_MAX_K, every B <=
 * HS_MAX_B, null pointers. Device data errors (a position outside
 * [0, length), a repeated position, an exhausted clock) set the unit's
 * error bits, write slots = -1 and miss = -1 and leave its state unchanged;
 * other units proceed. The fetch list (slot and position of every miss) is
 * kept in the unit's state for hs_prefetch. A batch holding two buffers of
 * one shared state is refused (HS_E_INVAL). Enqueue only; capture-safe. */
hs_status hs_resolve(hs_batch_t batch, const int32_t *d_topk, int32_t k,
                     int32_t *d_slots, int32_t *d_miss, void *stream);

/* ------------- sparse attention (HiSparse summary, sections 3, 5) ----------
 * Decode attention of each unit's queries over the k rows named by
 * d_slots[u][0..k) in its buffer:
 *   out[u][h] = sum_i softmax_i(sm_scale * q[u][h] . K_i) V_i
 * HS_KV_MHA: q [n][n_q_heads][head_dim] of the pool's dtype; query head h
 *   reads KV head h / (n_q_heads / n_kv_heads); out [n][n_q_heads][head_dim].
 *   Supported: head_dim 64 or 128, n_q_heads / n_kv_heads in {1, 2, 4, 8}.
 * HS_KV_LATENT: q [n][n_q_heads][latent_dim + rope_dim] bf16; K is the whole
 *   record, V its latent part; out [n][n_q_heads][latent_dim]. Supported:
 *   bf16, latent_dim 512, rope_dim 64, n_q_heads 16, 32 or 64.
 *   Attention over the same buffers must not run concurrently with a resolve
 *   of them.
 * Outputs are fp32 (accumulation is fp32; for latent records the split-k
 * partials in the workspace are rounded to bf16, their (m, l) kept in fp32,
 * which the relative-L2 bound of 4e-3 on bf16 records covers). A slot
 * outside [0, B) makes the unit's output NaN and sets HS_ERR_SLOT. d_ws is
 * scratch of at least
 * hs_sparse_attn_workspace(...) bytes (may be NULL when that is 0); its
 * contents need no initialisation. Enqueue only; capture-safe.
 * HS_E_INVAL for unsupported shapes or a small workspace. */
size_t hs_sparse_attn_workspace(hs_batch_t batch, int32_t n_q_heads,
                                int32_t k);
hs_status hs_sparse_attn(hs_batch_t batch, const void *d_q, int32_t n_q_heads,
                         const int32_t *d_slots, int32_t k, float sm_scale,
                         float *d_out, void *d_ws, size_t ws_bytes,
                         void *stream);

/* Allocation-free sparse attention, for callers that cannot allocate device
 * memory or pass a workspace: code under graph capture, tight serving loops,
 * harnesses that forbid allocation. The same computation, kernels and
 * results as hs_sparse_attn, bit for bit; the split-k partials go to a
 * scratch array of HS_NOALLOC_SCRATCH_BYTES that the library holds in
 * device memory on each GPU it runs on, from that GPU's first such call
 * until the process ends (its address is looked up on that first call, so
 * make the first call outside graph capture). Calls that would need more
 * scratch than that are refused (HS_E_INVAL, before anything is enqueued).
 * Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (different streams, or graphs replayed concurrently)
 * race and give wrong results; order them on one stream. Enqueue only;
 * capture-safe after the first call; no allocation of any kind. */
#define HS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hs_status hs_sparse_attn_noalloc(hs_batch_t batch, const void *d_q,
                                 int32_t n_q_heads, const int32_t *d_slots,
                                 int32_t k, float sm_scale, float *d_out,
                                 void *stream);

/* ---------- RESOLVE + sparse attention, fused (HiSparse summary, §5) -------
 * The same effect as hs_resolve followed by hs_sparse_attn on the same
 * stream - identical page tables, stamps, clocks, error words, slot vectors,
 * miss counts, row bytes and outputs, bit for bit. For HS_KV_MHA records the
 * misses travel differently: instead of a separate copy kernel, the
 * attention workgroup that needs a just-resolved miss loads its record
 * straight from the pinned host pool, uses it, and stores it into the slot
 * the resolve assigned, so the host-link transfer overlaps the attention over
 * the resident rows. Every missing byte still crosses the host link once.
 * For HS_KV_LATENT records it is exactly the two calls (the resolve moves
 * the misses, its first host reads overlapping its victim selection).
 * Arguments, checks and workspace as for the two calls. Enqueue only;
 * capture-safe. */
hs_status hs_resolve_attn(hs_batch_t batch, const int32_t *d_topk, int32_t k,
                          int32_t *d_slots, int32_t *d_miss, const void *d_q,
                          int32_t n_q_heads, float sm_scale, float *d_out,
                          void *d_ws, size_t ws_bytes, void *stream);

/* -------------- exact cross-layer prefetch (HiSparse summary, §6) ----------
 * For every unit of the batch, copies into its rows the records its state's
 * last resolve missed: slot s_j of the fetch list receives the record at
 * position p_j of the unit's own (request, layer) pool. For a buffer that
 * shares the state of another layer (hs_buffer_create_shared), this is that
 * layer's share of the group's plan: after it, the buffer holds the record
 * of its own layer at every position the group's page table names, so
 * attention over it with the group's slot vector equals attention over a
 * buffer resolved on its own. Must be ordered after the group's resolve
 * (same stream, or an event) and before the next one; it may run on another
 * stream concurrently with attention over other buffers. A fetch-list
 * position at or past the unit's pool length is skipped and sets
 * HS_ERR_RANGE. The number of workgroups and the host reads each lane keeps
 * in flight are hs_tuning.prefetch_workgroups and prefetch_batch (defaults
 * 64 and 1: few long-latency reads per compute unit, so that attention
 * running beside the prefetch is slowed little). Enqueue only; capture-safe.
 * HS_E_INVAL for a null batch or one made before a buffer of its pool grew. */
hs_status hs_prefetch(hs_batch_t batch, void *stream);

/* ------------- staging the inputs of a decode step (HiSparse summary, §5) ---
 * The resolve sits inside the decode step's graph, which reads the indexer's
 * selection (and the query, and the new token's record) from fixed device
 * buffers that the step's earlier kernels fill. A stage stands in for those
 * producers: it copies, for step t, entry t % ring of each region's source
 * ring into the region's fixed destination, where t is a step counter kept
 * in device memory and advanced by one on the device after the copy. One
 * captured hs_stage_run therefore stages a new step on every replay of the
 * graph, with no host involvement.
 * hs_stage_create: 1 to 8 regions[i] = {d_src, d_dst, bytes, src_stride}: entry j
 *   of the ring is d_src + j * src_stride; bytes and src_stride multiples of
 *   16 and pointers 16-byte aligned; destinations must not overlap any
 *   source or each other. ring >= 1 entries. The step counter starts at 0.
 *   Synchronous. HS_E_INVAL for a malformed region or more than 8 regions.
 * hs_stage_run: enqueue only; capture-safe. One kernel for every region.
 * hs_stage_set_step: sets the counter (enqueued; a kernel, not a memset).
 * hs_stage_get_step: reads the counter; synchronous (waits for the device).
 */
typedef struct hs_stage_s *hs_stage_t;
typedef struct hs_stage_region {
  const void *d_src;  /* ring of entries, device memory */
  void *d_dst;        /* fixed destination, device memory */
  size_t bytes;       /* bytes per entry */
  size_t src_stride;  /* bytes from one ring entry to the next */
} hs_stage_region;
hs_status hs_stage_create(const hs_stage_region *regions, int32_t n,
                          int32_t ring, hs_stage_t *out);
hs_status hs_stage_destroy(hs_stage_t stage);
hs_status hs_stage_run(hs_stage_t stage, void *stream);
hs_status hs_stage_set_step(hs_stage_t stage, uint32_t step, void *stream);
hs_status hs_stage_get_step(hs_stage_t stage, uint32_t *step);

/* ------------------------------- tracing -----------------------------------
 * Event timing of individual kernels, for measurement. While enabled, every
 * kernel that the enqueueing calls launch carries a pair of HIP events that
 * take the dispatch's own start and end times (hipExtLaunchKernel), so the
 * elapsed time is the kernel's execution without launch overhead (do not
 * enable it around graph capture). hs_trace_read synchronises the device,
 * adds up the elapsed time of every pair per kernel class and clears the
 * record. Classes:
 * HS_TRACE_RESOLVE (hash, probe, victim select, update; for hs_resolve on
 * batches of 4 or more units also the host-to-device miss fetch),
 * HS_TRACE_GATHER (the miss fetch of hs_resolve on smaller batches, a kernel
 * of its own, and hs_prefetch), HS_TRACE_ATTN (sparse attention; for hs_resolve_attn it
 * includes the miss fetch), HS_TRACE_COMBINE (split-k merge), HS_TRACE_STAGE
 * (hs_stage_run), HS_TRACE_APPEND (device-source appends). At most 4096
 * launches are recorded between reads; later ones are counted in
 * `dropped`. */
#define HS_TRACE_RESOLVE 0
#define HS_TRACE_GATHER 1
#define HS_TRACE_ATTN 2
#define HS_TRACE_COMBINE 3
#define HS_TRACE_STAGE 4
#define HS_TRACE_APPEND 5
#define HS_TRACE_CLASSES 6
typedef struct hs_trace {
  double total_us[HS_TRACE_CLASSES];
  int64_t launches[HS_TRACE_CLASSES];
  int64_t dropped;
} hs_trace;
hs_status hs_trace_enable(int32_t on);
hs_status hs_trace_read(hs_trace *out);

#ifdef __cplusplus
}
#endif
#endif /* HISPARSE_H */
