/* CPU oracle of the HiSparse decode hot path: RESOLVE and top-k sparse
 * attention over the resolved slots.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path
 * never calls it, and it shares no code, header, table or constant with the
 * GPU library.
 *
 * Source. "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
 * Cache Management", as summarised on the marsggbo.github.io page of
 * 2026-09-23 titled "HiSparse | 稀疏注意力省了算力却没省显存…" (cited below
 * as "HiSparse summary"):
 *   section 3: a host pool holds every record; the GPU holds a fixed B-slot
 *              buffer per request and layer with a page table and LRU
 *              metadata; hits are used in place, misses are swapped in from
 *              host in one batch, and LRU victims are evicted; the output is
 *              exactly full-KV attention at the selected positions.
 *   section 4: hits are kept and the LRU state is updated in place, never
 *              rebuilt from the current selection.
 *   section 5: per-slot probe against the selected set; hits become most
 *              recently used and fetched misses rank right after the hits;
 *              the published slot vector is aligned with the selection.
 *
 * Readings where the page leaves a step open (each is also listed in the
 * design notes):
 *   - Recency is a per-slot stamp. At step c (the buffer's clock after the
 *     call) hits get 2c and misses 2c - 1, so reading from most recent down
 *     the order is [hits][misses][untouched residents].
 *   - Eviction takes the m non-hit slots with the smallest key
 *     (stamp, position, slot); empty slots hold stamp 0 and position -1, so
 *     they go first, lowest slot first; equal stamps go to the smaller
 *     logical position first.
 *   - The i-th miss in selection order fills the i-th victim in ascending
 *     slot order.
 *   - Data errors leave the buffer untouched: a position outside [0, len)
 *     sets error bit 1, a repeated in-range position sets bit 2, an
 *     exhausted clock sets bit 4; the slot vector is then all -1 and the
 *     miss count -1. Error bits accumulate (sticky) and do not block later
 *     valid calls.
 *   - Attention runs in fp64 over the selected positions in selection order
 *     with one division at the end, rounded once to fp32.
 *
 * Nothing here is blocked, fused or reordered beyond those definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_ERR_RANGE 1
#define OR_ERR_DUP 2
#define OR_ERR_CLOCK 4

#define OR_DT_F32 0
#define OR_DT_BF16 1

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */

typedef struct {
  int32_t pos;
  int32_t idx;
} or_pair;

static int cmp_pair_pos(const void *a, const void *b) {
  int32_t x = ((const or_pair *)a)->pos, y = ((const or_pair *)b)->pos;
  return (x > y) - (x < y);
}

typedef struct {
  uint32_t stamp;
  int32_t pos;
  int32_t slot;
} or_key;

/* Lexicographic (stamp, position, slot), all ascending. */
static int cmp_key(const void *a, const void *b) {
  const or_key *x = (const or_key *)a, *y = (const or_key *)b;
  if (x->stamp != y->stamp) return x->stamp < y->stamp ? -1 : 1;
  if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
  return (x->slot > y->slot) - (x->slot < y->slot);
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Index into the position-sorted selection, or -1 if p is not selected. */
static int32_t find_selected(const or_pair *sorted, int32_t n, int32_t p) {
  int32_t lo = 0, hi = n - 1;
  while (lo <= hi) {
    int32_t mid = lo + (hi - lo) / 2;
    if (sorted[mid].pos == p) return sorted[mid].idx;
    if (sorted[mid].pos < p)
      lo = mid + 1;
    else
      hi = mid - 1;
  }
  return -1;
}

/* bf16 bit pattern -> double, exactly (the bf16 bits are the top half of an
 * fp32 pattern). */
static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_elem(const void *base, int64_t i, int32_t dtype) {
  if (dtype == OR_DT_F32) return (double)((const float *)base)[i];
  return bf16_to_f64(((const uint16_t *)base)[i]);
}

/* ------------------------------------------------------------------ */
/* RESOLVE                                                             */
/* ------------------------------------------------------------------ */

/* One resolve of one (request, layer) buffer, in place.
 *
 * State: pos[B] (logical position per slot, -1 empty), stamp[B] (0 = never
 * used), *clock, *err, rows[B][rec_bytes] (may be NULL to skip the record
 * copies). pool points at the unit's record array in host memory (record p
 * at pool + p * rec_bytes, valid for p < pool_len; may be NULL when rows is
 * NULL). topk[k] is the selection. Outputs slots[k] aligned with topk and
 * *miss.
 *
 * Returns 0 when the call was well formed (data errors included, they are
 * reported through *err), -1 when it was not (k outside [1, B], B < 1, null
 * state pointers); then nothing is touched. */
int oracle_resolve(int32_t B, int32_t *pos, uint32_t *stamp, uint32_t *clock,
                   int32_t *err, uint8_t *rows, int64_t rec_bytes,
                   const uint8_t *pool, int64_t pool_len, const int32_t *topk,
                   int32_t k, int32_t *slots, int32_t *miss) {
  if (B < 1 || k < 1 || k > B || !pos || !stamp || !clock || !err || !topk ||
      !slots || !miss)
    return -1;
  if (rows && !pool) return -1;

  /* 1. validate the selection */
  int32_t bad = 0;
  or_pair *sorted = (or_pair *)malloc(sizeof(or_pair) * (size_t)k);
  int32_t n_in = 0;
  for (int32_t i = 0; i < k; ++i) {
    if (topk[i] < 0 || (int64_t)topk[i] >= pool_len) {
      bad |= OR_ERR_RANGE;
    } else {
      sorted[n_in].pos = topk[i];
      sorted[n_in].idx = i;
      ++n_in;
    }
  }
  qsort(sorted, (size_t)n_in, sizeof(or_pair), cmp_pair_pos);
  for (int32_t i = 1; i < n_in; ++i)
    if (sorted[i].pos == sorted[i - 1].pos) bad |= OR_ERR_DUP;
  if (*clock >= 0x7FFFFFFFu) bad |= OR_ERR_CLOCK;
  if (bad) {
    *err |= bad;
    for (int32_t i = 0; i < k; ++i) slots[i] = -1;
    *miss = -1;
    free(sorted);
    return 0;
  }

  /* 2. the new clock value */
  uint32_t c = *clock + 1;

  /* 3. probe every slot against the selected set */
  int32_t *slot_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  uint8_t *is_hit = (uint8_t *)calloc((size_t)B, 1);
  for (int32_t i = 0; i < k; ++i) slot_of[i] = -1;
  for (int32_t s = 0; s < B; ++s) {
    if (pos[s] < 0) continue;
    int32_t i = find_selected(sorted, k, pos[s]);
    if (i >= 0) {
      slot_of[i] = s;
      is_hit[s] = 1;
    }
  }

  /* 4. misses in selection order */
  int32_t *miss_idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  int32_t m = 0;
  for (int32_t i = 0; i < k; ++i)
    if (slot_of[i] < 0) miss_idx[m++] = i;

  /* 5. victims: the m non-hit slots with the smallest (stamp, pos, slot) */
  or_key *cand = (or_key *)malloc(sizeof(or_key) * (size_t)B);
  int32_t n_cand = 0;
  for (int32_t s = 0; s < B; ++s) {
    if (is_hit[s]) continue;
    cand[n_cand].stamp = stamp[s];
    cand[n_cand].pos = pos[s];
    cand[n_cand].slot = s;
    ++n_cand;
  }
  qsort(cand, (size_t)n_cand, sizeof(or_key), cmp_key);
  int32_t *victim = (int32_t *)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
  for (int32_t j = 0; j < m; ++j) victim[j] = cand[j].slot; /* n_cand >= m since B >= k */
  qsort(victim, (size_t)m, sizeof(int32_t), cmp_i32);

  /* 6. fill: j-th miss into the j-th victim, copying its record */
  for (int32_t j = 0; j < m; ++j) {
    int32_t s = victim[j];
    int32_t i = miss_idx[j];
    pos[s] = topk[i];
    stamp[s] = 2u * c - 1u;
    if (rows)
      memcpy(rows + (int64_t)s * rec_bytes, pool + (int64_t)topk[i] * rec_bytes,
             (size_t)rec_bytes);
    slot_of[i] = s;
  }

  /* 7. promote the hits to most recently used */
  for (int32_t s = 0; s < B; ++s)
    if (is_hit[s]) stamp[s] = 2u * c;

  /* 8. publish */
  *clock = c;
  for (int32_t i = 0; i < k; ++i) slots[i] = slot_of[i];
  *miss = m;

  free(sorted);
  free(slot_of);
  free(is_hit);
  free(miss_idx);
  free(cand);
  free(victim);
  return 0;
}

/* ------------------------------------------------------------------ */
/* attention                                                           */
/* ------------------------------------------------------------------ */

/* Softmax attention of one query row over k selected rows, fp64.
 * kq(i) = dot(q, K_i) is given through the score array; V_i through vrow.
 * Writes out[dv] (fp32, one rounding) and, if non-NULL, out64[dv]. */
static void softmax_av(const double *score, int32_t k, const uint8_t *const *vrow,
                       int64_t v_off_elems, int32_t dv, int32_t dtype,
                       double *acc, float *out, double *out64) {
  double mu = -INFINITY;
  for (int32_t i = 0; i < k; ++i)
    if (score[i] > mu) mu = score[i];
  double z = 0.0;
  for (int32_t j = 0; j < dv; ++j) acc[j] = 0.0;
  for (int32_t i = 0; i < k; ++i) {
    double e = exp(score[i] - mu);
    z += e;
    for (int32_t j = 0; j < dv; ++j)
      acc[j] += e * load_elem(vrow[i], v_off_elems + j, dtype);
  }
  for (int32_t j = 0; j < dv; ++j) {
    double o = acc[j] / z;
    out[j] = (float)o;
    if (out64) out64[j] = o;
  }
}

/* Multi-head / grouped-query attention over the resolved slots of one unit.
 *
 * Record layout: [K: Hkv x D][V: Hkv x D] elements of kv_dtype.
 * q: [Hq][D] of q_dtype. Query head h reads KV head h / (Hq / Hkv).
 * rows: n_rows records; slots[k] index them. A slot outside [0, n_rows)
 * makes every output NaN and the call returns 1.
 * out: [Hq][D] fp32; out64 (optional): [Hq][D] fp64 before rounding.
 * s_i = sm_scale * sum_d q[d] K_i[d] (d ascending), softmax in fp64,
 * out = sum_i e_i V_i / sum_i e_i. */
int oracle_attend_mha(int32_t Hq, int32_t Hkv, int32_t D, int32_t kv_dtype,
                      int32_t q_dtype, const void *q, const uint8_t *rows,
                      int64_t rec_bytes, int64_t n_rows, const int32_t *slots,
                      int32_t k, float sm_scale, float *out, double *out64) {
  if (Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv || k < 1) return -1;
  int32_t bad = 0;
  for (int32_t i = 0; i < k; ++i)
    if (slots[i] < 0 || (int64_t)slots[i] >= n_rows) bad = 1;
  if (bad) {
    for (int64_t j = 0; j < (int64_t)Hq * D; ++j) {
      out[j] = NAN;
      if (out64) out64[j] = NAN;
    }
    return 1;
  }
  const int32_t group = Hq / Hkv;
  const double scale = (double)sm_scale;
  double *score = (double *)malloc(sizeof(double) * (size_t)k);
  double *acc = (double *)malloc(sizeof(double) * (size_t)D);
  const uint8_t **vrow = (const uint8_t **)malloc(sizeof(void *) * (size_t)k);
  for (int32_t i = 0; i < k; ++i) vrow[i] = rows + (int64_t)slots[i] * rec_bytes;
  for (int32_t h = 0; h < Hq; ++h) {
    int32_t g = h / group;
    for (int32_t i = 0; i < k; ++i) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d)
        dot += load_elem(q, (int64_t)h * D + d, q_dtype) *
               load_elem(vrow[i], (int64_t)g * D + d, kv_dtype);
      score[i] = scale * dot;
    }
    softmax_av(score, k, vrow, (int64_t)(Hkv + g) * D, D, kv_dtype, acc,
               out + (int64_t)h * D, out64 ? out64 + (int64_t)h * D : NULL);
  }
  free(score);
  free(acc);
  free(vrow);
  return 0;
}

/* Latent (MLA-style) attention over the resolved slots of one unit.
 *
 * Record layout: [latent: Dl][rope: Dr] elements of kv_dtype. The key is the
 * whole record (Dl + Dr elements), the value is the latent part (first Dl).
 * q: [Hq][Dl + Dr]. out: [Hq][Dl]. Otherwise as oracle_attend_mha. */
int oracle_attend_latent(int32_t Hq, int32_t Dl, int32_t Dr, int32_t kv_dtype,
                         int32_t q_dtype, const void *q, const uint8_t *rows,
                         int64_t rec_bytes, int64_t n_rows, const int32_t *slots,
                         int32_t k, float sm_scale, float *out, double *out64) {
  if (Hq < 1 || Dl < 1 || Dr < 0 || k < 1) return -1;
  const int32_t Dk = Dl + Dr;
  int32_t bad = 0;
  for (int32_t i = 0; i < k; ++i)
    if (slots[i] < 0 || (int64_t)slots[i] >= n_rows) bad = 1;
  if (bad) {
    for (int64_t j = 0; j < (int64_t)Hq * Dl; ++j) {
      out[j] = NAN;
      if (out64) out64[j] = NAN;
    }
    return 1;
  }
  const double scale = (double)sm_scale;
  double *score = (double *)malloc(sizeof(double) * (size_t)k);
  double *acc = (double *)malloc(sizeof(double) * (size_t)Dl);
  const uint8_t **vrow = (const uint8_t **)malloc(sizeof(void *) * (size_t)k);
  for (int32_t i = 0; i < k; ++i) vrow[i] = rows + (int64_t)slots[i] * rec_bytes;
  for (int32_t h = 0; h < Hq; ++h) {
    for (int32_t i = 0; i < k; ++i) {
      double dot = 0.0;
      for (int32_t d = 0; d < Dk; ++d)
        dot += load_elem(q, (int64_t)h * Dk + d, q_dtype) *
               load_elem(vrow[i], d, kv_dtype);
      score[i] = scale * dot;
    }
    softmax_av(score, k, vrow, 0, Dl, kv_dtype, acc, out + (int64_t)h * Dl,
               out64 ? out64 + (int64_t)h * Dl : NULL);
  }
  free(score);
  free(acc);
  free(vrow);
  return 0;
}

/* ------------------------------------------------------------------ */
/* write-through append                                                */
/* ------------------------------------------------------------------ */

/* Write n records into a unit's host record array at [p, p + n) and extend
 * its length; the device buffer is not touched (HiSparse summary, section 3,
 * arrow 5: the new token's record is written through to the host pool).
 * Requires p <= *len and p + n <= capacity; returns -1 otherwise. */
int oracle_append(uint8_t *pool, int64_t rec_bytes, int64_t capacity,
                  int64_t *len, int64_t p, int64_t n, const uint8_t *src) {
  if (p < 0 || n < 0 || p > *len || p + n > capacity) return -1;
  memcpy(pool + p * rec_bytes, src, (size_t)(n * rec_bytes));
  if (p + n > *len) *len = p + n;
  return 0;
}

/* ------------------------------------------------------------------ */
/* one decode step over many units, for the CPU timing baseline        */
/* ------------------------------------------------------------------ */

typedef struct {
  /* resolve */
  int32_t B;
  int32_t k;
  int32_t *pos;
  uint32_t *stamp;
  uint32_t *clock;
  int32_t *err;
  uint8_t *rows;
  int64_t rec_bytes;
  const uint8_t *pool;
  int64_t pool_len;
  const int32_t *topk;
  int32_t *slots;
  int32_t *miss;
  /* attention: kind 0 = MHA/GQA, 1 = latent */
  int32_t kind;
  int32_t Hq;
  int32_t Hkv;
  int32_t D;
  int32_t Dl;
  int32_t Dr;
  int32_t kv_dtype;
  int32_t q_dtype;
  float sm_scale;
  const void *q;
  float *out;
} oracle_unit;

/* Resolve then attend for every unit; units are independent, so they are
 * spread over n_threads OpenMP threads (<= 0: the runtime's default team).
 * The team is set per call (a num_threads clause), leaving the process-wide
 * setting alone. Returns the number of threads that get work: the team
 * size, at most one thread per unit. */
int oracle_step_batch(int32_t n, const oracle_unit *u, int32_t n_threads) {
  int used = 1;
#ifdef _OPENMP
  const int team = n_threads > 0 ? n_threads : omp_get_max_threads();
  used = team < n ? team : (n > 0 ? n : 1);
#pragma omp parallel for num_threads(team) schedule(dynamic, 1)
#endif
  for (int32_t i = 0; i < n; ++i) {
    const oracle_unit *x = &u[i];
    oracle_resolve(x->B, x->pos, x->stamp, x->clock, x->err, x->rows,
                   x->rec_bytes, x->pool, x->pool_len, x->topk, x->k, x->slots,
                   x->miss);
    if (x->kind == 0)
      oracle_attend_mha(x->Hq, x->Hkv, x->D, x->kv_dtype, x->q_dtype, x->q,
                        x->rows, x->rec_bytes, x->B, x->slots, x->k,
                        x->sm_scale, x->out, NULL);
    else
      oracle_attend_latent(x->Hq, x->Dl, x->Dr, x->kv_dtype, x->q_dtype, x->q,
                           x->rows, x->rec_bytes, x->B, x->slots, x->k,
                           x->sm_scale, x->out, NULL);
  }
  return used;
}
