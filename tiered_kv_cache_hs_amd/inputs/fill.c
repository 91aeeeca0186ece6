/* Seeded synthetic input values for the HiSparse decode workloads.
 *
 * This file only draws numbers. It holds none of the method's arithmetic:
 * no resolve, no attention, no replacement policy. Both the CPU oracle
 * (through the tests) and the GPU path read the bytes it writes.
 *
 * Every value is a pure function of (seed, stream, request, layer, index,
 * element), so a record or query can be regenerated anywhere, in any order,
 * by any number of threads, with identical bytes.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter hash, then the
 * Box-Muller transform (Box and Muller, 1958) for N(0, sigma).
 * Rounding to bfloat16 is round-to-nearest-even on the fp32 bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* Key of one (seed, stream, request, layer, index) tuple. */
static inline uint64_t tuple_key(uint64_t seed, uint64_t stream, uint64_t req,
                                 uint64_t layer, uint64_t index) {
  uint64_t h = sm64(seed);
  h = sm64(h ^ stream);
  h = sm64(h ^ req);
  h = sm64(h ^ layer);
  return sm64(h ^ index);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

/* Fill n_elem normal values N(0, sigma) for one tuple.
 * dtype 0: float32, dtype 1: bfloat16 (RNE). dst receives n_elem values. */
static void fill_one(void *dst, int64_t n_elem, int dtype, uint64_t key,
                     double sigma) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t e = 0; e < n_elem; e += 2) {
    uint64_t x = sm64(key + (uint64_t)(e >> 1) * 0xD1B54A32D192ED03ull);
    double u1 = ((double)(x >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = ((double)(x & 0xFFFFFFFFull) + 0.5) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    float z[2];
    z[0] = (float)(sigma * rad * cos(two_pi * u2));
    z[1] = (float)(sigma * rad * sin(two_pi * u2));
    for (int j = 0; j < 2 && e + j < n_elem; ++j) {
      if (dtype == 0)
        ((float *)dst)[e + j] = z[j];
      else
        ((uint16_t *)dst)[e + j] = f32_to_bf16_rne(z[j]);
    }
  }
}

/* Records for a list of positions of one (request, layer) unit.
 * dst is the unit's record array: record p lives at dst + p * rec_bytes.
 * Each listed position p gets n_elem values keyed by (seed, stream, req,
 * layer, p). Positions are filled in parallel; the bytes do not depend on
 * the thread count. */
void hsin_fill_positions(void *dst, int64_t rec_bytes, const int64_t *positions,
                         int64_t n_pos, int64_t n_elem, int dtype, uint64_t seed,
                         uint64_t stream, int64_t req, int64_t layer,
                         double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_pos; ++i) {
    int64_t p = positions[i];
    fill_one((char *)dst + p * rec_bytes, n_elem, dtype,
             tuple_key(seed, stream, (uint64_t)req, (uint64_t)layer, (uint64_t)p),
             sigma);
  }
}

/* Records for the contiguous position range [p0, p1) of one unit. */
void hsin_fill_range(void *dst, int64_t rec_bytes, int64_t p0, int64_t p1,
                     int64_t n_elem, int dtype, uint64_t seed, uint64_t stream,
                     int64_t req, int64_t layer, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t p = p0; p < p1; ++p) {
    fill_one((char *)dst + p * rec_bytes, n_elem, dtype,
             tuple_key(seed, stream, (uint64_t)req, (uint64_t)layer, (uint64_t)p),
             sigma);
  }
}

/* A dense block of n_rows rows of n_elem values each (queries), row i keyed
 * by (seed, stream, req, layer, index0 + i), rows packed back to back. */
void hsin_fill_rows(void *dst, int64_t n_rows, int64_t n_elem, int dtype,
                    uint64_t seed, uint64_t stream, int64_t req, int64_t layer,
                    int64_t index0, double sigma) {
  int64_t es = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    fill_one((char *)dst + i * n_elem * es, n_elem, dtype,
             tuple_key(seed, stream, (uint64_t)req, (uint64_t)layer,
                       (uint64_t)(index0 + i)),
             sigma);
  }
}

/* Records of the listed positions of one unit, packed: the i-th listed
 * position's record is written at dst + i * rec_bytes. */
void hsin_fill_packed(void *dst, int64_t rec_bytes, const int64_t *positions,
                      int64_t n_pos, int64_t n_elem, int dtype, uint64_t seed,
                      uint64_t stream, int64_t req, int64_t layer, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_pos; ++i) {
    fill_one((char *)dst + i * rec_bytes, n_elem, dtype,
             tuple_key(seed, stream, (uint64_t)req, (uint64_t)layer,
                       (uint64_t)positions[i]),
             sigma);
  }
}
