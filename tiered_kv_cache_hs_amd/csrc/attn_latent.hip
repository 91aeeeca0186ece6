// Top-k sparse decode attention over resolved slots for the latent
// (MLA-style) record: one 576-element bf16 row per token, [latent 512 |
// rope 64], shared by all query heads; the key is the whole row and the value
// its latent part.
//
// HiSparse summary (marsggbo.github.io, 2026-09-23), section 3, arrow 4: the
// resolved slots feed the sparse-attention backend; section 5 sizes it (about
// 60 us per layer at per-GPU batch 8 on the page's hardware). The backend
// itself is not described on the page; this one is written for gfx950.
//
// With 16-64 query heads sharing each row, QK^T is a real dense contraction
// (heads x 576 by 576 x slots) and PV another (heads x slots by slots x 512),
// about 111 flop per byte read at 64 heads: bandwidth-bound only if both run
// on the bf16 matrix cores, so both use v_mfma_f32_16x16x32_bf16.
//
// Work split. A workgroup (4 waves) owns a chunk of one unit's selection for
// every query head, walked 32 slots at a time (two 16-row MFMA tiles). The
// 18 32-wide d-steps of the 576-element key are divided among the waves
// (wave w: latent d-steps 4w..4w+3, plus rope d-step 16+w for w < 2), so
// every row byte is loaded once per workgroup and each wave's latent slice is
// exactly the value slice [128w, 128w+128) it needs for PV. Per 32 slots:
//   1. each wave multiplies its row slices by the Q^T slices of every head
//      group of 16 heads (MFMA A = rows, B = Q^T), reusing the loaded rows,
//      and writes its value slice transposed into its own LDS area (two
//      slots packed per 32-bit word);
//   2. the partial score tiles go to LDS (barrier); wave g sums the four
//      partials of head group g in a fixed order and runs that group's
//      online softmax (log2 units), rounding P to bf16 (barrier);
//   3. every wave reads P of every head group and accumulates
//      O^T[v][head] += V^T[v][slot] P^T[slot][head] with MFMA, each value
//      tile read once and used by every head group.
// The running maximum is a lazy reference: it moves only when a score
// exceeds it by more than 2^8 (log2 units), so P stays in [0, 256] and the
// accumulators are rescaled only on those rare steps; the partial state
// (reference max, sum, accumulators) combines exactly as with the true max.
// The P^T operand is the softmax lane's own score layout: lane l of a 16x16
// tile holds rows 4(l/16)+i, so the lane's 8 P values (2 tiles x 4 rows)
// are the 8 k-elements of the PV operand, and the V^T words are laid out in
// that same order. The chunk's slot ids are staged in LDS once; row slices
// are loaded DEPTH steps ahead (one for 16 and 64 heads per workgroup, two
// for 32) through DEPTH + 1 register buffers.
//
// Fetch mode (resolve + attention fused): a selected row that the resolve
// just assigned to a victim slot has not been copied from the host pool yet;
// the wave that needs it loads its slice straight from pinned host memory,
// uses it, and stores it into the slot's row, so the host-link transfer
// overlaps the attention over the resident rows. Each row slice is read by
// exactly one wave, so every fetched byte crosses the host link once.
#include "hs_device.h"

namespace hs {

namespace {

constexpr int LAT_THREADS = 256;
constexpr int LAT_DL = 512;
constexpr int LAT_DR = 64;
constexpr int LAT_DK = LAT_DL + LAT_DR;            // 576
constexpr int LAT_REC = LAT_DK * 2;                // 1152 bytes
constexpr int LAT_VT_STRIDE = 20;                  // words per value row (16 used)
constexpr int LAT_VT_WORDS = 128 * LAT_VT_STRIDE;  // per wave: 128 value rows
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LAT_LAZY_LOG2 = 8.f;               // reference-max slack, log2 units
// Split partials of at most this many bytes per launch are written with
// streaming (nontemporal) stores: the kernel then ends without writing back
// that many dirty L2 lines, and the combine, latency-bound at that size,
// reads them as fast from memory. Larger partials are read faster by the
// combine when they were written through the cache. (Batch-8 MLA, 8.4 MB of
// partials: attention 21.0 -> 19.9 us, combine unchanged; 64 requests,
// 34 MB: attention +2.2 us, combine +4 us.)
constexpr size_t LAT_STREAM_PARTIAL_BYTES = 16u << 20;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotation of a value within each row of 16 lanes (DPP row_ror); every
// lane reads a lane of its own row, so the move folds into the consuming
// max or add as a DPP operand.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xF, 0xF, true));
}
// Maximum / sum over the 16 lanes of a row, left in every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  return fmaxf(x, row_ror<1>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  return x + row_ror<1>(x);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest even, v_cvt_pk_bf16_f32): a in the
// low half, b in the high half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
}

// The bits of x, or of a quiet NaN when c. Error outputs are stored as
// integers: the file is compiled assuming no NaN operands, so a float select
// of a NaN constant could be folded away.
__device__ __forceinline__ uint32_t nan_bits_if(bool c, float x) {
  return c ? 0x7FC00000u : __float_as_uint(x);
}

// Word address of value row v (0..127) of a wave's transposed-value area.
// Rows are 20 words apart (16 used): 16-byte aligned, and 8 (or 16)
// consecutive rows start in distinct groups of 4 banks, so the 16-byte reads
// of the PV operand (one row per lane) are free of bank conflicts.
__device__ __forceinline__ int vt_row(int v) { return LAT_VT_STRIDE * v; }

// A tile row: its slot, and in fetch mode its pool position when it must
// come from the host (else -1).
struct RowRef {
  int slot;
  int src;
};

// HG head groups of 16 per workgroup; HS workgroups split a unit's Hq =
// HS * HG * 16 heads; DEPTH steps of row loads in flight ahead of the one
// computing (1 or 2; the register budget allows 2 up to HG = 2).
//
// Score layout: QK^T is computed transposed, S^T[head][slot] = Q x K^T
// (MFMA A = Q slices, B = row slices), so a lane holds 4 heads x 1 slot per
// 16-slot tile and the reductions over slots run within a row of 16 lanes
// (DPP). Every wave issues the same loads in every step (rows past the
// chunk repeat its last row and are masked), so the number of loads in
// flight is the same on every path and each step waits only for its own.
template <int HG, int DEPTH, bool FETCH, bool STREAM>
__global__ __launch_bounds__(LAT_THREADS) void hs_k_attn_latent(
    const UnitDesc *__restrict__ units, const uint16_t *__restrict__ q_all,
    const int32_t *__restrict__ slots_all, int n_units, int k, float scale_log2, int S,
    int HS, int chunk, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    float *__restrict__ out) {
  static_assert(DEPTH == 1 || DEPTH == 2, "prefetch depth 1 or 2");
  __shared__ uint32_t s_vt[4][LAT_VT_WORDS];
  __shared__ floatx4 s_part[HG][4][2][64];
  __shared__ v4u s_p[HG][64];          // PV operand P^T of every lane
  __shared__ float s_alpha[HG][16];    // per head: rescale factor, then l
  __shared__ int s_rescale[4];         // per wave: its reference maximum moved
  __shared__ int s_ids[LAT_MAX_CHUNK];
  __shared__ int s_src[FETCH ? LAT_MAX_CHUNK : 1];

  // XCD-aware order: the S x HS workgroups of a unit get block ids equal
  // mod 8, i.e. run on one XCD and share its L2 for the unit's queries and,
  // across head splits, its rows.
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j8 = b >> 3;
  const int sp = j8 % S;
  const int hh = (j8 / S) % HS;
  const int u = (j8 / (S * HS)) * 8 + xcd;
  if (u >= n_units) return;
  const int Hq = HS * HG * 16;
  const int h0 = hh * HG * 16;  // first head of this workgroup

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int r = lane & 15;
  const int q4 = lane >> 4;

  const UnitG d = unit_g(units[u]);
  const int B = d.B;
  const int i_begin = sp * chunk;
  const int i_end = min(k, i_begin + chunk);
  const int n_rows = i_end - i_begin;
  // uniform by construction; said so explicitly, or the step loop compiles
  // as a divergent loop that drains every load at its back edge
  const int n_steps = __builtin_amdgcn_readfirstlane((n_rows + 31) >> 5);
  const HS_GLOBAL int32_t *slots = glb(slots_all) + (size_t)u * k;
  const int64_t pool_len = FETCH ? *d.len : 0;

  // the chunk's slot ids (and fetch sources) into LDS; the ids past the
  // chunk repeat its last row
  for (int i = tid; i < n_steps * 32; i += LAT_THREADS) {
    const int j = i_begin + min(i, n_rows - 1);
    s_ids[i] = slots[j];
    if (FETCH) s_src[i] = d.fsrc[j];
  }

  // the wave's d-steps: 4 latent ones, and one rope step for waves 0 and 1.
  // Waves 2 and 3 load rope slices too and multiply them by a zero query
  // slice, so every wave runs the same loads and MFMAs (no branch makes the
  // number of loads in flight differ between paths).
  const int n_own = w < 2 ? 5 : 4;
  bf16x8 qb[HG][5];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + (w & 1);
      qb[hg][jj] = *(const HS_GLOBAL bf16x8 *)(q_all + ((size_t)u * Hq + h0 + hg * 16 + r) *
                                                           LAT_DK + 32 * ds + 8 * q4);
    }
    if (w >= 2) qb[hg][4] = __builtin_bit_cast(bf16x8, short8{0, 0, 0, 0, 0, 0, 0, 0});
  }

  floatx4 o[HG][8];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) o[hg][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  // softmax share of wave w: head group hg_w, heads my_h + i (i < HG) of it
  // for lane (r, q4); they sit in score tile lanes r + 16 (my_h / 4),
  // elements my_h % 4 + i
  const int hg_w = w * HG / 4;
  const int my_h = (w % (4 / HG)) * 4 * HG + HG * q4;
  const float *part_src =
      (const float *)&s_part[hg_w][0][0][r + 16 * (my_h >> 2)] + (my_h & 3);
  float m_run[HG], l_run[HG];
#pragma unroll
  for (int i = 0; i < HG; ++i) {
    m_run[i] = NEG_INF;
    l_run[i] = 0.f;
  }
  bool bad = false;
  uint32_t *vt = s_vt[w];
  lds_barrier();  // s_ids complete

  struct Rows {
    v4u a[5], b[5];
    RowRef ra, rb;
  };
  // Loads the wave's slices of a tile row: from its slot in HBM, or (fetch
  // mode, just-resolved miss) from the host pool. An invalid slot sets the
  // error and reads row 0 (its output becomes NaN).
  auto load_row = [&](const RowRef &rf, v4u *dst) {
    const bool valid = (unsigned)rf.slot < (unsigned)B;
    const bool from_host = FETCH && valid && rf.src >= 0;
    const bool host_ok = from_host && (int64_t)rf.src < pool_len;
    if (!valid || from_host != host_ok) bad = true;
    // base and row index selected without branches, then one 32 x 32 -> 64
    // multiply-add
    const HS_GLOBAL uint8_t *base =
        host_ok ? (const HS_GLOBAL uint8_t *)d.pages[(uint32_t)rf.src >> d.page_shift] : d.rows;
    const uint32_t row = host_ok ? ((uint32_t)rf.src & ((1u << d.page_shift) - 1u))
                                 : (valid && !from_host ? (uint32_t)rf.slot : 0u);
    const HS_GLOBAL uint8_t *p = base + (uint64_t)row * LAT_REC + 16 * q4;
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + (w & 1);
      dst[jj] = *(const HS_GLOBAL v4u *)(p + 64 * ds);
    }
  };
  // fetch mode: the wave's slices of a host-loaded row go to the row's slot
  auto store_row = [&](const RowRef &rf, const v4u *src) {
    if (!FETCH) return;
    if ((unsigned)rf.slot >= (unsigned)B || rf.src < 0 || (int64_t)rf.src >= pool_len) return;
    HS_GLOBAL uint8_t *p = d.rows + (size_t)rf.slot * LAT_REC + 16 * q4;
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + w;
      if (jj < n_own) *(HS_GLOBAL v4u *)(p + 64 * ds) = src[jj];
    }
  };
  // loads of step st (clamped to the last step: the tail of the pipeline
  // re-reads it, and nothing uses those values)
  auto issue = [&](int st, Rows &R) {
    const int i = 32 * min(st, n_steps - 1) + r;
    R.ra.slot = s_ids[i];
    R.rb.slot = s_ids[i + 16];
    R.ra.src = FETCH ? s_src[i] : -1;
    R.rb.src = FETCH ? s_src[i + 16] : -1;
    load_row(R.ra, R.a);
    load_row(R.rb, R.b);
  };

  // One 32-slot step on the rows in `cur`; first starts the loads of the
  // step DEPTH ahead into `pre`.
  auto step = [&](int st, Rows &cur, Rows &pre) {
    issue(st + DEPTH, pre);
    const int i0 = i_begin + 32 * st;

    // 1. partial S^T tiles of this wave's d-slices, every head group
    floatx4 acc[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      acc[hg][0] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[hg][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 5; ++jj) {
        acc[hg][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qb[hg][jj], __builtin_bit_cast(bf16x8, cur.a[jj]), acc[hg][0], 0, 0, 0);
        acc[hg][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qb[hg][jj], __builtin_bit_cast(bf16x8, cur.b[jj]), acc[hg][1], 0, 0, 0);
      }
    }
    store_row(cur.ra, cur.a);
    store_row(cur.rb, cur.b);
    // transposed value slice: value row 32jj + 8q4 + e, column r, packed
    // (tile 0 low half, tile 1 high half) with one v_perm_b32 per word
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = cur.a[jj][e], c = cur.b[jj][e];
        const int v = 32 * jj + 8 * q4 + 2 * e;
        vt[vt_row(v) + r] = __builtin_amdgcn_perm(c, a, 0x05040100u);
        vt[vt_row(v + 1) + r] = __builtin_amdgcn_perm(c, a, 0x07060302u);
      }
    }
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      s_part[hg][w][0][lane] = acc[hg][0];
      s_part[hg][w][1][lane] = acc[hg][1];
    }
    lds_barrier();

    // 2. online softmax, spread over the four waves: wave w takes heads
    // hb + HG q4 + i (i < HG) of head group hg_w; lane (r, q4) holds them
    // for slots i0 + 16t + r. Scores are the four waves' partials summed in
    // a fixed order; the maximum is a lazy reference.
    {
      float sc[2][HG];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < HG; ++i) {
          float x = 0.f;
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) x += part_src[(ww * 2 + t) * 256 + i];
          sc[t][i] = x;
        }
      }
      if (i0 + 32 > i_end) {  // the last, partial step: slots past the chunk get -inf
        const bool in0 = i0 + r < i_end, in1 = i0 + 16 + r < i_end;
#pragma unroll
        for (int i = 0; i < HG; ++i) {
          sc[0][i] = in0 ? sc[0][i] : NEG_INF;
          sc[1][i] = in1 ? sc[1][i] : NEG_INF;
        }
      }
      bool moved = false;
      float alpha[HG];
      uint32_t pw[HG];
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        // raw scores; the reference maximum is kept in log2 units. It moves
        // to the row maximum when some score exceeds it by more than the
        // slack: a ballot finds out, and only then is the maximum over the
        // row's 16 lanes taken (max(x) s = max(x s) for s > 0, so the
        // decision is the one the row maximum would give)
        const float m_old = m_run[i];
        const float x = fmaxf(sc[0][i], sc[1][i]);
        if (__any(x * scale_log2 > m_old + LAT_LAZY_LOG2)) {
          const float mx = row_max16(x) * scale_log2;  // finite
          if (mx > m_old + LAT_LAZY_LOG2) m_run[i] = mx;
        }
        moved |= m_run[i] != m_old;
        alpha[i] = exp2_fast(m_old - m_run[i]);  // 1 when unchanged, 0 at the start
        pw[i] = pack_bf16(exp2_fast(__builtin_fmaf(sc[0][i], scale_log2, -m_run[i])),
                          exp2_fast(__builtin_fmaf(sc[1][i], scale_log2, -m_run[i])));
        // the lane's share of l (alpha is the same on every lane of the
        // row); the row sum is taken once, after the last step
        l_run[i] = l_run[i] * alpha[i] +
                   (__uint_as_float(pw[i] << 16) + __uint_as_float(pw[i] & 0xFFFF0000u));
      }
      // P^T operand of PV lane (head h, k-group r / 4): word r % 4 holds
      // slots 4(r / 4) + r % 4 of tiles 0 and 1
      uint32_t *pdst = (uint32_t *)&s_p[hg_w][0];
#pragma unroll
      for (int i = 0; i < HG; ++i) pdst[((r >> 2) * 16 + my_h + i) * 4 + (r & 3)] = pw[i];
      // alpha of every head every step (1 where unchanged): a group rescales
      // all its heads when any of its waves moved
      if (r == 0) {
#pragma unroll
        for (int i = 0; i < HG; ++i) s_alpha[hg_w][my_h + i] = alpha[i];
      }
      const bool any_moved = __any(moved);
      if (lane == 0) s_rescale[w] = any_moved ? 1 : 0;
    }
    lds_barrier();

    // 3. PV: each value tile is read once and used by every head group; all
    // eight tiles are read before the MFMAs so the reads overlap
    v4u vtile[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) vtile[jj] = *(const v4u *)(vt + vt_row(16 * jj + r) + 4 * q4);
    bf16x8 pB[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      pB[hg] = __builtin_bit_cast(bf16x8, s_p[hg][lane]);
      int moved = 0;  // any wave of the group moved its reference maximum
#pragma unroll
      for (int ww = hg * (4 / HG); ww < (hg + 1) * (4 / HG); ++ww) moved |= s_rescale[ww];
      if (__builtin_amdgcn_readfirstlane(moved)) {
        const float a = s_alpha[hg][r];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) o[hg][jj] *= a;
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
        o[hg][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vtile[jj]),
                                                             pB[hg], o[hg][jj], 0, 0, 0);
    }
  };

  // The loop leaves only at its latch, the remaining steps after it: an
  // exit between the register rotations gave the compiler a path from the
  // middle of the loop back to its header on which the loads of the next
  // step were still in flight, and it waited for them there, at the top of
  // every iteration (each second step then waited the whole load latency).
  int st = 0;
  if (DEPTH == 2) {
    Rows R0, R1, R2;
    issue(0, R0);
    issue(1, R1);
    for (; st + 3 <= n_steps; st += 3) {
      step(st, R0, R2);
      step(st + 1, R1, R0);
      step(st + 2, R2, R1);
    }
    if (st < n_steps) step(st++, R0, R2);
    if (st < n_steps) step(st, R1, R0);
  } else {
    Rows R0, R1;
    issue(0, R0);
    for (; st + 2 <= n_steps; st += 2) {
      step(st, R0, R1);
      step(st + 1, R1, R0);
    }
    if (st < n_steps) step(st, R0, R1);
  }

#pragma unroll
  for (int i = 0; i < HG; ++i) l_run[i] = row_sum16(l_run[i]);
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad && tid == 0) set_error(d.ctl, HS_ERR_SLOT);
  // every wave needs l of every head of the workgroup
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < HG; ++i) s_alpha[hg_w][my_h + i] = l_run[i];
  }
  lds_barrier();

  // lane holds O^T[v = 128w + 16jj + 4q4 + i][head 16hg + r]
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const size_t row = (size_t)u * Hq + h0 + hg * 16 + r;
    if (S == 1) {
      const float inv = 1.f / s_alpha[hg][r];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const floatx4 v = o[hg][jj] * inv;
        const v4u bits = {nan_bits_if(any_bad, v[0]), nan_bits_if(any_bad, v[1]),
                          nan_bits_if(any_bad, v[2]), nan_bits_if(any_bad, v[3])};
        *(HS_GLOBAL v4u *)(out + row * LAT_DL + 128 * w + 16 * jj + 4 * q4) = bits;
      }
    } else {
      HS_GLOBAL float *dst = glb(ws_o) + (row * S + sp) * LAT_DL + 128 * w + 4 * q4;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (STREAM)
          __builtin_nontemporal_store(o[hg][jj], (HS_GLOBAL floatx4 *)(dst + 16 * jj));
        else
          *(HS_GLOBAL floatx4 *)(dst + 16 * jj) = o[hg][jj];
      }
    }
  }
  if (S > 1 && r == 0) {
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      const size_t row = (size_t)u * Hq + h0 + hg_w * 16 + my_h + i;
      ((HS_GLOBAL uint32_t *)ws_ml)[(row * S + sp) * 2] = nan_bits_if(any_bad, m_run[i]);
      ws_ml[(row * S + sp) * 2 + 1] = l_run[i];
    }
  }
}

template <int HG, int DEPTH, bool FETCH, bool STREAM>
hipError_t launch_latent_t(const AttnLatentArgs &a, hipStream_t stream) {
  const int HS = a.Hq / (HG * 16);
  if (a.chunk > LAT_MAX_CHUNK || a.chunk % 32) return hipErrorInvalidValue;
  const int grid = ((a.n_units + 7) / 8) * 8 * a.splits * HS;
  return launch_k(HS_TRACE_ATTN, hs_k_attn_latent<HG, DEPTH, FETCH, STREAM>, dim3(grid),
                  dim3(LAT_THREADS), 0, stream, a.units, a.q, a.slots, a.n_units, a.k, a.scale_log2,
                  a.splits, HS, a.chunk, a.ws_o, a.ws_ml, a.out);
}

template <bool FETCH, bool STREAM>
hipError_t launch_latent_f(const AttnLatentArgs &a, hipStream_t stream) {
  switch (a.hpw / 16) {
    case 1: return launch_latent_t<1, 1, FETCH, STREAM>(a, stream);
    case 2: return launch_latent_t<2, 2, FETCH, STREAM>(a, stream);
    case 4: return launch_latent_t<4, 1, FETCH, STREAM>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream) {
  const bool stream_partials = a.splits > 1 && (size_t)a.n_units * a.Hq * a.splits * LAT_DL *
                                                      sizeof(float) <= LAT_STREAM_PARTIAL_BYTES;
  hipError_t e;
  if (a.fetch)
    e = stream_partials ? launch_latent_f<true, true>(a, stream)
                        : launch_latent_f<true, false>(a, stream);
  else
    e = stream_partials ? launch_latent_f<false, true>(a, stream)
                        : launch_latent_f<false, false>(a, stream);
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.ws_o, a.ws_ml, a.n_units * a.Hq, a.splits, LAT_DL, a.out, stream);
}

}  // namespace hs
