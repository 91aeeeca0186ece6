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
//      group of 16 heads (MFMA A = rows, B = Q^T), reusing the loaded rows;
//   2. the four waves' partial score tiles are summed through LDS in a fixed
//      order (one barrier), so every wave holds the same scores;
//   3. each wave runs the same online softmax (log2 units) per head group
//      and rounds P to bf16;
//   4. each wave writes its value slice transposed into its own LDS area
//      once (two slots packed per 32-bit word) and accumulates
//      O^T[v][head] += V^T[v][slot] P^T[slot][head] with MFMA, each value
//      tile read once and used by every head group.
// The P^T operand is the lane's own score accumulators: lane l of a 16x16
// tile holds rows 4(l/16)+i, so the lane's 8 P values (2 tiles x 4 rows)
// are used directly as the 8 k-elements of the PV operand, and the V^T
// words are laid out in that same order. While one 32-slot step computes,
// the rows of the next step and the slot ids of the one after are loading.
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
constexpr int PAST_END = -0x7FFFFFFF - 1;          // row index beyond the chunk

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even (finite inputs)
}

// Word address of value row v (0..127) of a wave's transposed-value area.
// Rows are 20 words apart (16 used): 16-byte aligned, and 8 (or 16)
// consecutive rows start in distinct groups of 4 banks, so the 16-byte reads
// of the PV operand (one row per lane) are free of bank conflicts.
__device__ __forceinline__ int vt_row(int v) { return LAT_VT_STRIDE * v; }

// A tile row: its slot (or PAST_END), and in fetch mode its pool position
// when it must come from the host (else -1).
struct RowRef {
  int slot;
  int src;
};

template <int HG, bool FETCH>
__global__ __launch_bounds__(LAT_THREADS) void hs_k_attn_latent(
    const UnitDesc *__restrict__ units, const uint16_t *__restrict__ q_all,
    const int32_t *__restrict__ slots_all, int n_units, int k, float scale_log2, int S,
    int chunk, float *__restrict__ ws_o, float *__restrict__ ws_ml, float *__restrict__ out) {
  constexpr int Hq = HG * 16;
  __shared__ uint32_t s_vt[4][LAT_VT_WORDS];
  __shared__ floatx4 s_part[2][HG][4][2][64];

  // XCD-aware order: the S splits of a unit get block ids equal mod 8, i.e.
  // run on one XCD and share its L2 for the unit's queries.
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j8 = b >> 3;
  const int sp = j8 % S;
  const int u = (j8 / S) * 8 + xcd;
  if (u >= n_units) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int q4 = lane >> 4;

  const UnitDesc d = units[u];
  const int B = d.B;
  const int i_begin = sp * chunk;
  const int i_end = min(k, i_begin + chunk);
  const int32_t *slots = slots_all + (size_t)u * k;
  const int64_t pool_len = FETCH ? *d.len : 0;

  // the wave's d-steps: 4 latent ones, and one rope step for waves 0 and 1
  const int n_own = w < 2 ? 5 : 4;
  bf16x8 qb[HG][5];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + w;
      if (jj < n_own)
        qb[hg][jj] = *(const bf16x8 *)(q_all + ((size_t)u * Hq + hg * 16 + r) * LAT_DK +
                                       32 * ds + 8 * q4);
      else
        qb[hg][jj] = __builtin_bit_cast(bf16x8, short8{0, 0, 0, 0, 0, 0, 0, 0});
    }
  }

  floatx4 o[HG][8];
  float m_run[HG], l_run[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    m_run[hg] = NEG_INF;
    l_run[hg] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) o[hg][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = false;
  uint32_t *vt = s_vt[w];

  auto fetch_ids = [&](int t0, RowRef &ra, RowRef &rb) {
    const bool ina = t0 + r < i_end, inb = t0 + 16 + r < i_end;
    ra.slot = ina ? slots[t0 + r] : PAST_END;
    rb.slot = inb ? slots[t0 + 16 + r] : PAST_END;
    if (FETCH) {
      ra.src = ina ? d.fsrc[t0 + r] : -1;
      rb.src = inb ? d.fsrc[t0 + 16 + r] : -1;
    } else {
      ra.src = rb.src = -1;
    }
  };
  // Loads the wave's slices of one tile row: from its slot in HBM, or (fetch
  // mode, just-resolved miss) from the host pool. Invalid rows read 0.
  auto load_row = [&](const RowRef &rf, v4u *dst) {
    const bool valid = (unsigned)rf.slot < (unsigned)B;
    if (!valid && rf.slot != PAST_END) bad = true;
    const bool from_host = FETCH && valid && rf.src >= 0;
    if (from_host && (int64_t)rf.src >= pool_len) bad = true;
    const bool host_ok = from_host && (int64_t)rf.src < pool_len;
    const uint8_t *p = host_ok ? d.pool + (size_t)rf.src * LAT_REC + 16 * q4
                               : d.rows + (size_t)(valid ? rf.slot : 0) * LAT_REC + 16 * q4;
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + w;
      dst[jj] = v4u{0, 0, 0, 0};
      if (jj < n_own && valid && (host_ok || !from_host)) {
        if (host_ok)
          dst[jj] = __builtin_nontemporal_load((const v4u *)(p + 64 * ds));
        else
          dst[jj] = *(const v4u *)(p + 64 * ds);
      }
    }
  };
  // fetch mode: the wave's slices of a host-loaded row go to the row's slot
  auto store_row = [&](const RowRef &rf, const v4u *src) {
    if (!FETCH) return;
    if ((unsigned)rf.slot >= (unsigned)B || rf.src < 0 || (int64_t)rf.src >= pool_len) return;
    uint8_t *p = d.rows + (size_t)rf.slot * LAT_REC + 16 * q4;
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + w;
      if (jj < n_own) *(v4u *)(p + 64 * ds) = src[jj];
    }
  };

  RowRef ca, cb, na, nb;
  v4u ka[5], kb[5];
  na.slot = nb.slot = PAST_END;
  na.src = nb.src = -1;
  fetch_ids(i_begin, ca, cb);
  if (i_begin + 32 < i_end) fetch_ids(i_begin + 32, na, nb);
  load_row(ca, ka);
  load_row(cb, kb);

  int it = 0;
  for (int i0 = i_begin; i0 < i_end; i0 += 32, ++it) {
    const bool has_next = i0 + 32 < i_end;
    v4u xa[5], xb[5];
    RowRef nna, nnb;
    nna.slot = nnb.slot = PAST_END;
    nna.src = nnb.src = -1;
    if (has_next) {
      load_row(na, xa);
      load_row(nb, xb);
      if (i0 + 64 < i_end) fetch_ids(i0 + 64, nna, nnb);
    }

    // partial scores of this wave's d-slices, every head group
    floatx4 acc[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      acc[hg][0] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[hg][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 5; ++jj) {
        if (jj < n_own) {
          acc[hg][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ka[jj]), qb[hg][jj], acc[hg][0], 0, 0, 0);
          acc[hg][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kb[jj]), qb[hg][jj], acc[hg][1], 0, 0, 0);
        }
      }
    }
    store_row(ca, ka);
    store_row(cb, kb);
    // transposed value slice: value row 32jj + 8q4 + e, column r, packed
    // (tile 0 low half, tile 1 high half) with one v_perm_b32 per word
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = ka[jj][e], c = kb[jj][e];
        const int v = 32 * jj + 8 * q4 + 2 * e;
        vt[vt_row(v) + r] = __builtin_amdgcn_perm(c, a, 0x05040100u);
        vt[vt_row(v + 1) + r] = __builtin_amdgcn_perm(c, a, 0x07060302u);
      }
    }
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      s_part[it & 1][hg][w][0][lane] = acc[hg][0];
      s_part[it & 1][hg][w][1][lane] = acc[hg][1];
    }
    lds_barrier();

    // per head group: full scores (fixed summation order), online softmax
    bf16x8 pB[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      floatx4 sc0 = s_part[it & 1][hg][0][0][lane], sc1 = s_part[it & 1][hg][0][1][lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        sc0 += s_part[it & 1][hg][ww][0][lane];
        sc1 += s_part[it & 1][hg][ww][1][lane];
      }
      // lane holds slots i0 + 16t + 4q4 + i for head 16hg + r; element e = 2i + t
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx0 = i0 + 4 * q4 + i, idx1 = i0 + 16 + 4 * q4 + i;
        sv[2 * i] = idx0 < i_end ? sc0[i] * scale_log2 : NEG_INF;
        sv[2 * i + 1] = idx1 < i_end ? sc1[i] * scale_log2 : NEG_INF;
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run[hg], mx);  // finite: slot i0 is always inside the chunk
      const float alpha = exp2_fast(m_run[hg] - mn);
      uint32_t pbits[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pbits[e] = f32_to_bf16_bits(exp2_fast(sv[e] - mn));
        psum += __uint_as_float(pbits[e] << 16);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run[hg] = l_run[hg] * alpha + psum;
      m_run[hg] = mn;
      const v4u pw = {pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16),
                      pbits[4] | (pbits[5] << 16), pbits[6] | (pbits[7] << 16)};
      pB[hg] = __builtin_bit_cast(bf16x8, pw);
      if (__any(alpha != 1.f)) {  // the running max moved for some head
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) o[hg][jj] *= alpha;
      }
    }
    // PV: each value tile is read once and used by every head group
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const v4u a = *(const v4u *)(vt + vt_row(16 * jj + r) + 4 * q4);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
        o[hg][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pB[hg],
                                                             o[hg][jj], 0, 0, 0);
    }
    if (has_next) {
#pragma unroll
      for (int jj = 0; jj < 5; ++jj) {
        ka[jj] = xa[jj];
        kb[jj] = xb[jj];
      }
      ca = na;
      cb = nb;
      na = nna;
      nb = nnb;
    }
  }

  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad && tid == 0) atomicOr(&d.ctl[CTL_ERR], HS_ERR_SLOT);

  // lane holds O^T[v = 128w + 16jj + 4q4 + i][head 16hg + r]
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const size_t row = (size_t)u * Hq + hg * 16 + r;
    if (S == 1) {
      const float inv = any_bad ? __builtin_nanf("") : 1.f / l_run[hg];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const floatx4 v = o[hg][jj] * inv;
        *(floatx4 *)(out + row * LAT_DL + 128 * w + 16 * jj + 4 * q4) = v;
      }
    } else {
      float *dst = ws_o + (row * S + sp) * LAT_DL + 128 * w + 4 * q4;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) *(floatx4 *)(dst + 16 * jj) = o[hg][jj];
      if (w == 0 && q4 == 0) {
        ws_ml[(row * S + sp) * 2] = any_bad ? __builtin_nanf("") : m_run[hg];
        ws_ml[(row * S + sp) * 2 + 1] = l_run[hg];
      }
    }
  }
}

template <int HG, bool FETCH>
hipError_t launch_latent_t(const AttnLatentArgs &a, hipStream_t stream) {
  const int grid = ((a.n_units + 7) / 8) * 8 * a.splits;
  trace_begin(HS_TRACE_ATTN, stream);
  hipLaunchKernelGGL((hs_k_attn_latent<HG, FETCH>), dim3(grid), dim3(LAT_THREADS), 0, stream,
                     a.units, a.q, a.slots, a.n_units, a.k, a.scale_log2, a.splits, a.chunk,
                     a.ws_o, a.ws_ml, a.out);
  trace_end(stream);
  return hipGetLastError();
}

template <bool FETCH>
hipError_t launch_latent_f(const AttnLatentArgs &a, hipStream_t stream) {
  switch (a.Hq / 16) {
    case 1: return launch_latent_t<1, FETCH>(a, stream);
    case 2: return launch_latent_t<2, FETCH>(a, stream);
    case 4: return launch_latent_t<4, FETCH>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream) {
  hipError_t e = a.fetch ? launch_latent_f<true>(a, stream) : launch_latent_f<false>(a, stream);
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.ws_o, a.ws_ml, a.n_units * a.Hq, a.splits, LAT_DL, a.out, stream);
}

}  // namespace hs
