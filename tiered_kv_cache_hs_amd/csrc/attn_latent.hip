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
// With 64 query heads sharing each row, QK^T is a real dense contraction
// (heads x 576 by 576 x slots) and PV another (heads x slots by slots x 512),
// about 111 flop per byte read: bandwidth-bound only if both run on the bf16
// matrix cores, so both use v_mfma_f32_16x16x32_bf16.
//
// Work split. A workgroup (4 waves) owns 16 query heads and a chunk of one
// unit's selection, walked 32 slots at a time (two 16-row MFMA tiles). The
// 18 32-wide d-steps of the 576-element key are divided among the waves
// (wave w: latent d-steps 4w..4w+3, plus rope d-step 16+w for w < 2), so
// every row byte is loaded from memory once per workgroup and each wave's
// loaded latent slice is exactly the value slice [128w, 128w+128) it needs
// for PV. Per 32 slots:
//   1. each wave multiplies its row slices by its Q^T slices (MFMA A = rows,
//      B = Q^T), giving partial scores S^T[slot][head];
//   2. the four partial score tiles are summed through LDS in a fixed order
//      (one barrier), so every wave holds the same scores;
//   3. each wave runs the same online softmax (log2 units) and rounds P to
//      bf16;
//   4. each wave writes its value slice transposed into its own LDS area
//      (two slots packed per 32-bit word) and accumulates
//      O^T[v][head] += V^T[v][slot] P^T[slot][head] with MFMA for its 8
//      16-wide value tiles.
// The P^T operand is the lane's own score accumulators: lane l of a 16x16
// tile holds rows 4(l/16)+i, so the lane's 8 P values (2 tiles x 4 rows)
// are used directly as the 8 k-elements of the PV operand, and the V^T
// words are laid out in that same order. Partials (m, l, O) per split go to
// the workspace and are merged by the combine kernel.
#include "hs_device.h"

namespace hs {

namespace {

constexpr int LAT_THREADS = 256;
constexpr int LAT_DL = 512;
constexpr int LAT_DR = 64;
constexpr int LAT_DK = LAT_DL + LAT_DR;   // 576
constexpr int LAT_REC = LAT_DK * 2;       // 1152 bytes
constexpr int LAT_VT_STRIDE = 20;                 // words per value row (16 used)
constexpr int LAT_VT_WORDS = 128 * LAT_VT_STRIDE;  // per wave: 128 value rows
constexpr float NEG_INF = -__builtin_huge_valf();

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

__global__ __launch_bounds__(LAT_THREADS) void hs_k_attn_latent(
    const UnitDesc *__restrict__ units, const uint16_t *__restrict__ q_all,
    const int32_t *__restrict__ slots_all, int k, int Hq, float scale_log2, int S, int chunk,
    int n_pairs, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    float *__restrict__ out) {
  __shared__ uint32_t s_vt[4][LAT_VT_WORDS];
  __shared__ floatx4 s_part[2][4][2][64];

  // XCD-aware order: the HG head-group workgroups of one (unit, split) pair
  // get block ids that are equal mod 8, i.e. land on the same XCD and share
  // its L2 for the rows they all read.
  const int HG = Hq >> 4;
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j = b >> 3;
  const int hg = j % HG;
  const int pair = (j / HG) * 8 + xcd;
  if (pair >= n_pairs) return;
  const int u = pair / S;
  const int sp = pair - u * S;

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
  const int head = hg * 16 + r;

  // the wave's d-steps: 4 latent ones, and one rope step for waves 0 and 1
  const int n_own = w < 2 ? 5 : 4;
  bf16x8 qb[5];
#pragma unroll
  for (int jj = 0; jj < 5; ++jj) {
    const int ds = jj < 4 ? 4 * w + jj : 16 + w;
    if (jj < n_own)
      qb[jj] = *(const bf16x8 *)(q_all + ((size_t)u * Hq + head) * LAT_DK + 32 * ds + 8 * q4);
    else
      qb[jj] = __builtin_bit_cast(bf16x8, short8{0, 0, 0, 0, 0, 0, 0, 0});
  }

  floatx4 o[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) o[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  bool bad = false;
  uint32_t *vt = s_vt[w];

  int it = 0;
  for (int i0 = i_begin; i0 < i_end; i0 += 32, ++it) {
    // rows of the two tiles: slot index i0 + 16t + r
    const int ia = i0 + r, ib = i0 + 16 + r;
    const bool va = ia < i_end, vb = ib < i_end;
    int sa = va ? slots[ia] : 0;
    int sb = vb ? slots[ib] : 0;
    if ((unsigned)sa >= (unsigned)B) { bad = bad || va; sa = 0; }
    if ((unsigned)sb >= (unsigned)B) { bad = bad || vb; sb = 0; }
    const uint8_t *pa = d.rows + (size_t)sa * LAT_REC + 16 * q4;
    const uint8_t *pb = d.rows + (size_t)sb * LAT_REC + 16 * q4;

    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    v4u ka[5], kb[5];
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int ds = jj < 4 ? 4 * w + jj : 16 + w;
      ka[jj] = v4u{0, 0, 0, 0};
      kb[jj] = v4u{0, 0, 0, 0};
      if (jj < n_own) {
        if (va) ka[jj] = *(const v4u *)(pa + 64 * ds);
        if (vb) kb[jj] = *(const v4u *)(pb + 64 * ds);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      if (jj < n_own) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[jj]),
                                                        qb[jj], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[jj]),
                                                        qb[jj], acc1, 0, 0, 0);
      }
    }
    // transposed value slice: value row 32jj + 8q4 + e, column r, packed
    // (tile 0 low half, tile 1 high half)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = ka[jj][e], c = kb[jj][e];
        const int v = 32 * jj + 8 * q4 + 2 * e;
        // v_perm_b32: bytes of (c:a) -> {a.lo, c.lo} and {a.hi, c.hi}
        vt[vt_row(v) + r] = __builtin_amdgcn_perm(c, a, 0x05040100u);
        vt[vt_row(v + 1) + r] = __builtin_amdgcn_perm(c, a, 0x07060302u);
      }
    }
    // sum the four waves' partial scores in a fixed order
    s_part[it & 1][w][0][lane] = acc0;
    s_part[it & 1][w][1][lane] = acc1;
    __syncthreads();
    floatx4 sc0 = s_part[it & 1][0][0][lane], sc1 = s_part[it & 1][0][1][lane];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      sc0 += s_part[it & 1][ww][0][lane];
      sc1 += s_part[it & 1][ww][1][lane];
    }
    // lane holds slots i0 + 16t + 4q4 + i for head r; element e = 2i + t
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
    const float mn = fmaxf(m_run, mx);  // finite: slot i0 is always valid
    const float alpha = exp2_fast(m_run - mn);
    uint32_t pbits[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pbits[e] = f32_to_bf16_bits(exp2_fast(sv[e] - mn));
      psum += __uint_as_float(pbits[e] << 16);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = mn;
    const v4u pw = {pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16),
                    pbits[4] | (pbits[5] << 16), pbits[6] | (pbits[7] << 16)};
    const bf16x8 pB = __builtin_bit_cast(bf16x8, pw);
    if (__any(alpha != 1.f)) {  // the running max moved for some head
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) o[jj] *= alpha;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const v4u a = *(const v4u *)(vt + vt_row(16 * jj + r) + 4 * q4);
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pB, o[jj],
                                                       0, 0, 0);
    }
  }

  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad && tid == 0) atomicOr(&d.ctl[CTL_ERR], HS_ERR_SLOT);

  // lane holds O^T[v = 128w + 16jj + 4q4 + i][head r]
  const size_t row = (size_t)u * Hq + head;
  if (S == 1) {
    const float inv = any_bad ? __builtin_nanf("") : 1.f / l_run;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      floatx4 v = o[jj] * inv;
      *(floatx4 *)(out + row * LAT_DL + 128 * w + 16 * jj + 4 * q4) = v;
    }
  } else {
    float *dst = ws_o + (row * S + sp) * LAT_DL + 128 * w + 4 * q4;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) *(floatx4 *)(dst + 16 * jj) = o[jj];
    if (w == 0 && q4 == 0) {
      ws_ml[(row * S + sp) * 2] = any_bad ? __builtin_nanf("") : m_run;
      ws_ml[(row * S + sp) * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream) {
  const int HG = a.Hq / 16;
  const int n_pairs = a.n_units * a.splits;
  const int grid = ((n_pairs + 7) / 8) * 8 * HG;
  trace_begin(HS_TRACE_ATTN, stream);
  hipLaunchKernelGGL(hs_k_attn_latent, dim3(grid), dim3(LAT_THREADS), 0, stream, a.units, a.q,
                     a.slots, a.k, a.Hq, a.scale_log2, a.splits, a.chunk, n_pairs, a.ws_o,
                     a.ws_ml, a.out);
  trace_end(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.ws_o, a.ws_ml, a.n_units * a.Hq, a.splits, LAT_DL, a.out, stream);
}

}  // namespace hs
