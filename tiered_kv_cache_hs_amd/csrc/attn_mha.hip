// Top-k sparse decode attention over resolved slots, MHA/GQA record layout
// ([K: Hkv x D][V: Hkv x D] per row), plus the split-k combine.
//
// HiSparse summary (marsggbo.github.io, 2026-09-23), section 3, arrow 4:
// the physical slots go to the sparse-attention backend, which gathers the
// selected rows from the device buffer; the output equals full-KV attention
// at the selected positions. The page does not describe the backend; this
// one is written for gfx950.
//
// Design: the work is HBM-bound (about 1 flop per byte), so it stays on the
// vector ALUs. A group of LPS lanes owns one slot's K (or V) slice of one KV
// head (16 bytes per lane, LPS = D * sizeof(T) / 16), so a wave reads
// 64 / LPS whole slices per load instruction. Every lane keeps the online
// softmax state (running max and sum in log2 units, and its 16-byte share of
// the value accumulator) for the GQ query heads of its KV head. Loads of
// UNROLL slots are issued before any of them is used. The split-k factor
// spreads a unit's k slots over enough workgroups to fill 256 CUs; each
// workgroup writes (m, l, acc) partials that hs_k_combine merges. The split
// boundaries depend only on the index in the selection, never on the slot,
// so the slot-indirected result is bit-identical to the same computation
// over a full-KV copy.
#include "hs_device.h"

namespace hs {

namespace {

constexpr int MHA_THREADS = 256;
constexpr int MHA_WAVES = MHA_THREADS / 64;
constexpr int MHA_UNROLL = 4;
constexpr float NEG_INF = -__builtin_huge_valf();

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int EPL = 4;  // elements per 16 bytes
  __device__ static void unpack(const v4u &w, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  }
};
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int EPL = 8;
  __device__ static void unpack(const v4u &w, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(w[e] << 16);
      f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float fdpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8, 16, 32 or 64); every lane of a
// group gets the group's sum. Within a row of 16 lanes the steps are DPP lane
// moves (quad swaps, half-row mirror, row mirror); wider groups add xor
// shuffles across rows.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group width");
  x += fdpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += fdpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += fdpp<0x141>(x);  // row_half_mirror: the other quad of the half-row
  if (G >= 16) x += fdpp<0x140>(x);  // row_mirror: the other half-row
  if (G >= 32) x += __shfl_xor(x, 16, 64);
  if (G >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Merge state (m2, l2, a2) into (m, l, a); m in log2 units, -inf = empty.
template <int EPL>
__device__ __forceinline__ void merge_state(float &m, float &l, float *a, float m2, float l2,
                                            const float *a2) {
  const float mn = fmaxf(m, m2);
  const float f1 = (m == NEG_INF) ? 0.f : exp2_fast(m - mn);
  const float f2 = (m2 == NEG_INF) ? 0.f : exp2_fast(m2 - mn);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = a[e] * f1 + a2[e] * f2;
  m = mn;
}

// FETCH: resolve + attention fused. A selected row that the resolve just
// assigned to a victim slot is read from the host pool instead of the slot,
// and the workgroup stores its head's K and V slices into the slot's row; the
// workgroups of the Hkv heads together write the whole record, each byte
// crossing the host link once.
template <typename T, int D, int GQ, bool FETCH>
__global__ __launch_bounds__(MHA_THREADS) void hs_k_attn_mha(
    const UnitDesc *__restrict__ units, const T *__restrict__ q_all,
    const int32_t *__restrict__ slots_all, int k, int Hq, int Hkv, float scale_log2,
    int S, int chunk, int rec_bytes, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    float *__restrict__ out) {
  constexpr int EPL = Elem<T>::EPL;
  constexpr int LPS = D / EPL;          // lanes per slice
  constexpr int NG = 64 / LPS;          // slice groups per wave
  constexpr int NGW = NG * MHA_WAVES;   // slice groups per workgroup
  static_assert(LPS >= 1 && LPS <= 64 && (64 % LPS) == 0, "bad slice width");

  __shared__ float s_acc[MHA_WAVES][GQ][D];
  __shared__ float s_ml[MHA_WAVES][GQ][2];

  const int b = blockIdx.x;
  const int s = b % S;
  const int rest = b / S;
  const int g = rest % Hkv;
  const int u = rest / Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = wave * NG + lane / LPS;
  const int gl = lane % LPS;

  const UnitG d = unit_g(units[u]);
  const int B = d.B;
  const int i_begin = s * chunk;
  const int i_end = min(k, i_begin + chunk);
  const int32_t *slots = slots_all + (size_t)u * k;

  float qf[GQ][EPL];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const v4u w = *(const v4u *)(q_all + ((size_t)u * Hq + g * GQ + h) * D + gl * EPL);
    Elem<T>::unpack(w, qf[h]);
  }
  const size_t koff = (size_t)g * D * sizeof(T) + (size_t)gl * 16;
  const size_t voff = (size_t)(Hkv + g) * D * sizeof(T) + (size_t)gl * 16;

  float m_run[GQ], l_run[GQ], acc[GQ][EPL];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_run[h] = NEG_INF;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  bool bad = false;
  const int64_t pool_len = FETCH ? *d.len : 0;

  for (int i0 = i_begin + grp; i0 < i_end; i0 += MHA_UNROLL * NGW) {
    v4u kw[MHA_UNROLL], vw[MHA_UNROLL];
    bool valid[MHA_UNROLL];
    int slot_of[MHA_UNROLL];
    int src[MHA_UNROLL];  // fetch mode: pool position of a just-resolved miss, else -1
#pragma unroll
    for (int uu = 0; uu < MHA_UNROLL; ++uu) {
      const int i = i0 + uu * NGW;
      valid[uu] = i < i_end;
      int slot = valid[uu] ? slots[i] : 0;
      src[uu] = (FETCH && valid[uu]) ? d.fsrc[i] : -1;
      if ((unsigned)slot >= (unsigned)B) {
        bad = true;
        slot = 0;
        src[uu] = -1;
      }
      if (FETCH && src[uu] >= 0 && (int64_t)src[uu] >= pool_len) {
        bad = true;
        src[uu] = -1;
      }
      slot_of[uu] = slot;
      const bool host = FETCH && src[uu] >= 0;
      const HS_GLOBAL uint8_t *row = host ? pool_record(d, (uint32_t)src[uu], rec_bytes)
                                          : d.rows + (size_t)slot * rec_bytes;
      if (valid[uu] && host) {
        kw[uu] = __builtin_nontemporal_load((const HS_GLOBAL v4u *)(row + koff));
        vw[uu] = __builtin_nontemporal_load((const HS_GLOBAL v4u *)(row + voff));
      } else if (valid[uu]) {
        kw[uu] = *(const HS_GLOBAL v4u *)(row + koff);
        vw[uu] = *(const HS_GLOBAL v4u *)(row + voff);
      } else {
        kw[uu] = v4u{0, 0, 0, 0};
        vw[uu] = v4u{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int uu = 0; uu < MHA_UNROLL; ++uu) {
      if (FETCH && src[uu] >= 0) {  // the fetched slices go to the slot's row
        HS_GLOBAL uint8_t *row = d.rows + (size_t)slot_of[uu] * rec_bytes;
        *(HS_GLOBAL v4u *)(row + koff) = kw[uu];
        *(HS_GLOBAL v4u *)(row + voff) = vw[uu];
      }
      float kf[EPL], vf[EPL];
      Elem<T>::unpack(kw[uu], kf);
      Elem<T>::unpack(vw[uu], vf);
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qf[h][e], kf[e], dot);
        dot = group_sum<LPS>(dot);
        if (valid[uu]) {
          const float sc = dot * scale_log2;
          const float mn = fmaxf(m_run[h], sc);
          const float a = exp2_fast(m_run[h] - mn);
          const float p = exp2_fast(sc - mn);
          l_run[h] = l_run[h] * a + p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(acc[h][e], a, p * vf[e]);
          m_run[h] = mn;
        }
      }
    }
  }

  // merge the slice groups of a wave (butterfly over lane offsets >= LPS)
#pragma unroll
  for (int o = LPS; o < 64; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float m2 = __shfl_xor(m_run[h], o, 64);
      const float l2 = __shfl_xor(l_run[h], o, 64);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[h][e], o, 64);
      merge_state<EPL>(m_run[h], l_run[h], acc[h], m2, l2, a2);
    }
  }
  if (lane < LPS) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][gl * EPL + e] = acc[h][e];
      if (lane == 0) {
        s_ml[wave][h][0] = m_run[h];
        s_ml[wave][h][1] = l_run[h];
      }
    }
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad && tid == 0) set_error(d.ctl, HS_ERR_SLOT);

  // merge the waves; threads index (head, element)
  for (int t = tid; t < GQ * D; t += MHA_THREADS) {
    const int h = t / D, e = t - h * D;
    float m = s_ml[0][h][0], l = s_ml[0][h][1], a = s_acc[0][h][e];
#pragma unroll
    for (int w = 1; w < MHA_WAVES; ++w)
      merge_state<1>(m, l, &a, s_ml[w][h][0], s_ml[w][h][1], &s_acc[w][h][e]);
    const size_t row = (size_t)u * Hq + g * GQ + h;
    if (S == 1) {
      out[row * D + e] = any_bad ? __builtin_nanf("") : a / l;
    } else {
      ws_o[(row * S + s) * D + e] = a;
      if (e == 0) {
        ws_ml[(row * S + s) * 2] = any_bad ? __builtin_nanf("") : m;
        ws_ml[(row * S + s) * 2 + 1] = l;
      }
    }
  }
}

// Merge S <= COMBINE_MAX_S split partials per output row.
// Grid: rows; block: 256 threads. Wave 0 turns the S (m, l) pairs into
// weights w_s = 2^(m_s - max m) and L = sum w_s l_s; then every thread sums
// its output elements over the splits with the loads of 8 splits in flight.
constexpr int COMBINE_MAX_S = 64;

// Partial element i of a row: fp32, or bf16 widened exactly.
__device__ __forceinline__ float partial_at(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float partial_at(const uint16_t *p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
// Partial elements i, i + 1 (i even) as loaded, and widened to fp32 (kept
// apart so that every load of a thread is issued before the first
// conversion waits for one).
__device__ __forceinline__ float2 partial_pair_raw(const float *p, size_t i) {
  return *(const float2 *)(p + i);
}
__device__ __forceinline__ uint32_t partial_pair_raw(const uint16_t *p, size_t i) {
  return *(const uint32_t *)(p + i);
}
__device__ __forceinline__ float2 widen_pair(float2 v) { return v; }
__device__ __forceinline__ float2 widen_pair(uint32_t w) {
  return float2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
}
template <typename P>
using partial_pair_t = decltype(partial_pair_raw((const P *)nullptr, 0));

template <typename P>
__global__ __launch_bounds__(256) void hs_k_combine(const P *__restrict__ ws_o,
                                                    const float *__restrict__ ws_ml, int S,
                                                    int dv, float *__restrict__ out) {
  __shared__ float s_w[COMBINE_MAX_S];
  __shared__ float s_inv;
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const float m = tid < S ? ws_ml[(row * S + tid) * 2] : NEG_INF;
    const float l = tid < S ? ws_ml[(row * S + tid) * 2 + 1] : 0.f;
    const bool nan = __any(m != m);
    float M = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float wgt = (m == NEG_INF) ? 0.f : exp2_fast(m - M);
    float L = wgt * l;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if (tid < S) s_w[tid] = wgt;
    if (tid == 0) s_inv = nan ? __builtin_nanf("") : 1.f / L;
  }
  __syncthreads();
  const float inv = s_inv;
  const P *src = ws_o + row * S * dv;
  for (int e = tid; e < dv; e += blockDim.x) {
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) o = fmaf(s_w[s], partial_at(src, (size_t)s * dv + e), o);
    out[row * dv + e] = o * inv;
  }
}

// The same merge for S <= MAXS splits and rows of at most 512 elements, in
// one memory round trip and without LDS or a barrier: lane s of every wave
// loads split s's (m, l) while each thread loads its two output elements'
// partials; the weights then come from wave reductions and shuffles, in the
// same arithmetic as the kernel above (same L tree, same order of the
// weighted sums), so both give identical results. With fp32 partials it is
// faster up to 8 splits (2 splits: 8.5 -> 7.2 us; 4: 13.4 -> 11.1), even at
// 8, and slower at 16 (7.8 -> 8.2 us), where the serial chain of 16 shuffles
// and products costs more than the barrier it saves; with bf16 partials it
// is faster at 16 too (4.7-4.8 -> 4.0-4.3 us for 8 latent units of 64 heads).
constexpr int COMBINE_WAVE_S = 8;
constexpr int COMBINE_WAVE_S_BF16 = 16;

template <typename P, int MAXS>
__global__ __launch_bounds__(256) void hs_k_combine_wave(const P *__restrict__ ws_o,
                                                         const float *__restrict__ ws_ml, int S,
                                                         int dv, float *__restrict__ out) {
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int e = 2 * threadIdx.x;  // dv <= 512: at most one pair of elements per thread
  const bool has = e < dv;
  const P *src = ws_o + row * S * dv + (has ? e : 0);
  const float2 my =
      lane < S ? ((const float2 *)ws_ml)[row * S + lane] : float2{NEG_INF, 0.f};
  partial_pair_t<P> ov[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < S) ov[s] = partial_pair_raw(src, (size_t)s * dv);
  const bool nan = __any(my.x != my.x);
  float M = my.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float wgt = (my.x == NEG_INF) ? 0.f : exp2_fast(my.x - M);
  float L = wgt * my.y;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < S) {
      const float ws = __shfl(wgt, s, 64);
      const float2 v = widen_pair(ov[s]);
      o0 = fmaf(ws, v.x, o0);
      o1 = fmaf(ws, v.y, o1);
    }
  }
  if (has) {
    const float inv = nan ? __builtin_nanf("") : 1.f / L;
    *(float2 *)(out + row * dv + e) = float2{o0 * inv, o1 * inv};
  }
}

template <typename T, int D, int GQ, bool FETCH>
hipError_t launch_mha_t(const AttnMhaArgs &a, hipStream_t stream) {
  const int grid = a.n_units * a.Hkv * a.splits;
  return launch_k(HS_TRACE_ATTN, hs_k_attn_mha<T, D, GQ, FETCH>, dim3(grid), dim3(MHA_THREADS),
                  0, stream, a.units, (const T *)a.q, a.slots, a.k, a.Hq, a.Hkv, a.scale_log2,
                  a.splits, a.chunk, a.rec_bytes, a.ws_o, a.ws_ml, a.out);
}

template <typename T, int D, bool FETCH>
hipError_t launch_mha_g(const AttnMhaArgs &a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_mha_t<T, D, 1, FETCH>(a, stream);
    case 2: return launch_mha_t<T, D, 2, FETCH>(a, stream);
    case 4: return launch_mha_t<T, D, 4, FETCH>(a, stream);
    case 8: return launch_mha_t<T, D, 8, FETCH>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_mha_d(const AttnMhaArgs &a, hipStream_t stream) {
  return a.fetch ? launch_mha_g<T, D, true>(a, stream) : launch_mha_g<T, D, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_mha(const AttnMhaArgs &a, hipStream_t stream) {
  hipError_t e;
  if (a.dtype == HS_F32)
    e = a.D == 64 ? launch_mha_d<float, 64>(a, stream) : launch_mha_d<float, 128>(a, stream);
  else
    e = a.D == 64 ? launch_mha_d<uint16_t, 64>(a, stream)
                  : launch_mha_d<uint16_t, 128>(a, stream);
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.ws_o, 0, a.ws_ml, a.n_units * a.Hq, a.splits, a.D, a.out, stream);
}

namespace {
template <typename P>
hipError_t launch_combine_t(const P *ws_o, const float *ws_ml, int rows, int splits, int dv,
                            float *out, hipStream_t stream) {
  const bool wave_rows = dv % 2 == 0 && dv <= 512;
  if (wave_rows && splits <= COMBINE_WAVE_S)
    return launch_k(HS_TRACE_COMBINE, hs_k_combine_wave<P, COMBINE_WAVE_S>, dim3(rows), dim3(256),
                    0, stream, ws_o, ws_ml, splits, dv, out);
  if (wave_rows && sizeof(P) == 2 && splits <= COMBINE_WAVE_S_BF16)
    return launch_k(HS_TRACE_COMBINE, hs_k_combine_wave<P, COMBINE_WAVE_S_BF16>, dim3(rows),
                    dim3(256), 0, stream, ws_o, ws_ml, splits, dv, out);
  return launch_k(HS_TRACE_COMBINE, hs_k_combine<P>, dim3(rows), dim3(256), 0, stream, ws_o,
                  ws_ml, splits, dv, out);
}
}  // namespace

hipError_t launch_combine(const void *ws_o, int partial_bf16, const float *ws_ml, int rows,
                          int splits, int dv, float *out, hipStream_t stream) {
  return partial_bf16
             ? launch_combine_t((const uint16_t *)ws_o, ws_ml, rows, splits, dv, out, stream)
             : launch_combine_t((const float *)ws_o, ws_ml, rows, splits, dv, out, stream);
}

}  // namespace hs
