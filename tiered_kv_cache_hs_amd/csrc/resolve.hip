// RESOLVE on gfx950: hit detection, LRU victim selection, in-place update and
// the batched fetch of missing records from pinned host memory.
//
// HiSparse summary (marsggbo.github.io, 2026-09-23), section 5: the selected
// positions go into an on-chip hash table; every buffer slot probes it in
// parallel and is marked hit or stale; a parallel scan picks the victims and
// updates the LRU state in place (hits most recent, fetched misses right
// after them); GPU threads then load the missing records straight from
// pinned host memory into the slots they claimed; the slot vector published
// for attention is aligned with the selection. Section 4: the state is kept
// across steps, never rebuilt from the current selection.
//
// Design on MI355X:
//  * hs_k_resolve: one 1024-thread workgroup per unit (request, layer).
//    Threads exchange data through LDS only, so its barriers order LDS only
//    and every global read is issued before the first one.
//    Thread t owns a contiguous run of SPT slots and KPT selection entries,
//    so ranks in slot order and in selection order are one exclusive block
//    scan of per-thread counts (wave64 shuffles + one LDS pass over waves).
//    Hits, for buffers of more than 1024 slots: each unit keeps an inverse
//    page table (position -> slot, -1 when not resident) in device memory,
//    updated with every eviction and fill, so one dependent read per
//    selected position tells hit from miss and the host reads of the misses
//    start without probing every slot; a hit claims its slot in an LDS
//    bitmap (a slot claimed twice is a repeated position) and only the
//    misses go into the hash table, which catches repeats among them. For
//    1024 slots or fewer, the probe is cheaper than that dependent read:
//    the whole selection goes into the hash table and every slot probes it.
//    The hash table is open addressing with linear probing in LDS,
//    capacity the power of two >= 4k (>= 2k for the largest k), keys
//    inserted with atomicCAS; inserts and lookups read 16-byte buckets of
//    four entries, so a probe run costs one LDS read per four entries.
//    Victims are the m smallest 64-bit keys (stamp << 32 | secondary) among
//    non-hit slots, where secondary = slot for an empty slot and B + position
//    otherwise; keys are distinct, so an MSB-first radix select with 8-bit
//    digits (LDS histogram, one wave scans it) finds the exact threshold.
//    Leading digits shared by every candidate are skipped, and the select
//    stops at the first digit whose bucket is taken whole.
//  * The fetch (batched gather): with 4 or more units per launch it runs in
//    the same workgroup: each thread reads 16-byte chunks of the missed
//    records with non-temporal loads from the device-mapped host pool, 4 per
//    thread in flight by default, the first batch issued as soon as the miss list
//    is known, so host-link latency overlaps the victim selection. One
//    compute unit keeps only so many host reads in flight, so smaller
//    batches fetch with hs_k_gather instead: many workgroups per unit copy
//    the fetch list the resolve wrote.
#include <type_traits>

#include "hs_device.h"

namespace hs {

namespace {

constexpr int RES_MAX_WAVES = 16;  // resolve workgroups have up to 1024 threads
constexpr int EMPTY_KEY = -1;

__device__ __forceinline__ uint32_t hash_pos(int32_t p, int hlog2) {
  return ((uint32_t)p * 0x9E3779B1u) >> (32 - hlog2);
}

// Cross-lane steps use DPP (VALU lane moves) rather than ds_bpermute, which
// goes through the LDS pipe with its latency. Controls for gfx9-family DPP:
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114,
              DPP_ROW_SHR8 = 0x118, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp(int x) {
  // lanes without a source (or outside ROW_MASK) read 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}

// Wave-wide inclusive prefix sum: Hillis-Steele within each row of 16 lanes,
// then the row totals are carried across rows with row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp<DPP_ROW_SHR1, 0xF>(x);
  x += dpp<DPP_ROW_SHR2, 0xF>(x);
  x += dpp<DPP_ROW_SHR4, 0xF>(x);
  x += dpp<DPP_ROW_SHR8, 0xF>(x);
  x += dpp<DPP_ROW_BCAST15, 0xA>(x);
  x += dpp<DPP_ROW_BCAST31, 0xC>(x);
  return x;
}

// Exclusive scan of one int per thread over the block with one barrier:
// every wave publishes its total in buf (one of two alternating rows, so a
// fast wave of the next scan cannot overwrite totals still being read), then
// each lane adds up the totals of the waves before its own.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int *total, int (*buf)[RES_MAX_WAVES],
                                               int &parity) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) buf[parity][wid] = x;
  lds_barrier();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = buf[parity][w];
    tot += t;
    before += w < wid ? t : 0;
  }
  parity ^= 1;
  *total = tot;
  return before + x - v;
}

// Wave-wide min / max of unsigned 32-bit values (result in every lane):
// prefix min/max with DPP, then lane 63 holds the answer.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  const uint32_t id = MAX ? 0u : 0xFFFFFFFFu;
  auto f = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  // inactive / sourceless lanes must contribute the identity, not 0
  auto mv = [&](uint32_t x, auto ctrl, auto rmask) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, decltype(ctrl)::value,
                                                 decltype(rmask)::value, 0xF, false);
  };
  using C1 = std::integral_constant<int, DPP_ROW_SHR1>;
  using C2 = std::integral_constant<int, DPP_ROW_SHR2>;
  using C4 = std::integral_constant<int, DPP_ROW_SHR4>;
  using C8 = std::integral_constant<int, DPP_ROW_SHR8>;
  using B15 = std::integral_constant<int, DPP_ROW_BCAST15>;
  using B31 = std::integral_constant<int, DPP_ROW_BCAST31>;
  using RA = std::integral_constant<int, 0xF>;
  using RB = std::integral_constant<int, 0xA>;
  using RC = std::integral_constant<int, 0xC>;
  v = f(v, mv(v, C1{}, RA{}));
  v = f(v, mv(v, C2{}, RA{}));
  v = f(v, mv(v, C4{}, RA{}));
  v = f(v, mv(v, C8{}, RA{}));
  v = f(v, mv(v, B15{}, RB{}));
  v = f(v, mv(v, B31{}, RC{}));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// GATHER: the kernel also copies the missed records from the host pool into
// their victim rows (the batched gather of the fetch); the first batch of
// host reads is issued as soon as the misses are known, so it overlaps the
// victim selection. Without GATHER the fetch is left to the attention
// kernels (fsrc says which rows they must read from the host).
template <int NT, int SPT, int KPT, bool GATHER, bool INV, int GB>
__global__ __launch_bounds__(NT) void hs_k_resolve(
    const UnitDesc *__restrict__ units, const int32_t *__restrict__ topk_all,
    int k, int hlog2, int rec16, int32_t *__restrict__ slots_all,
    int32_t *__restrict__ miss_all) {
  // LDS: region A holds the hash table (keys, and without INV the
  // selection index of each: 2H ints) during the hit search, then the miss
  // and victim lists (k ints each), the missed records' host addresses (k
  // 64-bit words), their positions and the victims' previous positions (k
  // ints each); region B holds slot_of[k]. s_claim (INV): one bit per slot,
  // set by the hit that claims it.
  extern __shared__ __attribute__((aligned(16))) int lds[];
  constexpr int NW = NT / 64;
  __shared__ int scan_buf[2][RES_MAX_WAVES];
  __shared__ uint32_t hist[3][256];
  __shared__ uint32_t s_claim[INV ? HS_MAX_B / 32 : 1];
  __shared__ uint32_t s_flag;
  __shared__ uint32_t s_smin, s_smax, s_cmin, s_cmax;  // stamp / secondary bounds

  const int H = 1 << hlog2;
  int *hkey = lds;
  int *hval = lds + H;
  int *miss_list = lds;
  int *victim_list = lds + k;
  uint64_t *miss_addr = (uint64_t *)(lds + 2 * k);
  int *miss_pos = lds + 4 * k;
  int *victim_old = lds + 5 * k;
  const int regionA = (2 * H > 6 * k) ? 2 * H : 6 * k;
  int *slot_of = lds + regionA;

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const UnitG d = unit_g(units[u]);
  const int B = d.B;
  const int32_t *topk = topk_all + (size_t)u * k;
  int32_t *slots = slots_all + (size_t)u * k;

  // ---- 0. every global read of the kernel is issued here, before the first
  // barrier, so the whole kernel waits for memory once
  const int64_t len = *d.len;
  const uint32_t clock = d.ctl[CTL_CLOCK];
  const int k0 = tid * KPT;
  const int s0 = tid * SPT;
  int32_t tk[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int32_t v = topk[min(k0 + j, k - 1)];  // clamped address, value masked
    tk[j] = k0 + j < k ? v : 0;
  }
  int32_t sp[SPT];
  uint32_t st[SPT];
  // the pool page (and with INV the inverse page-table entry) of each
  // selected position, clamped into the table: an invalid position is a
  // data error found below, its entries never used
  uint64_t tpage[KPT];
  int32_t tinv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (GATHER)
      tpage[j] = d.pages[min((uint32_t)tk[j] >> d.page_shift, (uint32_t)d.n_pages - 1u)];
    if (INV) tinv[j] = d.inv[min((uint32_t)tk[j], (uint32_t)d.inv_len - 1u)];
  }
  if (s0 + SPT <= B && (SPT % 4) == 0) {
    // the whole run is in range: 16-byte loads, no per-slot branches
#pragma unroll
    for (int j = 0; j < SPT; j += 4) {
      const int4 a = *(const int4 *)(d.pos + s0 + j);
      const uint4 b = *(const uint4 *)(d.stamp + s0 + j);
      sp[j] = a.x; sp[j + 1] = a.y; sp[j + 2] = a.z; sp[j + 3] = a.w;
      st[j] = b.x; st[j + 1] = b.y; st[j + 2] = b.z; st[j + 3] = b.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int s = min(s0 + j, B - 1);  // clamped address, value masked below
      const int32_t pv = d.pos[s];
      const uint32_t sv = d.stamp[s];
      sp[j] = s0 + j < B ? pv : -1;
      st[j] = s0 + j < B ? sv : 0u;
    }
  }

  for (int i = tid; i < H; i += NT) hkey[i] = EMPTY_KEY;
  for (int i = tid; i < k; i += NT) slot_of[i] = -1;
  if (INV)
    for (int i = tid; i < (B + 31) / 32; i += NT) s_claim[i] = 0u;
  if (tid < 256) {
    hist[0][tid] = 0;
    hist[1][tid] = 0;
  }
  if (tid == 0) {
    s_flag = clock >= 0x7FFFFFFFu ? HS_ERR_CLOCK : 0u;
    s_smin = 0xFFFFFFFFu;
    s_smax = 0u;
    s_cmin = 0xFFFFFFFFu;
    s_cmax = 0u;
  }
  int parity = 0;
  lds_barrier();

  // ---- 1. hits. INV: through the inverse page table, a selected position
  // whose entry names a slot is resident there; each hit claims its slot in
  // an LDS bitmap, and a slot claimed twice means a repeated position.
  // Otherwise the hits are found by the probe of step 2.
  uint32_t myflag = 0;
  if (INV) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (k0 + j >= k || tk[j] < 0 || (int64_t)tk[j] >= len) continue;
      const int c = tinv[j];
      if ((unsigned)c < (unsigned)B) {
        const uint32_t bit = 1u << (c & 31);
        if (atomicOr(&s_claim[c >> 5], bit) & bit) myflag |= HS_ERR_DUP;
        slot_of[k0 + j] = c;
      }
    }
    if (myflag) atomicOr(&s_flag, myflag);
    lds_barrier();
    myflag = 0;
  }

  // hash build (with range and repeat checks): INV, of the missed positions
  // only (repeats among them); otherwise of the whole selection, each entry
  // keeping its selection index for the probe. The KPT inserts of a thread
  // advance together, one probe step per round.
  uint32_t hcur[KPT];
  uint32_t pend = 0;  // inserts still probing
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    hcur[j] = hash_pos(tk[j], hlog2);
    if (k0 + j >= k) continue;
    if (tk[j] < 0 || (int64_t)tk[j] >= len)
      myflag |= HS_ERR_RANGE;
    else if (!INV || slot_of[k0 + j] < 0)
      pend |= 1u << j;
  }
  // INV: only the misses are inserted, so the table is nearly empty and an
  // insert almost always takes its hashed entry: one compare-and-swap there
  // first, without reading the bucket (one LDS round trip instead of two on
  // the path to the first host read; the batch-8 MLA step measured 73.1-73.4
  // against 74.0-74.5 us per layer). The rest probe on below.
  if (INV) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((pend >> j) & 1u)) continue;
      const int old = atomicCAS(&hkey[hcur[j]], EMPTY_KEY, tk[j]);
      if (old == EMPTY_KEY) {
        pend &= ~(1u << j);
      } else if (old == tk[j]) {
        myflag |= HS_ERR_DUP;
        pend &= ~(1u << j);
      } else {
        hcur[j] = (hcur[j] + 1u) & (uint32_t)(H - 1);
      }
    }
  }
  // Linear probing, read 4 entries (one 16-byte aligned bucket) at a time:
  // entries before the first empty one are taken for good (nothing is ever
  // removed), so skipping them equals failed compare-and-swaps on them.
  while (pend) {
    int4 kb[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if ((pend >> j) & 1u) kb[j] = *(const int4 *)&hkey[hcur[j] & ~3u];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((pend >> j) & 1u)) continue;
      const int e0 = (int)(hcur[j] & 3u);
      const int kv[4] = {kb[j].x, kb[j].y, kb[j].z, kb[j].w};
      int target = -1;
      bool dup = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e < e0 || target >= 0 || dup) continue;
        if (kv[e] == tk[j]) dup = true;
        else if (kv[e] == EMPTY_KEY) target = e;
      }
      if (dup) {
        myflag |= HS_ERR_DUP;
        pend &= ~(1u << j);
      } else if (target < 0) {
        hcur[j] = ((hcur[j] | 3u) + 1u) & (uint32_t)(H - 1);  // next bucket
      } else {
        const uint32_t at = (hcur[j] & ~3u) + (uint32_t)target;
        const int old = atomicCAS(&hkey[at], EMPTY_KEY, tk[j]);
        if (old == EMPTY_KEY) {
          if (!INV) hval[at] = k0 + j;
          pend &= ~(1u << j);
        } else if (old == tk[j]) {
          myflag |= HS_ERR_DUP;
          pend &= ~(1u << j);
        } else {
          hcur[j] = (at + 1u) & (uint32_t)(H - 1);  // taken meanwhile: probe on
        }
      }
    }
  }
  if (myflag) atomicOr(&s_flag, myflag);
  lds_barrier();
  const uint32_t flag = s_flag;
  if (flag) {
    for (int i = tid; i < k; i += NT) {
      slots[i] = -1;
      d.fsrc[i] = -1;
    }
    if (tid == 0) {
      d.ctl[CTL_ERR] |= flag;
      d.ctl[CTL_FETCH] = 0;
      if (miss_all) miss_all[u] = -1;
    }
    return;
  }

  // candidate keys: (stamp << 32) | secondary, secondary = slot when empty,
  // B + position otherwise; bounds of both halves over the candidates (non-
  // hit slots), met in LDS
  uint32_t hitmask = 0;
  uint64_t key[SPT];
  uint32_t candmask = 0;
  auto candidate_keys = [&]() {
    uint32_t smin = 0xFFFFFFFFu, smax = 0u, cmin = 0xFFFFFFFFu, cmax = 0u;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int s = s0 + j;
      const uint32_t second = sp[j] < 0 ? (uint32_t)s : (uint32_t)(B + sp[j]);
      key[j] = ((uint64_t)st[j] << 32) | second;
      if (s < B && !((hitmask >> j) & 1u)) {
        candmask |= 1u << j;
        smin = st[j] < smin ? st[j] : smin;
        smax = st[j] > smax ? st[j] : smax;
        cmin = second < cmin ? second : cmin;
        cmax = second > cmax ? second : cmax;
      }
    }
    smin = wave_minmax_u32<false>(smin);
    smax = wave_minmax_u32<true>(smax);
    cmin = wave_minmax_u32<false>(cmin);
    cmax = wave_minmax_u32<true>(cmax);
    if (lane == 0) {
      atomicMin(&s_smin, smin);
      atomicMax(&s_smax, smax);
      atomicMin(&s_cmin, cmin);
      atomicMax(&s_cmax, cmax);
    }
  };

  if (!INV) {
    // ---- 2. probe every slot of the buffer (SPT lookups advance together)
    uint32_t h[SPT];
    uint32_t pend = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      h[j] = hash_pos(sp[j], hlog2);
      if (s0 + j < B && sp[j] >= 0) pend |= 1u << j;
    }
    // lookups read one 16-byte bucket (4 entries) per round, entries in
    // probe order from the hashed one; a key is absent at the first empty
    while (pend) {
      int4 kb[SPT];
#pragma unroll
      for (int j = 0; j < SPT; ++j)
        if ((pend >> j) & 1u) kb[j] = *(const int4 *)&hkey[h[j] & ~3u];
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        if (!((pend >> j) & 1u)) continue;
        const int e0 = (int)(h[j] & 3u);
        const int kv[4] = {kb[j].x, kb[j].y, kb[j].z, kb[j].w};
        int found = -1;
        bool empty = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < e0 || found >= 0 || empty) continue;
          if (kv[e] == sp[j]) found = e;
          else if (kv[e] == EMPTY_KEY) empty = true;
        }
        if (found >= 0) {
          slot_of[hval[(h[j] & ~3u) + (uint32_t)found]] = s0 + j;
          hitmask |= 1u << j;
          pend &= ~(1u << j);
        } else if (empty) {
          pend &= ~(1u << j);
        } else {
          h[j] = ((h[j] | 3u) + 1u) & (uint32_t)(H - 1);  // next bucket
        }
      }
    }
    candidate_keys();
    lds_barrier();  // slot_of complete
  }

  // ---- 3. misses in selection order (the hash table is dead from here on)
  int my_miss = 0;
  bool miss_here[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = k0 + j;
    miss_here[j] = i < k && slot_of[i] < 0;
    my_miss += miss_here[j] ? 1 : 0;
  }
  int m;
  int mrank = block_excl_scan<NW>(my_miss, &m, scan_buf, parity);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (miss_here[j]) {
      miss_pos[mrank] = tk[j];
      if (GATHER)
        miss_addr[mrank] = tpage[j] + (uint64_t)((uint32_t)tk[j] & ((1u << d.page_shift) - 1u)) *
                                          (uint64_t)(rec16 * 16);
      miss_list[mrank++] = k0 + j;
    }
  }
  const int n_cand = B - (k - m);

  // ---- gather, first batch: host reads of the first GB * NT record chunks
  // (16 bytes each) of the misses, in flight during the victim selection.
  // Every lane issues the same loads and stores: a lane past the last chunk
  // takes the last chunk again (the same bytes to the same place), so no
  // load or store sits on a lane-dependent path and the waits before each
  // store count exactly the loads it needs (a guarded load made the
  // compiler wait for every earlier load before the next one).
  // GB chunks per thread per batch (the tuned swap-in block; by default 4:
  // with 8 the waves stay blocked at the issue of their first batch for
  // longer before the victim selection can run, and the batch-8 MLA step
  // measured 74.1-74.4 against 75.4-75.5 us per layer with 4 (the 64-request
  // one 852-853 against 854-855); with fewer than 4 the link is not kept
  // full (75.8-76.6))
  const size_t rec = (size_t)rec16 * 16;
  const int g_total = m * rec16;
  v4u gv[GB];
  auto chunk_src = [&](int c) {
    c = min(c, g_total - 1);
    const int j = c / rec16;
    return (const HS_GLOBAL v4u *)miss_addr[j] + (c - j * rec16);
  };
  auto chunk_dst = [&](int c) {
    c = min(c, g_total - 1);
    const int j = c / rec16;
    return (HS_GLOBAL v4u *)(d.rows + (size_t)victim_list[j] * rec) + (c - j * rec16);
  };
  if (GATHER) {
    lds_barrier();  // miss_addr complete
    if (g_total > 0) {
#pragma unroll
      for (int b = 0; b < GB; ++b) gv[b] = __builtin_nontemporal_load(chunk_src(tid + NT * b));
    }
  }

  if (INV) {
    // hit slots (claimed in step 1) and the candidate keys, while the first
    // host reads are in flight
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int s = s0 + j;
      if (s < B && ((s_claim[s >> 5] >> (s & 31)) & 1u)) hitmask |= 1u << j;
    }
    candidate_keys();
    lds_barrier();
  }

  // ---- 4. victims: the m smallest keys among non-hit slots, by an MSB-first
  // radix select over 8-bit digits; one barrier per digit (histograms rotate
  // through three buffers: the one two passes ahead is cleared while the
  // current one is read)
  uint32_t vmask = 0;
  if (m == n_cand) {
    vmask = candmask;
  } else if (m > 0) {
    // highest bit in which the candidates' keys differ: in the stamp half if
    // the stamps differ, else in the secondary half (n_cand >= 2, keys are
    // distinct); prefix starts as (smallest stamp, smallest secondary), whose
    // bits above that position every candidate shares
    const uint32_t smin_b = s_smin, smax_b = s_smax, cmin_b = s_cmin, cmax_b = s_cmax;
    const int hb = smin_b != smax_b ? 63 - __clz((int)(smin_b ^ smax_b))
                                    : 31 - __clz((int)(cmin_b ^ cmax_b));
    const uint64_t kmin = ((uint64_t)smin_b << 32) | cmin_b;
    // secondaries are below B + len: digits of the low word above that are 0
    const uint64_t sec_lim = (uint64_t)B + (uint64_t)len;
    const int sec_top = 64 - __clzll((long long)sec_lim);  // bits needed
    int sh = (hb / 8) * 8;
    uint64_t prefix = kmin;
    int need = m;
    int final_sh = 0;
    int pass = 0;
    while (true) {
      uint32_t *hcur = hist[pass % 3];
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        if (!((candmask >> j) & 1u)) continue;
        const bool match = (sh + 8 >= 64) || ((key[j] >> (sh + 8)) == (prefix >> (sh + 8)));
        if (match) atomicAdd(&hcur[(key[j] >> sh) & 255u], 1u);
      }
      lds_barrier();
      if (tid < 256) hist[(pass + 2) % 3][tid] = 0;
      // every wave finds the digit on its own (no broadcast barrier)
      const uint32_t c0 = hcur[4 * lane], c1 = hcur[4 * lane + 1];
      const uint32_t c2 = hcur[4 * lane + 2], c3 = hcur[4 * lane + 3];
      const int tot = (int)(c0 + c1 + c2 + c3);
      const int incl = wave_incl_scan(tot);
      const int excl = incl - tot;
      const bool here = excl < need && need <= incl;
      int dg = 0, below = 0, bucket = 0;
      if (here) {
        int run = excl;
        const int cc[4] = {(int)c0, (int)c1, (int)c2, (int)c3};
        for (int b = 0; b < 4; ++b) {
          if (run + cc[b] >= need) {
            dg = 4 * lane + b;
            below = run;
            bucket = cc[b];
            break;
          }
          run += cc[b];
        }
      }
      const unsigned long long ball = __ballot(here);
      const int src = __ffsll(ball) - 1;  // wave-uniform
      dg = __builtin_amdgcn_readlane(dg, src);
      below = __builtin_amdgcn_readlane(below, src);
      bucket = __builtin_amdgcn_readlane(bucket, src);
      need -= below;
      const uint64_t mask_low = (sh + 8 >= 64) ? ~0ull : ((1ull << (sh + 8)) - 1ull);
      prefix = (prefix & ~mask_low) | ((uint64_t)dg << sh);
      ++pass;
      if (need == bucket || sh == 0) {
        final_sh = sh;
        break;
      }
      // next digit; inside the low word skip the digits above the secondary's
      // highest possible bit (they are 0 for every key)
      sh -= 8;
      if (sh < 32 && sh >= sec_top) sh = ((sec_top - 1) / 8) * 8;
    }
    const uint64_t lim = prefix >> final_sh;
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (((candmask >> j) & 1u) && (key[j] >> final_sh) <= lim) vmask |= 1u << j;
  }

  // ---- 5. rank victims in ascending slot order and pair them with misses
  int vtot;
  int vrank = block_excl_scan<NW>(__popc(vmask), &vtot, scan_buf, parity);
  if (vtot != m) {
    // cannot happen for a valid state (keys are distinct); refuse to update
    for (int i = tid; i < k; i += NT) {
      slots[i] = -1;
      d.fsrc[i] = -1;
    }
    if (tid == 0) {
      d.ctl[CTL_ERR] |= HS_ERR_INTERNAL;
      d.ctl[CTL_FETCH] = 0;
      if (miss_all) miss_all[u] = -1;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    if ((vmask >> j) & 1u) {
      victim_old[vrank] = sp[j];  // the position it held, -1 if empty
      victim_list[vrank++] = s0 + j;
    }
  }
  lds_barrier();

  // ---- 6. in-place update: fills get 2c - 1, hits get 2c
  const uint32_t c = clock + 1u;
  for (int r = tid; r < m; r += NT) {
    // the position from LDS, not from the selection in global memory: a
    // global load here would wait behind every host read in flight
    const int s = victim_list[r];
    const int i = miss_list[r];
    const int32_t p = miss_pos[r];
    const int32_t op = victim_old[r];
    d.pos[s] = p;
    d.stamp[s] = 2u * c - 1u;
    slot_of[i] = s;
    // inverse page table: the evicted position leaves, the fetched one
    // enters (distinct positions: one is outside the selection, one in it)
    if (op >= 0) d.inv[op] = -1;
    d.inv[p] = s;
    // the fetch list is written even when this kernel fetches: buffers of
    // other layers that share this state fetch their own records from it
    d.work[r] = int2v{s, p};
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if ((hitmask >> j) & 1u) d.stamp[s0 + j] = 2u * c;
  lds_barrier();

  // ---- gather: the first batch into the victim rows, then the rest
  if (GATHER) {
    for (int base = 0; base < g_total; base += GB * NT) {
      if (base > 0) {
#pragma unroll
        for (int b = 0; b < GB; ++b)
          gv[b] = __builtin_nontemporal_load(chunk_src(base + tid + NT * b));
      }
#pragma unroll
      for (int b = 0; b < GB; ++b) *chunk_dst(base + tid + NT * b) = gv[b];
    }
  }

  // ---- 7. publish the slot vector, aligned with the selection
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = k0 + j;
    if (i < k) {
      slots[i] = slot_of[i];
      d.fsrc[i] = miss_here[j] ? tk[j] : -1;
    }
  }
  if (tid == 0) {
    d.ctl[CTL_CLOCK] = c;
    d.ctl[CTL_FETCH] = (uint32_t)m;
    if (miss_all) miss_all[u] = m;
  }
}

// Copy each unit's fetch list from host records into device rows: the list
// of the last resolve of the unit's state. A buffer that shares the state of
// another layer's buffer (layers reusing one selection) reads the list that
// the group's resolve wrote and copies its own layer's records, which is why
// positions are checked against this unit's pool length here (the resolve
// checked them against the resolving unit's); a position past it is not read
// (its row is rewritten with its own bytes) and sets HS_ERR_RANGE.
// Grid: n_units * G workgroups of 256 threads; lane t of workgroup g of a
// unit copies the unit's 16-byte chunks g*256 + t + j*G*256. Per batch of
// BATCH chunks a lane first loads their fetch-list and page-table entries
// (device memory), then issues all its host loads back to back, then
// stores: the vector-memory counter retires in issue order, so a device load
// issued after a host load would wait for it. Lanes past the last chunk
// repeat it (the same bytes to the same place), so every lane issues the
// same instructions and the waits count exactly. BATCH sets the host reads
// in flight per lane: a copy running alone takes 8; one running beside
// attention takes 1 (enough workgroups keep the link busy, and fewer
// long-latency reads per compute unit slow the attention less).
constexpr int GATHER_THREADS = 256;

template <int BATCH>
__global__ __launch_bounds__(GATHER_THREADS) void hs_k_gather(
    const UnitDesc *__restrict__ units, int G, int rec16) {
  const int u = blockIdx.x / G;
  const int g = blockIdx.x - u * G;
  const UnitG d = unit_g(units[u]);
  const int m = (int)d.ctl[CTL_FETCH];
  if (m <= 0 || m > d.B) return;
  const int64_t len = *d.len;
  const int total = m * rec16;
  const int stride = G * GATHER_THREADS;
  const size_t rec = (size_t)rec16 * 16;
  const uint32_t in_mask = (1u << d.page_shift) - 1u;
  bool bad = false;
  for (int b0 = g * GATHER_THREADS; b0 < total; b0 += stride * BATCH) {
    int2v w[BATCH];
    int off[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int c = min(b0 + (int)threadIdx.x + j * stride, total - 1);
      const int r = c / rec16;
      off[j] = c - r * rec16;
      w[j] = d.work[r];
    }
    uint64_t page[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      page[j] = d.pages[min((uint32_t)w[j].y >> d.page_shift, (uint32_t)d.n_pages - 1u)];
    v4u v[BATCH];
    HS_GLOBAL v4u *dst[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      dst[j] = (HS_GLOBAL v4u *)(d.rows + (size_t)w[j].x * rec) + off[j];
      const bool ok = w[j].y >= 0 && (int64_t)w[j].y < len;
      bad |= !ok;
      const HS_GLOBAL v4u *src =
          ok ? (const HS_GLOBAL v4u *)((const HS_GLOBAL uint8_t *)page[j] +
                                        (size_t)((uint32_t)w[j].y & in_mask) * rec) + off[j]
             : dst[j];
      v[j] = __builtin_nontemporal_load(src);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) *dst[j] = v[j];
  }
  if (bad) set_error(d.ctl, HS_ERR_RANGE);
}

// Re-gather every occupied row of one buffer (checkpoint restore).
__global__ __launch_bounds__(256) void hs_k_regather(const UnitDesc *__restrict__ unit,
                                                     int B, int rec16) {
  const UnitG d = unit_g(*unit);
  const size_t rec = (size_t)rec16 * 16;
  const int64_t total = (int64_t)B * rec16;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int s = (int)(c / rec16);
    const int off = (int)(c - (int64_t)s * rec16);
    const int32_t p = d.pos[s];
    if (p < 0) continue;
    const HS_GLOBAL v4u *src = (const HS_GLOBAL v4u *)pool_record(d, (uint32_t)p, rec) + off;
    ((HS_GLOBAL v4u *)(d.rows + (size_t)s * rec))[off] = __builtin_nontemporal_load(src);
  }
}

__global__ void hs_k_buffer_init(int32_t *pos, uint32_t *stamp, int32_t *fsrc, uint32_t *ctl,
                                 int B) {
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < B; s += gridDim.x * blockDim.x) {
    pos[s] = -1;
    stamp[s] = 0u;
    fsrc[s] = -1;
  }
  if (ctl && blockIdx.x == 0 && threadIdx.x < CTL_WORDS) ctl[threadIdx.x] = 0u;
}

// Write-through append from device memory into the mapped host pool (records
// [pos, pos + n), each through the unit's page table), then extend the unit's
// length.
__global__ __launch_bounds__(256) void hs_k_append(const uint64_t *pages, int page_shift,
                                                   int64_t pos, int64_t n16, int rec16,
                                                   const uint8_t *src, int64_t *len,
                                                   int64_t new_len) {
  const uint64_t mask = (1ull << page_shift) - 1ull;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n16;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / rec16;
    const int64_t off = c - r * rec16;
    const uint64_t p = (uint64_t)(pos + r);
    v4u *dst = (v4u *)(pages[p >> page_shift] + (p & mask) * (uint64_t)rec16 * 16u) + off;
    *dst = ((const v4u *)src)[c];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && *len < new_len) *len = new_len;
}

// Write-through append at the end (a decode graph replayed every step): one
// workgroup per unit writes src[u] to position *len of the unit's pool and
// then sets *len + 1. Every thread reads the length (its value addresses the
// thread's stores, so the read is complete once they are issued) before the
// LDS barrier, and only thread 0 writes it after, so all of the workgroup's
// stores go to one position; nothing in the kernel waits for the host
// writes themselves. A position with no page allocated (entry 0, or past the
// page table) is not written and sets HS_ERR_APPEND.
__global__ __launch_bounds__(256) void hs_k_append_next(const UnitDesc *__restrict__ units,
                                                        int rec16, const uint8_t *__restrict__ src) {
  const int u = blockIdx.x;
  const UnitG d = unit_g(units[u]);
  const HS_GLOBAL v4u *s = (const HS_GLOBAL v4u *)src + (size_t)u * rec16;
  // the record first: its loads do not depend on the length
  const bool mine = (int)threadIdx.x < rec16;
  const v4u v = mine ? s[threadIdx.x] : v4u{0u, 0u, 0u, 0u};
  const int64_t p = *d.len;
  const int64_t pg = p >> d.page_shift;
  const uint64_t page = (p >= 0 && pg < d.n_pages) ? d.pages[pg] : 0ull;
  if (page != 0ull) {
    const uint64_t in_page = (uint64_t)p & ((1ull << d.page_shift) - 1ull);
    HS_GLOBAL v4u *dst =
        (HS_GLOBAL v4u *)((HS_GLOBAL uint8_t *)page + in_page * (uint64_t)rec16 * 16u);
    if (mine) dst[threadIdx.x] = v;
    for (int c = threadIdx.x + 256; c < rec16; c += 256) dst[c] = s[c];
  }
  lds_barrier();
  if (threadIdx.x == 0) {
    if (page != 0ull)
      *(HS_GLOBAL int64_t *)d.len = p + 1;
    else
      set_error(d.ctl, HS_ERR_APPEND);
  }
}

// gb: host-read chunks of 16 bytes per thread per fetch batch (1, 2, 4 or
// 8; 0 = the default for the buffer size), used when the kernel gathers.
template <int NT, int SPT, int KPT>
hipError_t launch_select(const UnitDesc *d_units, int n, const int32_t *d_topk, int k,
                         int hlog2, int rec16, bool gather, int gb, size_t lds, int32_t *d_slots,
                         int32_t *d_miss, hipStream_t stream) {
  // hits through the inverse page table for buffers of more than 1024
  // slots (two or more per thread), where probing every slot costs more
  // than the table's dependent read; through the probe below that
  constexpr bool INV = SPT >= 2;
  const dim3 grid(n), block(NT);
#define HS_RES(G, B)                                                                          \
  launch_k(HS_TRACE_RESOLVE, hs_k_resolve<NT, SPT, KPT, G, INV, B>, grid, block, (uint32_t)lds, \
           stream, d_units, d_topk, k, hlog2, rec16, d_slots, d_miss)
  if (!gather) return HS_RES(false, 1);
  if (gb == 0) gb = 4;
  switch (gb) {
    case 1: return HS_RES(true, 1);
    case 2: return HS_RES(true, 2);
    case 4: return HS_RES(true, 4);
    default: return HS_RES(true, 8);
  }
#undef HS_RES
}

// picks per thread: the power of two >= k / NT
template <int NT, int SPT>
hipError_t launch_select_k(const UnitDesc *d_units, int n, const int32_t *d_topk, int k,
                           int hlog2, int rec16, bool gather, int gb, size_t lds, int32_t *d_slots,
                           int32_t *d_miss, hipStream_t stream) {
#define HS_SEL(KPT)                                                                          \
  if (k <= NT * KPT)                                                                         \
    return launch_select<NT, SPT, KPT>(d_units, n, d_topk, k, hlog2, rec16, gather, gb, lds, \
                                       d_slots, d_miss, stream);
  HS_SEL(1)
  HS_SEL(2)
#undef HS_SEL
  return launch_select<NT, SPT, 4>(d_units, n, d_topk, k, hlog2, rec16, gather, gb, lds, d_slots,
                                   d_miss, stream);
}

template <int BATCH>
hipError_t launch_gather(const UnitDesc *d_units, int n, int G, int rec16, hipStream_t stream) {
  return launch_k(HS_TRACE_GATHER, hs_k_gather<BATCH>, dim3(n * G), dim3(GATHER_THREADS), 0,
                  stream, d_units, G, rec16);
}

hipError_t launch_gather_b(const UnitDesc *d_units, int n, int G, int rec16, int batch,
                           hipStream_t stream) {
  if (batch >= 8) return launch_gather<8>(d_units, n, G, rec16, stream);
  if (batch >= 4) return launch_gather<4>(d_units, n, G, rec16, stream);
  if (batch >= 2) return launch_gather<2>(d_units, n, G, rec16, stream);
  return launch_gather<1>(d_units, n, G, rec16, stream);
}

// Hash capacity: the power of two >= 4k (load factor <= 1/4, short probe
// runs) while the resolve's LDS stays within 128 KB, else >= 2k.
int hash_log2(int k) {
  int h = 2;
  while ((1 << h) < 4 * k) ++h;
  const size_t region_a = (size_t)(2 * (1 << h) > 6 * k ? 2 * (1 << h) : 6 * k);
  if ((region_a + k) * sizeof(int) > (128u << 10)) --h;
  return h;
}

}  // namespace

size_t resolve_lds_bytes(int k) {
  const int H = 1 << hash_log2(k);
  const int regionA = (2 * H > 6 * k) ? 2 * H : 6 * k;
  return (size_t)(regionA + k) * sizeof(int);
}

hipError_t launch_resolve(const UnitDesc *d_units, int n, int max_B, const int32_t *d_topk,
                          int k, int32_t *d_slots, int32_t *d_miss, int fetch, int gb,
                          int rec_bytes, hipStream_t stream) {
  const int hlog2 = hash_log2(k);
  const size_t lds = resolve_lds_bytes(k);
  const int rec16 = rec_bytes / 16;
  const bool inl = fetch == FETCH_INLINE;
  hipError_t e;
  // 16 waves per unit; each thread owns SPT = B / 1024 consecutive slots
  if (max_B <= 1024)
    e = launch_select_k<1024, 1>(d_units, n, d_topk, k, hlog2, rec16, inl, gb, lds, d_slots,
                                 d_miss, stream);
  else if (max_B <= 2048)
    e = launch_select_k<1024, 2>(d_units, n, d_topk, k, hlog2, rec16, inl, gb, lds, d_slots,
                                 d_miss, stream);
  else if (max_B <= 4096)
    e = launch_select_k<1024, 4>(d_units, n, d_topk, k, hlog2, rec16, inl, gb, lds, d_slots,
                                 d_miss, stream);
  else if (max_B <= 8192)
    e = launch_select_k<1024, 8>(d_units, n, d_topk, k, hlog2, rec16, inl, gb, lds, d_slots,
                                 d_miss, stream);
  else
    e = launch_select_k<1024, 16>(d_units, n, d_topk, k, hlog2, rec16, inl, gb, lds, d_slots,
                                  d_miss, stream);
  if (e != hipSuccess || fetch != FETCH_KERNEL) return e;
  // enough workgroups that about 512 copy the batch's misses
  const int G = std::max(1, std::min(64, (512 + n - 1) / n));
  return launch_gather_b(d_units, n, G, rec16, gb > 0 ? gb : 8, stream);
}

// A prefetch runs beside attention kernels: 64 workgroups keep enough host
// reads in flight for the link (about 1 MB) while leaving most compute units
// free of long-latency host loads; 512 slowed the attention beside them and,
// on a batch of 8 latent units, was slower even alone.
hipError_t launch_prefetch(const UnitDesc *d_units, int n, int rec_bytes, int workgroups,
                           int batch, hipStream_t stream) {
  const int wg = workgroups > 0 ? workgroups : 64;
  const int G = std::max(1, std::min(64, (wg + n - 1) / n));
  return launch_gather_b(d_units, n, G, rec_bytes / 16, batch, stream);
}

__global__ __launch_bounds__(256) void hs_k_inv_clear(int32_t *inv, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    inv[i] = -1;
}

__global__ __launch_bounds__(256) void hs_k_inv_fill(int32_t *inv, int64_t n,
                                                     const int32_t *pos, int B) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s < B && pos[s] >= 0 && (int64_t)pos[s] < n) inv[pos[s]] = s;
}

hipError_t launch_inv_clear(int32_t *inv, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(hs_k_inv_clear, dim3((unsigned)blocks), dim3(256), 0, stream, inv, n);
  return hipGetLastError();
}

hipError_t launch_inv_rebuild(int32_t *inv, int64_t n, const int32_t *pos, int B,
                              hipStream_t stream) {
  hipError_t e = launch_inv_clear(inv, n, stream);
  if (e != hipSuccess || B < 1) return e;
  hipLaunchKernelGGL(hs_k_inv_fill, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, stream, inv,
                     n, pos, B);
  return hipGetLastError();
}

hipError_t launch_regather(const UnitDesc *d_unit, int B, int rec_bytes, hipStream_t stream) {
  const int64_t total = (int64_t)B * (rec_bytes / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(hs_k_regather, dim3((unsigned)blocks), dim3(256), 0, stream, d_unit, B,
                     rec_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_buffer_init(int32_t *pos, uint32_t *stamp, int32_t *fsrc, uint32_t *ctl, int B,
                              hipStream_t stream) {
  int blocks = (B + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(hs_k_buffer_init, dim3(blocks), dim3(256), 0, stream, pos, stamp, fsrc, ctl,
                     B);
  return hipGetLastError();
}

hipError_t launch_append(const uint64_t *d_pages, int page_shift, int64_t pos, int64_t n,
                         int rec_bytes, const uint8_t *src, int64_t *d_len, int64_t new_len,
                         hipStream_t stream) {
  const int64_t n16 = n * (rec_bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  return launch_k(HS_TRACE_APPEND, hs_k_append, dim3((unsigned)blocks), dim3(256), 0, stream,
                  d_pages, page_shift, pos, n16, rec_bytes / 16, src, d_len, new_len);
}

hipError_t launch_append_batch(const UnitDesc *d_units, int n, int rec_bytes, const uint8_t *src,
                               hipStream_t stream) {
  return launch_k(HS_TRACE_APPEND, hs_k_append_next, dim3(n), dim3(256), 0, stream, d_units,
                  rec_bytes / 16, src);
}

}  // namespace hs
