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
// about 111 flop per byte read at 64 heads: both run on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16).
//
// Work split. A workgroup of 4 waves covers 32 NHG query heads (NHG = 1 or 2)
// of one (unit, split). The split's selection entries are cut into tiles of
// 32 rows, processed in steps of 3 - NHG tiles. Wave w = (x, vh), x = w & 1,
// vh = w >> 1, owns 32 heads x 256 values of the output: with NHG = 2 head
// group x over every tile; with NHG = 1 the workgroup's 32 heads over tile
// x of each step (two streams, merged at the end). Per step:
//   * rows: the 4 waves copy the step's rows from HBM straight into LDS with
//     global_load_lds (one instruction per row for its 1 KB latent part, one
//     per 8 rows for their 128-byte rope parts; 9 per wave per tile); the
//     copies of a later step go out between this step's QK^T MFMAs. The
//     step buffers rotate (three of 36 KB with NHG = 2, two of 72 KB with
//     NHG = 1) and one barrier per step tells every wave that the step has
//     landed and the buffer about to be refilled is free;
//   * S^T = K Q^T over 36 d-steps of 16: A = the tile's rows (one 1 KB LDS
//     read per d-step), B = Q^T of the wave's 32 heads (registers, read once
//     from a query tile that the prologue copies into LDS like a row tile).
//     A lane ends with 16 slots of one head: the head is the lane's column,
//     the same column as in the PV accumulators;
//   * online softmax per head in log2 units with a lazy reference maximum: it
//     moves only when a score exceeds it by more than 2^8, so P stays in
//     [0, 256] and the accumulators are rescaled only on those rare steps;
//     the maximum over a head's 32 slots (two lanes) is taken only when a
//     ballot says some score passed the slack;
//   * O^T += V^T P^T: A = V^T read with gfx950's LDS transpose reads
//     (ds_read_b64_tr_b16, two per operand), B = P^T, the softmax lane's own
//     16 values rounded to bf16 (8 per k-block of 16 slots); the slot order
//     inside a k-block follows the score layout, and the transpose reads take
//     the rows in that same order;
//   * LDS operand reads run a few MFMAs ahead of their use;
//   * the accumulators (128 per lane) live in the accumulation registers and
//     only MFMAs touch them inside the loop; the queries (144 registers) and
//     everything else fit the ordinary ones, so a compute unit runs one
//     workgroup.
// At the end each wave stages its accumulators in LDS and the workgroup
// stores whole row halves: the output (fp32, 1 KB), or its split's partial
// for the split-k combine, rounded to bf16 (512 bytes; with (m, l) in fp32).
// A split's partial is as large as the rows it covers would be in fp32 at
// 256 rows, and all workgroups write theirs at the same moment, so halving
// it shortens the kernel's end and the combine's reads.
#include "hs_device.h"

#define HS_LDS __attribute__((address_space(3)))

namespace hs {

namespace {

constexpr int LAT_THREADS = 256;
constexpr int LAT_DL = 512;
constexpr int LAT_DR = 64;
constexpr int LAT_DK = LAT_DL + LAT_DR;            // 576
constexpr int LAT_REC = LAT_DK * 2;                // 1152 bytes
constexpr int LAT_TILE = 32;                       // rows per tile
constexpr int LAT_BLOCKS = LAT_REC / 32;           // 36 blocks (= d-steps of 16)
constexpr int LAT_TILE_BYTES = LAT_BLOCKS * 1024;  // 36 KB
constexpr int LAT_LDS_BUF = 4 * LAT_TILE_BYTES;     // step buffers: 144 KB
constexpr int LAT_KPF = 6;                         // K operands read ahead
constexpr int LAT_VPF = 4;                         // V^T operands read ahead
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LAT_LAZY_LOG2 = 8.f;               // reference-max slack, log2 units
// Split partials of at most this many bytes per launch are written with
// streaming (nontemporal) stores: the kernel then ends without writing back
// that many dirty L2 lines, and the combine reads them as fast from memory.
constexpr size_t LAT_STREAM_PARTIAL_BYTES = 16u << 20;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Tile layout (36 KB): the latent part (1 KB) of tile row r at r * 1024, its
// 16-byte chunk c at position c ^ lat_sw(r); the rope part (128 bytes) of row
// r at 32768 + 128 r, its chunk c at position c ^ rope_sw(r).
__device__ __forceinline__ int lat_sw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int rope_sw(int r) { return (r >> 1) & 7; }
constexpr int LAT_ROPE_OFF = 32 * 1024;

// One 16-byte global_load_lds per lane: the lane's 16 bytes at src land at
// LDS byte address lds + 16 * lane (lds wave-uniform, in M0). Written as
// inline assembly so that the compiler does not track it: its own wait
// insertion would otherwise wait for every LDS load in flight (the next
// pair's too) before each LDS read of the pair being computed. Waits for
// these loads are explicit (wait_vmcnt). The instruction has no output
// register; its address registers are read at issue; M0 is set in the same
// statement and declared clobbered (nothing else in this kernel keeps a value
// in M0). Loads the compiler does not know of can only make its own vmcnt
// waits stricter: the counter retires in issue order.
// (The compiler warns that M0 is a reserved register; these kernels use M0
// nowhere else, which the generated code shows.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const HS_GLOBAL uint8_t *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"((uint64_t)(uintptr_t)src), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N vector-memory operations of this wave are in flight
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// o *= a for accumulators that stay in the accumulation registers: each is
// moved out, scaled and moved back in one statement, so the compiler never
// keeps a second copy of the accumulators in ordinary registers (it would
// otherwise do so around the loop that these multiplies sit in). Used only
// on the rare moves of the reference maximum, where no MFMA is in flight
// (their results were read since); the leading and trailing wait states
// cover the MFMA-to-move and move-to-MFMA distances regardless.
template <int NVT>
__device__ __forceinline__ void scale_acc(floatx16 (&o)[NVT], float a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float t;
      asm volatile(
          "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
          : "+a"(o[vt][e]), "=&v"(t)
          : "v"(a));
    }
  }
  asm volatile("s_nop 7");
}

// Grid: n8 * HS * S workgroups in XCD-aware order (the HS * S workgroups of a
// unit get block ids equal mod 8, so they run on one XCD and share its L2 for
// the unit's rows); workgroup (u, head group hh, split sp) covers heads
// [32 NHG hh, 32 NHG (hh + 1)) of unit u (those below Hq) over selection
// entries [sp * chunk, min(k, (sp + 1) * chunk)).
template <int NHG, bool STREAM>
__global__ __launch_bounds__(LAT_THREADS, 1) void hs_k_attn_latent(
    const UnitDesc *__restrict__ units, const uint16_t *__restrict__ q_all,
    const int32_t *__restrict__ slots_all, int n_units, int k, int Hq, float scale_log2, int S,
    int HS, int chunk, uint16_t *__restrict__ ws_o, float *__restrict__ ws_ml,
    float *__restrict__ out) {
  constexpr int NVT = LAT_DL / 32 / 2;            // value tiles of 32 per wave
  constexpr int NST = 3 - NHG;                     // tiles per step
  constexpr int NBUF = NHG == 2 ? 3 : 2;           // step buffers
  constexpr int DEPTH = NBUF - 1;                  // steps copied ahead
  constexpr int STEP_BYTES = NST * LAT_TILE_BYTES;
  constexpr int CPS = 9 * NST;                     // copies per wave per step
  static_assert(NBUF * STEP_BYTES <= LAT_LDS_BUF, "step buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t s_buf[LAT_LDS_BUF];
  __shared__ int s_ids[LAT_MAX_CHUNK];
  __shared__ floatx2 s_ml[4][32];  // per wave: (m, l) of its 32 heads
  __shared__ int s_bad;

  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int j8 = b >> 3;
  const int sp = j8 % S;
  const int hh = (j8 / S) % HS;
  const int u = (j8 / (S * HS)) * 8 + xcd;
  if (u >= n_units) return;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int hg = NHG == 2 ? (w & 1) : 0;  // head group of 32 within the workgroup
  const int st = NHG == 2 ? 0 : (w & 1);  // tile within a step
  const int vh = w >> 1;                  // value half
  const int h0 = 32 * NHG * hh;           // the workgroup's first head
  const int head = h0 + 32 * hg + (lane & 31);  // the lane's column
  const bool head_ok = head < Hq;
  const int half = lane >> 5;

  const UnitG d = unit_g(units[u]);
  const int B = d.B;
  const int i_begin = sp * chunk;
  const int n_rows = __builtin_amdgcn_readfirstlane(min(k, i_begin + chunk) - i_begin);
  const int n_tiles = __builtin_amdgcn_readfirstlane((n_rows + LAT_TILE - 1) / LAT_TILE);
  const int n_steps = __builtin_amdgcn_readfirstlane((n_tiles + NST - 1) / NST);
  const HS_GLOBAL int32_t *slots = glb(slots_all) + (size_t)u * k;
  const uint32_t lds0 = (uint32_t)(uintptr_t)&s_buf[0];
  auto step_buf = [&](int i) { return (i % NBUF) * STEP_BYTES; };

  // ---- row copies. Wave w copies, of each 32-row tile, the latent parts of
  // rows w, w + 4, ..., w + 28 (one instruction per row: the 64 lanes read
  // the row's 1 KB, 16 bytes each, the swizzle only permuting within it)
  // and the rope parts of rows 8w .. 8w + 7 (one instruction, 128 bytes from
  // each of 8 rows): 9 global_load_lds per wave per tile. The queries of the
  // workgroup's heads are copied the same way (a head's 1152 bytes are laid
  // out as a row), into tiles of 32 heads.
  int lofs[4];  // lane part of a latent copy's source, by (row >> 2) & 3
#pragma unroll
  for (int m = 0; m < 4; ++m) lofs[m] = 16 * (lane ^ (4 * w + m));
  const int rope_row = 8 * w + (lane >> 3);
  const int rofs_src = LAT_DL * 2 + 16 * ((lane & 7) ^ rope_sw(rope_row));
  // copy m (0..8) of a tile whose row r starts at base(r) (wave-uniform for
  // the latent copies; per lane, row rope_row, for the rope copy)
  auto copy_part = [&](int m, const HS_GLOBAL uint8_t *lat_src, const HS_GLOBAL uint8_t *rope_src,
                       uint32_t tile_dst) {
    if (m < 8)
      lds_dma16(lat_src + lofs[m & 3], tile_dst + 1024 * (w + 4 * m));
    else
      lds_dma16(rope_src + rofs_src, tile_dst + LAT_ROPE_OFF + 1024 * w);
  };
  // the slot ids a wave's copies of step i need: lanes 8t .. 8t + 7 hold
  // those of tile t's rows w + 4 (lane & 7); rope[t] that of row rope_row
  struct CopySrc {
    int lat;
    int rope[NST];
  };
  auto copy_ids = [&](int i) {
    CopySrc c;
    c.lat = s_ids[(NST * i + min((lane >> 3) & 1, NST - 1)) * LAT_TILE + w + 4 * (lane & 7)];
#pragma unroll
    for (int t = 0; t < NST; ++t) c.rope[t] = s_ids[(NST * i + t) * LAT_TILE + rope_row];
    return c;
  };
  // copy m (0 .. CPS - 1) of step i
  const HS_GLOBAL uint8_t *rows = d.rows;
  auto copy_one = [&](const CopySrc &c, int i, int m) {
    const int t = m / 9, mm = m % 9;
    const int slot = __builtin_amdgcn_readlane(c.lat, 8 * t + min(mm, 7));
    copy_part(mm, rows + (size_t)slot * LAT_REC, rows + (size_t)c.rope[t] * LAT_REC,
              lds0 + step_buf(i) + t * LAT_TILE_BYTES);
  };

  // ---- prologue, in two memory round trips. First the loads the compiler
  // waits for: the unit's descriptor and every slot id of the split (a wait
  // for them issued after the row copies would wait for the copies too, the
  // counter retiring in issue order). Then the copies of the queries (into
  // the buffer of step 1, or of steps 1 and 2) and of step 0's rows, back
  // to back; the queries land first and are read while step 0's rows are
  // still arriving.
  if (tid == 0) s_bad = 0;
  // the split's slot ids in whole steps (entries past the split repeat its
  // last one: those rows are loaded and masked)
  const int n_ids = n_steps * NST * LAT_TILE;
  constexpr int IDS_PT = LAT_MAX_CHUNK / LAT_THREADS;
  int ids[IDS_PT];
#pragma unroll
  for (int j = 0; j < IDS_PT; ++j) {
    const int i = tid + j * LAT_THREADS;
    ids[j] = i < n_ids ? slots[i_begin + min(i, n_rows - 1)] : 0;
  }
  // step 0's copy ids, and with two tiles per step step 1's, straight from
  // global memory (step 1's second tile goes to the second half of the
  // buffer whose first half takes the queries, so it is copied now)
  auto load_ids = [&](int i) {
    CopySrc c;
    c.lat = slots[i_begin + min((NST * i + min((lane >> 3) & 1, NST - 1)) * LAT_TILE + w +
                                    4 * (lane & 7),
                                n_rows - 1)];
#pragma unroll
    for (int t = 0; t < NST; ++t)
      c.rope[t] = slots[i_begin + min((NST * i + t) * LAT_TILE + rope_row, n_rows - 1)];
    return c;
  };
  const bool early1 = NHG == 1 && n_steps > 1;  // wave-uniform
  CopySrc c0, c1;
  if (n_steps > 0) c0 = load_ids(0);
  if (early1) c1 = load_ids(1);
  // an invalid slot is flagged and replaced by slot 0 (the unit's output
  // becomes NaN)
  bool bad = false;
  auto checked = [&](int sl) {
    if ((unsigned)sl >= (unsigned)B) {
      bad = true;
      sl = 0;
    }
    return sl;
  };
#pragma unroll
  for (int j = 0; j < IDS_PT; ++j) {
    const int i = tid + j * LAT_THREADS;
    if (i < n_ids) s_ids[i] = checked(ids[j]);
  }
  const uint32_t q_dst = lds0 + STEP_BYTES;
  {
    const HS_GLOBAL uint8_t *qb0 = (const HS_GLOBAL uint8_t *)glb(q_all) + (size_t)u * Hq * LAT_REC;
    const int hmax = Hq - 1;
#pragma unroll
    for (int g = 0; g < NHG; ++g)
#pragma unroll
      for (int m = 0; m < 9; ++m)
        copy_part(m, qb0 + (size_t)min(h0 + 32 * g + w + 4 * m, hmax) * LAT_REC,
                  qb0 + (size_t)min(h0 + 32 * g + rope_row, hmax) * LAT_REC,
                  q_dst + g * LAT_TILE_BYTES);
  }
  if (n_steps > 0) {
    c0.lat = checked(c0.lat);
#pragma unroll
    for (int t = 0; t < NST; ++t) c0.rope[t] = checked(c0.rope[t]);
#pragma unroll
    for (int m = 0; m < CPS; ++m) copy_one(c0, 0, m);
  }
  if (early1) {
    c1.lat = checked(c1.lat);
    c1.rope[NST - 1] = checked(c1.rope[NST - 1]);
#pragma unroll
    for (int m = 9; m < CPS; ++m) copy_one(c1, 1, m);
  }
  lds_barrier();  // s_bad's initial value is visible to every wave
  if (bad) s_bad = 1;
  // this wave's query copies have landed (the later ones may still be in
  // flight), then every wave's have
  if (early1)
    wait_vmcnt<CPS + 9>();
  else if (n_steps > 0)
    wait_vmcnt<CPS>();
  else
    wait_vmcnt<0>();
  lds_barrier();

  // K read of d-step ds from a tile: lane (row r = lane & 31, chunk 2 ds +
  // half). Latent d-steps: tile + 256 (ds >> 3) + kofs[ds & 7]; rope d-steps
  // 32 + j: tile + rofs[j]
  const int kr_row = lane & 31;
  int kofs[8], rofs[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) kofs[j] = 1024 * kr_row + 16 * ((2 * j + half) ^ lat_sw(kr_row));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    rofs[j] = LAT_ROPE_OFF + 128 * kr_row + 16 * ((2 * j + half) ^ rope_sw(kr_row));
  auto kread = [&](const HS_LDS uint8_t *tl, int ds) {
    const int off = ds < 32 ? 256 * (ds >> 3) + kofs[ds & 7] : rofs[ds - 32];
    return *(const HS_LDS bf16x8 *)(tl + off);
  };

  // Q^T of the wave's 32 heads (the B operand: lane (head, d 16 ds + 8 half
  // .. + 7)), read from the query tile like a K operand; padding heads
  // (Hq = 16) are zero
  bf16x8 qb[LAT_BLOCKS];
  {
    const HS_LDS uint8_t *qt = (const HS_LDS uint8_t *)&s_buf[q_dst - lds0 + hg * LAT_TILE_BYTES];
    const uint32_t keep = head_ok ? ~0u : 0u;
#pragma unroll
    for (int ds = 0; ds < LAT_BLOCKS; ++ds)
      qb[ds] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(v4u, kread(qt, ds)) & keep);
  }
  // step 0's rows have landed (step 1's second tile may still be in
  // flight), and every wave's; the query tiles' buffers are free; the slot
  // ids and s_bad are visible
  if (early1)
    wait_vmcnt<9>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  if (DEPTH > 1 && n_steps > 1) {
    const CopySrc c1 = copy_ids(1);
#pragma unroll
    for (int m = 0; m < CPS; ++m) copy_one(c1, 1, m);
  }

  // transpose read q (0/1) of value tile vt, k-block kb: 16-lane group g
  // reads rows 16 kb + 8 q + 4 (g >> 1) + 0..3, values 32 vt + 16 (g & 1) +
  // 0..15 (lane j: row + j / 4, values 4 (j % 4) .. + 3); lane j of the group
  // receives value 32 vt + 16 (g & 1) + j of those 4 rows. Address: tile +
  // 16384 kb + 256 (vt >> 2) + tr_off[q][vt & 3].
  const int g = lane >> 4, jj = lane & 15;
  int tr_off[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rb = 8 * q + 4 * (g >> 1) + (jj >> 2);  // row within its k-block
    const int a = 2 * (g & 1) + ((jj & 3) >> 1);     // chunk within the value tile
#pragma unroll
    for (int v3 = 0; v3 < 4; ++v3) {
      const int pos = 4 * ((v3 ^ (rb & 3)) & 3) + (a ^ ((rb >> 2) & 3));  // = chunk ^ lat_sw
      tr_off[q][v3] = 1024 * rb + 16 * pos + 8 * (jj & 1);
    }
  }
  // V^T operand m (value tile m / 2 of the wave's half, k-block m % 2)
  auto vread = [&](const HS_LDS uint8_t *tl, int m) {
    const int vt = vh * NVT + (m >> 1);
    const HS_LDS uint8_t *vb = tl + 16384 * (m & 1) + 256 * (vt >> 2);
    const short4v lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS short4v *)(vb + tr_off[0][vt & 3]));
    const short4v hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS short4v *)(vb + tr_off[1][vt & 3]));
    return __builtin_bit_cast(bf16x8,
                              short8v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  floatx16 o[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[vt][e] = 0.f;
  float m_run = NEG_INF;  // reference maximum of the lane's head (log2 units)
  float l_run = 0.f;      // this lane's share of the head's sum

  // LDS operand reads run a few MFMAs ahead of their use (register rings of
  // LAT_KPF K operands and LAT_VPF V^T operands), so the MFMA pipe does not
  // wait out an LDS round trip per instruction
  bf16x8 vring[LAT_VPF];
  // S^T of the wave's tile: lane (head column, slots 8 (e / 4) + 4 half + e %
  // 4 of the tile), slots past the split at -inf. The copies of step ci go
  // out between the MFMAs (one per 36 / CPS d-steps), where their issue cost
  // overlaps the matrix work; the first V^T operands are read after the last
  // K operand, so they arrive during the softmax.
  auto scores = [&](const HS_LDS uint8_t *tl, int tile, bool copy, const CopySrc &cs, int ci) {
    bf16x8 kring[LAT_KPF];
#pragma unroll
    for (int j = 0; j < LAT_KPF; ++j) kring[j] = kread(tl, j);
    floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < LAT_BLOCKS; ++ds) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kring[ds % LAT_KPF], qb[ds], acc, 0, 0, 0);
      if (ds + LAT_KPF < LAT_BLOCKS)
        kring[ds % LAT_KPF] = kread(tl, ds + LAT_KPF);
      else if (ds + LAT_KPF - LAT_BLOCKS < LAT_VPF)
        vring[ds + LAT_KPF - LAT_BLOCKS] = vread(tl, ds + LAT_KPF - LAT_BLOCKS);
      constexpr int every = LAT_BLOCKS / CPS;
      // (step 1's second tile went out in the prologue)
      if (copy && ds % every == 0 && !(NHG == 1 && ci == 1 && ds / every >= 9))
        copy_one(cs, ci, ds / every);
      // keep this order: the scheduler would otherwise pull the reads next
      // to their MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
    const int valid = __builtin_amdgcn_readfirstlane(n_rows - LAT_TILE * tile);  // in the split
    if (valid < LAT_TILE) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[e] = 8 * (e >> 2) + 4 * half + (e & 3) < valid ? acc[e] : NEG_INF;
    }
    return acc;
  };
  // P = 2^(s scale_log2 - m_run) rounded to bf16, the lane's share of l, and
  // O^T += V^T P^T over the wave's value tiles
  auto accumulate = [&](const HS_LDS uint8_t *tl, const floatx16 &sc) {
    // a wave that has seen only masked slots keeps m_run = -inf; its P is 0
    const float m_ref = fmaxf(m_run, -__FLT_MAX__);
    uint32_t pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pw[e] = pack_bf16(exp2_fast(__builtin_fmaf(sc[2 * e], scale_log2, -m_ref)),
                        exp2_fast(__builtin_fmaf(sc[2 * e + 1], scale_log2, -m_ref)));
      l_run += __uint_as_float(pw[e] << 16) + __uint_as_float(pw[e] & 0xFFFF0000u);
    }
    // P^T of k-block kb: the lane's scores 8 kb .. 8 kb + 7 (slots 16 kb +
    // 8 (e / 4) + 4 half + e % 4)
    const bf16x8 pB0 = __builtin_bit_cast(bf16x8, v4u{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 pB1 = __builtin_bit_cast(bf16x8, v4u{pw[4], pw[5], pw[6], pw[7]});
#pragma unroll
    for (int m = 0; m < 2 * NVT; ++m) {
      o[m >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vring[m % LAT_VPF], (m & 1) ? pB1 : pB0,
                                                          o[m >> 1], 0, 0, 0);
      if (m + LAT_VPF < 2 * NVT) vring[m % LAT_VPF] = vread(tl, m + LAT_VPF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The accumulators are touched only by MFMAs and, on the rare moves of the
  // reference maximum, by scale_acc, so they stay in their registers across
  // the loop. Every wave passes the same barriers; the step index and every
  // branch are wave-uniform (readfirstlane says so; otherwise the loop
  // compiles to a divergent one under exec masks).
  for (int i = 0; i < n_steps; ++i) {
    // this wave's copies of step i have landed (those of the steps after it
    // may still be in flight), then every wave's have, and every wave is done
    // with step i - 1, whose buffer step i + DEPTH reuses
    if (DEPTH > 1 && i + 1 < n_steps)
      wait_vmcnt<(DEPTH - 1) * CPS>();
    else if (early1 && i == 0)
      wait_vmcnt<9>();  // step 1's second tile, copied in the prologue
    else
      wait_vmcnt<0>();
    __syncthreads();
    const int ci = i + DEPTH;  // the step whose copies go out with QK^T
    const bool copy = ci < n_steps;
    const CopySrc cs = copy_ids(copy ? ci : i);
    // a tile past the split (an odd last tile of a two-tile step) has every
    // score masked and adds zeros (a skip would give the accumulators a
    // second path through the loop, which the compiler serves with copies)
    const int tile = __builtin_amdgcn_readfirstlane(NST * i + st);
    const HS_LDS uint8_t *tl =
        (const HS_LDS uint8_t *)&s_buf[step_buf(i) + st * LAT_TILE_BYTES];
    const floatx16 sc = scores(tl, tile, copy, cs, ci);
    float x = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) x = fmaxf(x, sc[e]);
    x *= scale_log2;
    if (__builtin_amdgcn_readfirstlane(__any(x > m_run + LAT_LAZY_LOG2))) {
      // max(x) s = max(x s) for s > 0: the decision is the head maximum's
      const float mx = fmaxf(x, __shfl_xor(x, 32, 64));
      const float m_new = mx > m_run + LAT_LAZY_LOG2 ? mx : m_run;
      if (__builtin_amdgcn_readfirstlane(__any(m_run != NEG_INF && m_new != m_run))) {
        const float alpha = exp2_fast(m_run - m_new);  // 1 where unchanged
        l_run *= alpha;
        scale_acc<NVT>(o, alpha);
      }
      m_run = m_new;
    }
    accumulate(tl, sc);
  }

  // ---- outputs, staged through LDS so that every store writes 1 KB of a
  // row: each wave puts its accumulators (32 heads x 256 values) and its
  // heads' (m, l) into its own 32 KB region (every copy has landed and been
  // read, so the step buffers are free), then each wave stores row halves
  // (head, value half) from LDS. With two tiles per step (NHG = 1) the two
  // streams' regions of a value half merge exactly on the way out.
  // Region layout: head row r at r * 1024, its 16-byte chunk q at position
  // q ^ (r & 15) (the writes, one head per lane, and the reads, one row per
  // instruction, are then free of bank conflicts).
  l_run += __shfl_xor(l_run, 32, 64);
  wait_vmcnt<0>();
  __syncthreads();
  const bool any_bad = s_bad != 0;
  if (any_bad && tid == 0) set_error(d.ctl, HS_ERR_SLOT);
  {
    uint8_t *reg = &s_buf[w * 32768];
    const int r = lane & 31;
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int q = 8 * vt + 2 * c + half;
        *(floatx4 *)(reg + 1024 * r + 16 * (q ^ (r & 15))) =
            floatx4{o[vt][4 * c], o[vt][4 * c + 1], o[vt][4 * c + 2], o[vt][4 * c + 3]};
      }
    if (lane < 32) s_ml[w][lane] = floatx2{m_run, l_run};
  }
  __syncthreads();
  // (m, l) of every head (for the split-k combine, or 1 / l for the output):
  // lanes 0..31 of waves 0 (and 1 with NHG = 2) take heads h0 + 32 w + lane
  if (w < NHG && lane < 32 && h0 + 32 * w + lane < Hq) {
    const floatx2 a = s_ml[w][lane];
    float M = a[0], L = a[1];
    if (NHG == 1) {
      const floatx2 c = s_ml[1][lane];
      M = fmaxf(a[0], c[0]);
      L = (a[0] == NEG_INF ? 0.f : a[1] * exp2_fast(a[0] - M)) +
          (c[0] == NEG_INF ? 0.f : c[1] * exp2_fast(c[0] - M));
    }
    const size_t row = (size_t)u * Hq + h0 + 32 * w + lane;
    if (S > 1) {
      ((HS_GLOBAL uint32_t *)ws_ml)[(row * S + sp) * 2] = nan_bits_if(any_bad, M);
      ws_ml[(row * S + sp) * 2 + 1] = L;
    } else {
      s_ml[w][lane][1] = L;  // the output's divisor (only its own lane reads it back)
    }
  }
  __syncthreads();
  // wave w stores 32 (NHG = 2: its region) or 16 (NHG = 1) row halves, all
  // read from LDS before any is stored
  constexpr int PIECES = NHG == 2 ? 32 : 16;
  const int pvh = w >> 1;
  const int ra = NHG == 2 ? w : 2 * pvh;  // (the first stream's) region
  auto piece = [&](int pc) {
    const int r = NHG == 2 ? pc : 16 * (w & 1) + pc;
    floatx4 v = *(const floatx4 *)&s_buf[ra * 32768 + 1024 * r + 16 * (lane ^ (r & 15))];
    if (NHG == 1) {
      const floatx2 m0 = s_ml[ra][r], m1 = s_ml[ra + 1][r];
      const floatx4 v1 =
          *(const floatx4 *)&s_buf[(ra + 1) * 32768 + 1024 * r + 16 * (lane ^ (r & 15))];
      const float M = fmaxf(m0[0], m1[0]);
      // a stream without tiles has m = -inf: its factor is 0
      v = v * (m0[0] == NEG_INF ? 0.f : exp2_fast(m0[0] - M)) +
          v1 * (m1[0] == NEG_INF ? 0.f : exp2_fast(m1[0] - M));
    }
    return v;
  };
  auto piece_row = [&](int pc) {
    const int r = NHG == 2 ? pc : 16 * (w & 1) + pc;
    return h0 + (NHG == 2 ? 32 * (w & 1) : 0) + r;  // the head
  };
  const int v0 = 256 * pvh + 4 * lane;
  // in batches of 16 pieces: every LDS read of a batch, then its stores (the
  // scheduler would otherwise pair each store with its read and wait out an
  // LDS round trip per store)
  constexpr int BATCH = 16;
#pragma unroll
  for (int p0 = 0; p0 < PIECES; p0 += BATCH) {
    floatx4 vb[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) vb[j] = piece(p0 + j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int ph = piece_row(p0 + j);
      if (NHG == 1 && ph >= Hq) continue;
      if (S == 1) {
        const float L = s_ml[NHG == 2 ? (w & 1) : 0][ph - h0 - (NHG == 2 ? 32 * (w & 1) : 0)][1];
        const floatx4 rr = vb[j] * (1.f / L);
        const v4u bits = {nan_bits_if(any_bad, rr[0]), nan_bits_if(any_bad, rr[1]),
                          nan_bits_if(any_bad, rr[2]), nan_bits_if(any_bad, rr[3])};
        *(HS_GLOBAL v4u *)(out + ((size_t)u * Hq + ph) * LAT_DL + v0) = bits;
      } else {
        // the split's partial, rounded to bf16 (nearest even): 512 bytes per
        // instruction
        HS_GLOBAL v2u *dst =
            (HS_GLOBAL v2u *)(glb(ws_o) + (((size_t)u * Hq + ph) * S + sp) * LAT_DL + v0);
        const v2u bits = {pack_bf16(vb[j][0], vb[j][1]), pack_bf16(vb[j][2], vb[j][3])};
        if (STREAM)
          __builtin_nontemporal_store(bits, dst);
        else
          *dst = bits;
      }
    }
  }
}

template <int NHG, bool STREAM>
hipError_t launch_latent_t(const AttnLatentArgs &a, hipStream_t stream) {
  const int HS = (a.Hq + 32 * NHG - 1) / (32 * NHG);
  if (a.chunk > LAT_MAX_CHUNK || a.chunk % (2 * LAT_TILE)) return hipErrorInvalidValue;
  const int grid = ((a.n_units + 7) / 8) * 8 * a.splits * HS;
  return launch_k(HS_TRACE_ATTN, hs_k_attn_latent<NHG, STREAM>, dim3(grid), dim3(LAT_THREADS), 0,
                  stream, a.units, a.q, a.slots, a.n_units, a.k, a.Hq, a.scale_log2, a.splits, HS,
                  a.chunk, a.ws_o, a.ws_ml, a.out);
}

}  // namespace

hipError_t launch_attn_latent(const AttnLatentArgs &a, hipStream_t stream) {
  const bool stream_partials = a.splits > 1 && (size_t)a.n_units * a.Hq * a.splits * LAT_DL *
                                                      sizeof(uint16_t) <= LAT_STREAM_PARTIAL_BYTES;
  const hipError_t e =
      a.hpw == 64 ? (stream_partials ? launch_latent_t<2, true>(a, stream)
                                   : launch_latent_t<2, false>(a, stream))
                  : (stream_partials ? launch_latent_t<1, true>(a, stream)
                                   : launch_latent_t<1, false>(a, stream));
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.ws_o, 1, a.ws_ml, a.n_units * a.Hq, a.splits, LAT_DL, a.out, stream);
}

}  // namespace hs
