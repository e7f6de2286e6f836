// Segment-batch attention (restore prefill).
//
// "Cache Engineering for Agents" review, "single-prefill restore with
// segment-batch attention" (§4.2, App. A.1.1, Fig. 10): queries are cut at every
// drop/repos point into segments; each segment attends causally to its own tokens
// and to the active cache that earlier segments left, so a dropped entry stays
// visible to the segments that used it and is hidden from later ones.  With the
// plan's tables this is: query i sees key j iff j <= i < tok_drop[j] (version rows
// of the query's repos stretch are all earlier tokens), with keys at the positions
// they hold in that stretch.
//
// bf16 kernels (gfx950, wave64, MFMA 32x32x16 bf16):
//   * one workgroup = one work item (stretch, 64-token q-tile) x one kv head; its
//     GROUP waves are the GROUP query heads sharing that kv head, so each K/V tile
//     staged in LDS feeds GROUP x 64 query rows;
//   * per key tile of 64: S^T = K Q'^T (keys on MFMA rows, queries on columns, Q'
//     = Q scaled by scale*log2 e), so a lane holds 32 scores of one query column;
//   * P^T stays in registers in exactly the layout the second MFMA wants as its B
//     operand; O^T = V^T P^T takes V^T from the row-major V tile through the
//     transposing LDS read ds_read_b64_tr_b16 (lane i of a 16-lane group gets
//     element i of 4 consecutive rows);
//   * the plan's tile list skips EMPTY tiles, FULL tiles run unmasked, PARTIAL
//     tiles build the mask from per-key (token, drop) pairs staged in LDS;
//   * the ping-pong kernel keeps Q' in registers for the whole tile loop and reads
//     each PV quarter's V^T fragments one quarter ahead (the registers that frees
//     pay for Q'), so its QK phase issues only MFMAs; the variant without version
//     buffers keeps Q' in per-wave LDS rows, read a d slice ahead, and spends those
//     registers on rotating its version rows;
//   * K/V tiles reach LDS by direct global -> LDS copies (global_load_lds, 16
//     bytes a lane) into unpadded rows whose 16-byte chunks are XOR-swizzled by
//     row, so the K row reads and the transposing V reads stay free of bank
//     conflicts; without version buffers, a version tile's rows are gathered from
//     their source tokens the same way and each wave turns its own key rows in
//     place in LDS, between the QK MFMAs;
//   * blockIdx -> (item, kv head) puts consecutive workgroups on different kv heads,
//     so with 8 kv heads each XCD's L2 streams a single head's K/V;
//   * 8 query heads per kv head (seg_attn_bf16_pp); 4, 2 or 1 with a plan whose
//     query tiles hold 64 * 8 / group tokens, each wave taking one 64-token part
//     of the tile for one query head; or 4 with an even number of kv heads and
//     64-token query tiles (two kv heads per workgroup): two wave groups
//     ping-pong between softmax and MFMA phases; the fast pass keeps the exponent
//     offset at 0 and takes the column sums from the matrix cores, with one range
//     check per work item and a redo through the rescaling softmax when it fails;
//   * otherwise, 1, 2 or 4 query heads per kv head with 64-token query tiles
//     (seg_attn_bf16<GROUP>): one wave per query
//     head, one synchronously staged tile buffer, the rescaling softmax (lazily
//     moved exponent offset, bf16 dot2 row sums, per-tile range check); several
//     workgroups share a CU, so one's MFMA work overlaps another's softmax and loads;
//   * queries arrive either rotated or raw; raw ones are rotated to their append
//     positions (tok_pos) in fp32 as they are loaded, before the scale and the one
//     bf16 rounding (review §3.3: a vector at position p is the raw vector rotated
//     pair by pair by p * theta_i);
//   * the ping-pong kernel writes its output tile through the wave's LDS rows as
//     whole 128-byte rows with streaming stores, so no dirty output lines are left
//     in the last-level cache for the next kernel to write back.
//
// fp32 kernel (seg_attn_f32): one thread per (query token, head), keys one at a
// time with an exact online softmax; for small problems and fp32 checks.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "internal.h"
#include "rope_angle.h"

namespace akv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

constexpr int D = 64;    // head dim
constexpr int BK = 64;   // keys per tile (= 2 MFMA row blocks)
constexpr int KP = 72;   // K tile row pitch (bf16): 144 B, conflict-free 16-B row reads
constexpr int VP = 80;   // V tile row pitch (bf16): 160 B, conflict-free transposing reads
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt) but lets global loads into registers stay in flight across it (a
// __syncthreads release fence would drain them).  The memory clobber keeps the
// compiler from moving LDS accesses across the barrier, the scheduling fences
// keep it from moving register-only work (exp, MFMA) from one phase to the other.
// The wait is issued through the builtin so the compiler's wait-count tracking
// knows the LDS and scalar-memory counters are drained here (a wait hidden in
// inline asm made it re-wait for reads issued after the barrier).
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained
constexpr int kWaitVm0 = 0x0F70;    // s_waitcnt vmcnt(0), expcnt and lgkmcnt unconstrained
constexpr int kWaitVm2 = 0x0F72;    // s_waitcnt vmcnt(2), expcnt and lgkmcnt unconstrained
constexpr int kWaitVm4 = 0x0F74;    // s_waitcnt vmcnt(4), expcnt and lgkmcnt unconstrained
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 cat4(s16x4 a, s16x4 b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}


struct TileSrc {
  const uint16_t* k;
  const uint16_t* v;
  int row0, nrows;
  bool ver;
};

__device__ __forceinline__ TileSrc tile_src(int ent, int nvt, int voff, int r, int tb, int te,
                                            const uint16_t* k, const uint16_t* v,
                                            const uint16_t* kver, const uint16_t* vver) {
  const int kt = ent >> 2;
  TileSrc ts;
  ts.ver = kt < nvt;
  ts.row0 = ts.ver ? voff + kt * BK : tb + (kt - nvt) * BK;
  ts.nrows = ts.ver ? min(BK, r - kt * BK) : min(BK, te - ts.row0);
  ts.k = ts.ver ? kver : k;
  ts.v = ts.ver ? vver : v;
  return ts;
}

// Per-wave state: 64 query tokens of one head.
struct WaveState {
  bf16x8 qf[2][4];        // Q'^T B operand: qf[qb][ds] = Q'[q0 + 32qb + lq][h][16ds + 8lg .. +8]
  f32x16 o[2][2];         // O^T accumulators [qb][db]: d = 32db + 8(i/4) + 4lg + i%4, query 32qb + lq
  f32x16 s[2][2];         // S^T [kb][qb]: key 32kb + 8(i/4) + 4lg + i%4, query 32qb + lq
  bf16x8 pb[2][2][2];     // P^T B operand [kb][qb][half]
  float ms[2], lrun[2];   // exponent offset (log2 units) and running sum per query column
  bool shifted;           // some column of the wave has a non-zero offset
};

// Operand fragments of one tile, read from LDS ahead of the MFMAs that use them.
struct KFrag { bf16x8 a[4][2]; };        // K rows: a[ds][kb] = K[32kb + lq][16ds + 8lg .. +8]
struct VFrag { bf16x8 a[2][2][2]; };     // V^T: a[kb][hf][db] (rows d, columns keys of the half)

// 16 bytes of row `row` at column 16ds + 8lg of a K-pitched LDS tile (K or Q').
__device__ __forceinline__ bf16x8 row_frag(const uint16_t* base, int row, int ds, int lg) {
  return *(const bf16x8*)(base + row * KP + ds * 16 + lg * 8);
}

// Swizzled tile layout (SW): rows of 64 bf16 with no padding, as the direct
// global -> LDS copies write them (64 lanes x 16 bytes, contiguous).  16-byte
// chunk c of K row r sits at chunk c ^ swz_k(r), of V row r at c ^ swz_v(r).  A K
// fragment read (lanes 0-31 read rows r0..r0+31 at one chunk) then spreads every 8
// consecutive rows, and every 16 rows of equal parity, over all eight chunks; a
// transposing V read (16 lanes: 4 consecutive rows x 32 bytes) puts its four rows
// on four different chunk pairs, and 32 lanes put rows of equal parity on
// different halves of the row.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }
template <bool SW>
__device__ __forceinline__ bf16x8 k_frag(const uint16_t* lkb, int row, int ds, int lg) {
  if (SW) return *(const bf16x8*)(lkb + row * D + (((2 * ds + lg) ^ swz_k(row)) << 3));
  return row_frag(lkb, row, ds, lg);
}

// Q' operand of query block qb, d slice ds: from registers, or (QL) from the
// wave's Q' rows in LDS.
template <bool QL>
__device__ __forceinline__ bf16x8 q_frag(const WaveState& w, const uint16_t* lqw, int qb, int ds, int lq, int lg) {
  if (QL) return row_frag(lqw, qb * 32 + lq, ds, lg);
  return w.qf[qb][ds];
}

// S^T = K Q'^T for one 64-key tile (16 MFMAs), operands read as they are used.
// Q' is Q scaled by scale*log2(e), so the scores are already in log2 units.
template <bool QL, bool SW = false>
__device__ __forceinline__ void tile_qk(WaveState& w, const uint16_t* lkb, const uint16_t* lqw, int lq, int lg) {
  const f32x16 zero = {};
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    const bf16x8 b0 = q_frag<QL>(w, lqw, 0, ds, lq, lg), b1 = q_frag<QL>(w, lqw, 1, ds, lq, lg);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = k_frag<SW>(lkb, kb * 32 + lq, ds, lg);
      w.s[kb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, ds ? w.s[kb][0] : zero, 0, 0, 0);
      w.s[kb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, ds ? w.s[kb][1] : zero, 0, 0, 0);
    }
  }
}

// V^T fragments of one tile from the row-major V tile through the transposing LDS
// read (lane i of a 16-lane group gets element i%4 of the 8-byte chunk that lane
// 4k + i/4 addresses, for k = 0..3).  Fragment g = 4kb + 2hf + db, two reads each.
template <bool SW = false>
__device__ __forceinline__ void read_vt_part(VFrag& f, const uint16_t* lvb, int lane, int g) {
  const int G = lane >> 4, i16 = lane & 15;
  const int kb = g >> 2, hf = (g >> 1) & 1, db = g & 1;
  const int key = kb * 32 + 16 * hf + 4 * (G >> 1) + (i16 >> 2);
  const int dc = db * 32 + 16 * (G & 1) + 4 * (i16 & 3);
  // swz_v(key + 8) == swz_v(key)
  const int off = SW ? key * D + (((dc >> 3) ^ swz_v(key)) << 3) + (dc & 7) : key * VP + dc;
  const int pitch = SW ? D : VP;
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lvb + off));
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lvb + off + 8 * pitch));
  f.a[kb][hf][db] = cat4(r0, r1);
}

template <bool SW = false>
__device__ __forceinline__ void read_vt(VFrag& f, const uint16_t* lvb, int lane) {
#pragma unroll
  for (int g = 0; g < 8; ++g) read_vt_part<SW>(f, lvb, lane, g);
}

// No work hooked into an MFMA sequence.
struct NoCopy {
  __device__ __forceinline__ void operator()() const {}
  static constexpr bool kActive = false;
};

// tile_qk with the K fragments already in registers.  SW (direct-copy kernel): Q'
// is held in registers for the whole loop (w.qf) and the V^T fragments are read
// inside PV, so QK issues only MFMAs.  Otherwise the first two Q' slices (qf[0],
// qf[1]) come from PV and the remaining ones are read from LDS two d slices ahead
// of their MFMAs, and after each d slice's MFMAs two of the next tile's V^T
// fragments (vf, from lvb) are read, so those LDS reads issue between MFMAs
// instead of in one block.
template <bool SW>
__device__ __forceinline__ void mfma_qk_lq(WaveState& w, const KFrag& f, const bf16x8 (&qf)[2][2], const uint16_t* lqw,
                                           int lq, int lg, VFrag& vf, const uint16_t* lvb, int lane) {
  const f32x16 zero = {};
  if (SW) {  // Q' in registers; V^T fragments are read inside PV
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          w.s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ds][kb], w.qf[qb][ds], ds ? w.s[kb][qb] : zero,
                                                                0, 0, 0);
    }
    return;
  }
  bf16x8 b[3][2];
  b[0][0] = qf[0][0];
  b[0][1] = qf[0][1];
  b[1][0] = qf[1][0];
  b[1][1] = qf[1][1];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    if (ds + 2 < 4) {
      b[(ds + 2) % 3][0] = row_frag(lqw, lq, ds + 2, lg);
      b[(ds + 2) % 3][1] = row_frag(lqw, 32 + lq, ds + 2, lg);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        w.s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ds][kb], b[ds % 3][qb], ds ? w.s[kb][qb] : zero,
                                                              0, 0, 0);
    read_vt_part<SW>(vf, lvb, lane, 2 * ds);
    read_vt_part<SW>(vf, lvb, lane, 2 * ds + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Bounds on a query column's tile probability sum.  The exponent offset m starts
// at 0, so p = exp2(s - m) is used as is while the sums stay in (2^-40, 2^40]:
// fp32/bf16 keep full relative precision anywhere in that range.  A sum above it
// (a score far above m) or a column with no mass below it (scores far under m)
// moves m to the tile's max and redoes the tile.
constexpr float kSumHi = 1099511627776.0f;        // 2^40
constexpr float kSumLo = 9.094947017729282e-13f;  // 2^-40

// P = exp2(S - m) rounded to bf16 into the PV B operand, and the column's tile
// sum of those rounded values (the weights the PV product uses, so the output is
// normalised by exactly their total), summed with bf16 dot2 against ones.
__device__ __forceinline__ void tile_exp(WaveState& w, int qb, float& tot) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 p;
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = (__bf16)__builtin_amdgcn_exp2f(w.s[kb][qb][8 * hf + j]);
      w.pb[kb][qb][hf] = p;
      asm volatile("" ::"v"(p));  // pack here, not after the range check (fewer live registers)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 pr = {p[2 * j], p[2 * j + 1]};
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
      }
    }
  tot = xhalf_sum(sum);
}

__device__ __forceinline__ float col_max(const WaveState& w, int qb) {
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, w.s[kb][qb][i]);
  return xhalf_max(m);
}

__device__ __forceinline__ bool out_of_range(float tot, float lrun) {
  return !(tot <= kSumHi) || (lrun + tot < kSumLo);
}

// Scores of a tile made ready for exp2: hidden pairs of a PARTIAL tile set to
// -inf, and the column offsets subtracted once any column has moved its offset.
template <bool OFFSETS = true>
__device__ __forceinline__ void prep_scores(WaveState& w, bool partial, const int* mtok, const int* mdrop, int q0,
                                            int lq, int lg) {
  if (partial) {
    asm volatile("");  // keep this rare path behind its branch (not speculated into every tile)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int tok = q0 + qb * 32 + lq;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
          const int mt = mtok[key], md = mdrop[key];
          const bool vis = (mt <= tok) & (tok < md);
          w.s[kb][qb][i] = vis ? w.s[kb][qb][i] : -INFINITY;
        }
    }
  }
  if (OFFSETS && w.shifted) {
    asm volatile("");  // only after a rescale: apply the column offsets
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.s[kb][qb][i] -= w.ms[qb];
  }
}

// Mask (PARTIAL tiles), online softmax in log2 units, P -> bf16 B operand.  The
// scores die as P is formed; the rare path that moves a column's offset
// recomputes them from the tile's K rows (still in LDS at lkb).
template <bool QL, bool SW = false>
__device__ __forceinline__ void tile_softmax(WaveState& w, bool partial, const int* mtok, const int* mdrop,
                                             const uint16_t* lkb, const uint16_t* lqw, int q0, int lq, int lg) {
  prep_scores(w, partial, mtok, mdrop, q0, lq, lg);
  float tot[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) tile_exp(w, qb, tot[qb]);
  const bool bad0 = out_of_range(tot[0], w.lrun[0]), bad1 = out_of_range(tot[1], w.lrun[1]);
  if (__any(bad0 || bad1)) {
    asm volatile("");  // rare: scores far above or below the offset
    tile_qk<QL, SW>(w, lkb, lqw, lq, lg);
    prep_scores(w, partial, mtok, mdrop, q0, lq, lg);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mx = col_max(w, qb);
      const bool on = (qb ? bad1 : bad0) && mx > -INFINITY;
      const float shift = on ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      w.ms[qb] += shift;
      w.lrun[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[qb][db][i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.s[kb][qb][i] -= shift;
      tile_exp(w, qb, tot[qb]);  // unchanged for a column whose offset stays
    }
    w.shifted = __any((w.ms[0] != 0.f) || (w.ms[1] != 0.f));
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) w.lrun[qb] += tot[qb];
}

// Fast-pass softmax: the exponent offset stays 0 and nothing is summed here.
// P = exp2(S) rounded to bf16 (hidden pairs of a PARTIAL tile give 0); the column
// sums come from the matrix cores in the MFMA phase, and the range of the final
// sums is checked once per work item.
__device__ __forceinline__ void tile_softmax_fast(WaveState& w, bool partial, const int* mtok, const int* mdrop,
                                                  int q0, int lq, int lg) {
  prep_scores<false>(w, partial, mtok, mdrop, q0, lq, lg);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 p;
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = (__bf16)__builtin_amdgcn_exp2f(w.s[kb][qb][8 * hf + j]);
        w.pb[kb][qb][hf] = p;
      }
}

// A operand of the column-sum MFMA (16x16x32): row m = lane%16, k = 8(lane/16) + i.
// Element (m, k) is 1 where bit 2 of m equals bit 3 of k.  With a P^T slice of 16
// keys x 32 queries as the B operand (query 32qb + lane%32, keys 8(lane/32) + i,
// read as k = 8(lane/16) + i, column lane%16), result rows 0-3 and 8-11 sum the
// query columns 0-15 and rows 4-7 and 12-15 the columns 16-31 over the 16 keys, so
// every register of lane l holds the sum of query column 32qb + l%32, the column
// that lane owns in the softmax.
__device__ __forceinline__ bf16x8 colsum_selector(int lane) {
  const bool on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
  const __bf16 x = on ? (__bf16)1.0f : (__bf16)0.0f;
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = x;
  return a;
}


// O^T += V^T P^T for one tile (16 MFMAs).
__device__ __forceinline__ void mfma_pv(WaveState& w, const VFrag& f) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          w.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kb][hf][db], w.pb[kb][qb][hf], w.o[qb][db], 0, 0, 0);
}

// mfma_pv with the next tile's K fragments read in between: after the 4 MFMAs of
// each (kb, hf) quarter, whose V^T and P registers then die, the two K fragments
// of one 16-wide d slice are read.  SW: before them, the next quarter's V^T
// fragments of this tile (lvb; the first quarter's were read at the end of the
// softmax phase).  QL (Q' in LDS): after the second and the last quarter, the
// first and the second Q' slice.  The reads' latency hides behind the MFMAs.  With SUMS, each
// quarter also adds its P slice into the column sums ls (colsum_selector).
template <bool SUMS, bool SW, class Copy = NoCopy, bool QL = !SW>
__device__ __forceinline__ void mfma_pv_read_k(WaveState& w, VFrag& f, KFrag& kf, bf16x8 (&qf)[2][2],
                                               f32x4 (&ls)[2], bf16x8 sel, const uint16_t* lkb,
                                               const uint16_t* lqw, int lq, int lg, const uint16_t* lvb, int lane,
                                               const Copy& copy = Copy()) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          w.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kb][hf][db], w.pb[kb][qb][hf], w.o[qb][db], 0, 0, 0);
      if (SUMS) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          ls[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, w.pb[kb][qb][hf], ls[qb], 0, 0, 0);
      }
      const int ds = kb * 2 + hf;
      if (SW && ds < 3) {  // the next quarter's V^T fragments
        read_vt_part<SW>(f, lvb, lane, 2 * (ds + 1));
        read_vt_part<SW>(f, lvb, lane, 2 * (ds + 1) + 1);
      }
      if (Copy::kActive && ds == 0) {
        copy();
#pragma unroll
        for (int g = 0; g < 6; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002 | 0x004, Copy::kValu, 0);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) kf.a[ds][kk] = k_frag<SW>(lkb, kk * 32 + lq, ds, lg);
      if (QL && (ds == 1 || ds == 3)) {
        qf[ds >> 1][0] = row_frag(lqw, lq, ds >> 1, lg);
        qf[ds >> 1][1] = row_frag(lqw, 32 + lq, ds >> 1, lg);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ void tile_pv(WaveState& w, const uint16_t* lvb, int lane) {
  VFrag f;
  read_vt(f, lvb, lane);
  mfma_pv(w, f);
}

// Q' = Q scaled by sl2 = scale * log2(e) and rounded to bf16, so that QK products
// come out in log2 units: the wave's head, its 64 query rows, kept in registers or
// (QL) in the wave's LDS rows lqw (64 rows, K pitch).  With rq.on the raw rows are
// first rotated to their append positions tok_pos[tok] in fp32 (the lane holds both
// members of each of its pairs: chunk ds pairs with ds + 2 in the half layout,
// neighbours within a chunk in the interleaved one), so the query is rounded to
// bf16 once.
template <bool QL>
__device__ __forceinline__ void load_q(WaveState& w, uint16_t* lqw, const uint16_t* q, int q0, int q1, int hq, int h,
                                       int lq, int lg, float sl2, const int* tok_pos, const RopeQ& rq) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tok = q0 + qb * 32 + lq;
    const uint4* src = (const uint4*)(q + ((long long)tok * hq + h) * D);
    float f[4][8];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tok < q1) x = src[ds * 2 + lg];
      const bf16x8 b = __builtin_bit_cast(bf16x8, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[ds][j] = (float)b[j];
    }
    if (rq.on) {
      const double pos = tok < q1 ? (double)tok_pos[tok] : 0.0;
      if (rq.layout == AKV_ROPE_HALF) {
#pragma unroll
        for (int ds = 0; ds < 2; ++ds)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float c, s;
            rope_angle_cs(pos, rq.rev[ds * 16 + lg * 8 + j], c, s);
            const float a = f[ds][j], bb = f[ds + 2][j];
            f[ds][j] = rot_first(a, bb, c, s);
            f[ds + 2][j] = rot_second(a, bb, c, s);
          }
      } else {
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float c, s;
            rope_angle_cs(pos, rq.rev[ds * 8 + lg * 4 + m], c, s);
            const float a = f[ds][2 * m], bb = f[ds][2 * m + 1];
            f[ds][2 * m] = rot_first(a, bb, c, s);
            f[ds][2 * m + 1] = rot_second(a, bb, c, s);
          }
      }
    }
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      bf16x8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (__bf16)(f[ds][j] * sl2);
      if (QL) *(bf16x8*)(lqw + (qb * 32 + lq) * KP + ds * 16 + lg * 8) = b;
      else w.qf[qb][ds] = b;
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    w.ms[qb] = 0.f;
    w.lrun[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.o[qb][db][i] = 0.f;
  }
  w.shifted = false;
}

// Output accumulators, exponent offsets and sums back to zero (a redo pass).
__device__ __forceinline__ void reset_acc(WaveState& w) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    w.ms[qb] = 0.f;
    w.lrun[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.o[qb][db][i] = 0.f;
  }
  w.shifted = false;
}

// Normalised output rows as bf16, and the optional LSE.  STAGED: the wave's 64 x 64
// output tile first goes to its own Q' rows of LDS (no longer read once the tile
// loop and any rescaling pass are done), then every store instruction writes eight
// whole 128-byte token rows with streaming stores.  The output (T x Hq x 128 B)
// outgrows the last-level cache; cached stores would leave dirty lines there for
// the next kernel to write back, and streaming stores of the 8-byte pieces the MFMA
// layout holds per lane would reach HBM as partial-line writes.  Without staging the
// pieces are stored directly (cached).
template <bool STAGED>
__device__ __forceinline__ void store_out(const WaveState& w, uint16_t* out, float* lse, int q0, int q1,
                                          int hq, int h, int lq, int lg, uint16_t* stage, int lane) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tok = q0 + qb * 32 + lq;
    if (!STAGED && tok >= q1) continue;
    const float inv = 1.f / w.lrun[qb];
    uint16_t* dst = STAGED ? stage + (qb * 32 + lq) * KP : out + ((long long)tok * hq + h) * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * lg;
        const __bf16 b0 = (__bf16)(w.o[qb][db][4 * j] * inv), b1 = (__bf16)(w.o[qb][db][4 * j + 1] * inv);
        const __bf16 b2 = (__bf16)(w.o[qb][db][4 * j + 2] * inv), b3 = (__bf16)(w.o[qb][db][4 * j + 3] * inv);
        uint2 u;
        u.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        u.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *(uint2*)(dst + d0) = u;
      }
    // natural-log sum of exp(scale * score) = (ms + log2 l) / log2 e
    if (lse && lg == 0 && tok < q1) lse[(long long)tok * hq + h] = (w.ms[qb] + __log2f(w.lrun[qb])) / kLog2e;
  }
  if (STAGED) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is in LDS before this wave reads it back
    const int c = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int tok = q0 + row;
      if (tok < q1) {
        const u32x4 v = *(const u32x4*)(stage + row * KP + 8 * c);
        __builtin_nontemporal_store(v, (u32x4*)(out + ((long long)tok * hq + h) * D + 8 * c));
      }
    }
  }
}

// threadIdx.x rebuilt from the lane id (v_mbcnt, a volatile asm so it is redone
// where it is used) and the wave-uniform wave index: the staging addresses derived
// from it are then recomputed each tile in a few VALU ops instead of being kept
// in registers, which under the loop's register pressure meant spill reloads.
__device__ __forceinline__ int local_tid(int wave_s) {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return wave_s * 64 + lane;
}

// Cooperative global -> register -> LDS staging of one K/V tile and its mask
// metadata (fetch, stash; the 1/2/4-head kernel), and the ping-pong kernel's direct
// copies (dma).  The tile's PARTIAL flag travels with its mask registers.
//
// With ROT (the ping-pong kernel without version buffers), row v of a version tile
// is the key of its source token ver_src[v] (rotated to its append position) turned
// by the shift of its run, v - tok_pos[src], whose (cos, sin) per frequency come
// from the run table; its value row is the source's, unchanged.  The rows are
// gathered from the source keys and values by the same direct copies (dma_gather),
// and each wave then turns its own eight key rows in place in LDS (rotate): lane l
// rotates the four pairs 4p .. 4p+3 (p = l % 8) of row l / 8 with the arithmetic of
// the version builder, in the half layout the 8-byte pieces at elements 4p and
// 32 + 4p, in the interleaved one the 16 bytes at element 8p.
// 16 bytes per lane from gbase + voff (bytes) into LDS at lds + 16 * lane, by the
// memory pipe (global_load_lds_dwordx4; lds must be uniform).  Issued as inline
// assembly so that the compiler, which cannot tell one tile slot from another,
// does not make every later LDS read wait for the copy; the pipeline orders the
// copy against the slot's readers itself (vmcnt waits before barriers).
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, const uint16_t* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(la)
               : "m0");
}

// As lds_copy16, from a 64-bit address per lane (gathered rows).
__device__ __forceinline__ void lds_copy16_a(const void* addr, const void* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(la) : "m0");
}

// v[j] of eight wave-uniform values, for the lane's row j in 0..7.
__device__ __forceinline__ int pick8(const int (&v)[8], int j) {
  const int a = (j & 1) ? v[1] : v[0], b = (j & 1) ? v[3] : v[2];
  const int c = (j & 1) ? v[5] : v[4], d = (j & 1) ? v[7] : v[6];
  const int e = (j & 2) ? b : a, f = (j & 2) ? d : c;
  return (j & 4) ? f : e;
}

template <int NT, bool ROT = false>
struct TileStage {
  static constexpr int CPT = (BK * 8 + NT - 1) / NT;  // 16-byte chunks of K (and V) per thread
  static constexpr bool EXACT = CPT * NT == BK * 8;   // every thread owns exactly CPT chunks
  static constexpr bool kRot = ROT;
  uint4 kx[CPT], vx[CPT];
  int mt, md;
  bool partial;
  int wave_s;  // this wave's index (uniform)
  // ROT only
  int gsrc[8], grun[8];  // source token and run of this wave's eight rows of the next tile (uniform)
  float* rl;             // this wave's 2 KB of LDS: the (cos, sin) of its lanes' pairs

  // Chunk c of a tile is 16-byte piece c % 8 of key row c / 8 (the masks tell the
  // compiler that the key index is below 64, so its products are 24-bit).
  __device__ __forceinline__ void fetch(const TileSrc& ts, bool part, int hkv, int hk, const int* tok_drop,
                                        const int* ver_src) {
    partial = part;
    const int tid = local_tid(wave_s);
    // row0's head-hk row as a uniform base; the per-thread byte offset is 32-bit
    const long long base = ((long long)ts.row0 * hkv + hk) * D;
    const char* kb = (const char*)(ts.k + base);
    const char* vb = (const char*)(ts.v + base);
    const uint32_t row_bytes = (uint32_t)hkv * (D * 2);
    if (ts.nrows == BK) {  // uniform: a whole tile of keys
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + j * NT;
        if (EXACT || c < BK * 8) {
          const uint32_t off = __umul24((uint32_t)(c >> 3) & (BK - 1), row_bytes) + (uint32_t)(c & 7) * 16u;
          kx[j] = *(const uint4*)(kb + off);
          vx[j] = *(const uint4*)(vb + off);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + j * NT;
        const int key = (c >> 3) & (BK - 1);
        kx[j] = make_uint4(0, 0, 0, 0);
        vx[j] = make_uint4(0, 0, 0, 0);
        if ((EXACT || c < BK * 8) && key < ts.nrows) {
          const uint32_t off = __umul24((uint32_t)key, row_bytes) + (uint32_t)(c & 7) * 16u;
          kx[j] = *(const uint4*)(kb + off);
          vx[j] = *(const uint4*)(vb + off);
        }
      }
    }
    if (part && tid < BK) {
      const int key = tid;
      mt = INT_MAX;
      md = INT_MIN;
      if (key < ts.nrows) {
        mt = ts.ver ? -1 : ts.row0 + key;
        md = tok_drop[ts.ver ? ver_src[ts.row0 + key] : ts.row0 + key];
      }
    }
  }
  // SW layout: this wave's eight rows of the tile (rows 8 wave .. 8 wave + 7) copied
  // by the memory pipe straight into LDS.  Lane l writes its 16 bytes at l * 16 of
  // the wave's 1 KB, which is chunk l % 8 of row 8 wave + l / 8, so it reads the
  // source chunk that the swizzle places there.  Rows past a ragged tile's end copy
  // its last row (finite values; the tile is PARTIAL and its mask hides them).
  __device__ __forceinline__ void dma(const TileSrc& ts, int hkv, int hk, uint16_t* lkb, uint16_t* lvb) {
    const int lane = local_tid(wave_s) & 63;
    const int row = 8 * wave_s + (lane >> 3), p = lane & 7;
    const int srow = row < ts.nrows ? row : ts.nrows - 1;
    // row0's head-hk row as a uniform base; the per-lane byte offset is 32-bit
    const long long base = ((long long)ts.row0 * hkv + hk) * D;
    const uint32_t rbytes = __umul24((uint32_t)srow & (BK - 1), (uint32_t)hkv * (D * 2));
    const uint32_t ok = rbytes + ((uint32_t)(p ^ swz_k(row)) << 4);
    const uint32_t ov = rbytes + ((uint32_t)(p ^ swz_v(row)) << 4);
    lds_copy16(ts.k + base, ok, lkb + 8 * wave_s * D);
    lds_copy16(ts.v + base, ov, lvb + 8 * wave_s * D);
  }
  // ROT: (source, run) of this wave's eight rows of tile ts when it is a version
  // tile, by scalar loads (the barrier that ends the phase waits for them); for
  // another tile the first eight entries, unused.  The version tables carry 64
  // entries of padding, so the rows past a ragged tile's end (and the first eight,
  // with no version rows at all) read valid entries; a tile's mask hides its rows
  // past the end.
  __device__ __forceinline__ void load_gather(const TileSrc& ts, const int* ver_src, const int* ver_run) {
    const int base = ts.ver ? ts.row0 + 8 * wave_s : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      gsrc[j] = ver_src[base + j];
      grun[j] = ver_run[base + j];
    }
  }
  // ROT: dma with a version tile's rows gathered from their source tokens (gsrc).
  // The lane's byte offset from head hk's row of token 0 is 32-bit (the host keeps
  // the key and value arrays under 4 GiB), so one form serves both kinds of tile.
  __device__ __forceinline__ void dma_gather(const TileSrc& ts, int hkv, int hk, uint16_t* lkb, uint16_t* lvb) {
    const int lane = local_tid(wave_s) & 63;
    const int j = lane >> 3, row = 8 * wave_s + j, p = lane & 7;
    const int tok = ts.ver ? pick8(gsrc, j) : ts.row0 + (row < ts.nrows ? row : ts.nrows - 1);
    const uint32_t rb = (uint32_t)tok * ((uint32_t)hkv * (D * 2));
    lds_copy16(ts.k + hk * D, rb + ((uint32_t)(p ^ swz_k(row)) << 4), lkb + 8 * wave_s * D);
    lds_copy16(ts.v + hk * D, rb + ((uint32_t)(p ^ swz_v(row)) << 4), lvb + 8 * wave_s * D);
  }
  __device__ __forceinline__ void dma_tile(const TileSrc& ts, int hkv, int hk, uint16_t* lkb, uint16_t* lvb) {
    if constexpr (ROT)
      dma_gather(ts, hkv, hk, lkb, lvb);
    else
      dma(ts, hkv, hk, lkb, lvb);
  }
  // ROT: the (cos, sin) of the four pairs of each lane's key in the version tile
  // whose runs load_gather holds, copied by the memory pipe into the wave's region
  // rl (lane l's 32 bytes at 16 l and 1024 + 16 l).
  __device__ __forceinline__ void dma_rot(const float* rot_tab) {
    const int lane = local_tid(wave_s) & 63;
    const float* t = rot_tab + ((long long)pick8(grun, lane >> 3) * (D / 2) + 4 * (lane & 7)) * 2;
    lds_copy16_a(t, rl);
    lds_copy16_a(t + 4, rl + 256);
  }
  // ROT: this wave's eight key rows of the version tile in slot lkb turned in place
  // by the (cos, sin) that dma_rot copied (the caller has waited for both copies).
  template <int RL>
  __device__ __forceinline__ void rotate(uint16_t* lkb) const {
    const int lane = local_tid(wave_s) & 63;
    const int row = 8 * wave_s + (lane >> 3), p = lane & 7, sw = swz_k(row);
    const float4 r0 = *(const float4*)(rl + 4 * lane), r1 = *(const float4*)(rl + 256 + 4 * lane);
    const float cs[4] = {r0.x, r0.z, r1.x, r1.z}, sn[4] = {r0.y, r0.w, r1.y, r1.w};
    uint16_t* rp = lkb + row * D;
    if (RL == AKV_ROPE_HALF) {  // pair 4p + i: elements 4p + i and 32 + 4p + i
      uint2* pa = (uint2*)(rp + (((p >> 1) ^ sw) << 3) + 4 * (p & 1));
      uint2* pb = (uint2*)(rp + (((4 + (p >> 1)) ^ sw) << 3) + 4 * (p & 1));
      const bf16x4 xa = __builtin_bit_cast(bf16x4, *pa), xb = __builtin_bit_cast(bf16x4, *pb);
      bf16x4 ya, yb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (float)xa[i], b = (float)xb[i];
        ya[i] = (__bf16)rot_first(a, b, cs[i], sn[i]);
        yb[i] = (__bf16)rot_second(a, b, cs[i], sn[i]);
      }
      *pa = __builtin_bit_cast(uint2, ya);
      *pb = __builtin_bit_cast(uint2, yb);
    } else {  // pair 4p + i: elements 8p + 2i and 8p + 2i + 1
      bf16x8* px = (bf16x8*)(rp + ((p ^ sw) << 3));
      const bf16x8 x = *px;
      bf16x8 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (float)x[2 * i], b = (float)x[2 * i + 1];
        y[2 * i] = (__bf16)rot_first(a, b, cs[i], sn[i]);
        y[2 * i + 1] = (__bf16)rot_second(a, b, cs[i], sn[i]);
      }
      *px = y;
    }
  }
  // The mask metadata of a PARTIAL tile into registers (wave 0), for stash_mask.
  __device__ __forceinline__ void fetch_mask(const TileSrc& ts, bool part, const int* tok_drop, const int* ver_src) {
    partial = part;
    const int tid = local_tid(wave_s);
    if (part && tid < BK) {
      mt = INT_MAX;
      md = INT_MIN;
      if (tid < ts.nrows) {
        mt = ts.ver ? -1 : ts.row0 + tid;
        md = tok_drop[ts.ver ? ver_src[ts.row0 + tid] : ts.row0 + tid];
      }
    }
  }
  __device__ __forceinline__ void stash_mask(int* mtok, int* mdrop) {
    const int tid = local_tid(wave_s);
    if (partial && tid < BK) {
      mtok[tid] = mt;
      mdrop[tid] = md;
    }
  }
  __device__ __forceinline__ void stash(uint16_t* lkb, uint16_t* lvb, int* mtok, int* mdrop) {
    const int tid = local_tid(wave_s);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * NT;
      if (EXACT || c < BK * 8) {
        const int key = (c >> 3) & (BK - 1), ch = c & 7;
        *(uint4*)(lkb + key * KP + ch * 8) = kx[j];
        *(uint4*)(lvb + key * VP + ch * 8) = vx[j];
      }
    }
    if (partial && tid < BK) {
      mtok[tid] = mt;
      mdrop[tid] = md;
    }
  }
};

#define AKV_ATTN_PARAMS                                                                            \
  const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, \
      const uint16_t *__restrict__ kver, const uint16_t *__restrict__ vver,                        \
      const int *__restrict__ item_desc, const int *__restrict__ tiles,                            \
      const int *__restrict__ order, const int *__restrict__ tok_drop,                             \
      const int *__restrict__ ver_src, uint16_t *__restrict__ out, float *__restrict__ lse,       \
      int hq, int hkv, float scale, const int *__restrict__ tok_pos, RopeQ rq

// One wave per query head for groups of 1, 2 or 4 query heads per kv head.  Each
// K/V tile is staged synchronously into a single LDS buffer (20 KB per workgroup),
// and the registers are held to two waves per SIMD, so several workgroups share a
// CU: while one waits for its tile or runs its softmax, another's MFMAs run.  (A
// double-buffered version that prefetched the next tile into registers spilled at
// this register budget and ran slower.)
template <int GROUP>
__global__ __launch_bounds__(64 * GROUP, 2) void seg_attn_bf16(AKV_ATTN_PARAMS) {
  constexpr int NT = 64 * GROUP;
  __shared__ __attribute__((aligned(16))) uint16_t lk[BK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t lv[BK * VP];
  __shared__ int mtok[BK], mdrop[BK];

  const int hk = blockIdx.x % hkv;
  const int item = order[blockIdx.x / hkv];
  const int* dsc = item_desc + item * ID_WORDS;
  const int q0 = dsc[ID_QBEGIN], q1 = dsc[ID_QEND], tb = dsc[ID_TB], te = dsc[ID_TE];
  const int r = dsc[ID_R], voff = dsc[ID_VEROFF], t0 = dsc[ID_TILE0], t1 = dsc[ID_TILE1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = hk * GROUP + wave;
  const int lq = lane & 31, lg = lane >> 5;
  const int nvt = (r + BK - 1) / BK;
  const float sl2 = scale * kLog2e;

  WaveState w;
  load_q<false>(w, nullptr, q, q0, q1, hq, h, lq, lg, sl2, tok_pos, rq);
  TileStage<NT> st;
  st.wave_s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = t0; t < t1; ++t) {
    const int ent = tiles[t];
    const bool partial = (ent & 3) == AKV_TILE_PARTIAL;
    st.fetch(tile_src(ent, nvt, voff, r, tb, te, k, v, kver, vver), partial, hkv, hk, tok_drop, ver_src);
    st.stash(lk, lv, mtok, mdrop);
    lds_barrier();
    tile_qk<false>(w, lk, nullptr, lq, lg);
    tile_softmax<false>(w, partial, mtok, mdrop, lk, nullptr, q0, lq, lg);
    tile_pv(w, lv, lane);
    lds_barrier();  // every wave is done with this tile before the next one is staged
  }
  store_out<false>(w, out, lse, q0, q1, hq, h, lq, lg, nullptr, lane);
}

// Ping-pong pipeline for 8 query heads per kv head (8 waves, two per SIMD), for
// two kv heads of 4 query heads each, or for 8 / M query heads over M parts of a
// query tile.
// Waves 0-3 (group A) and 4-7 (group B) run the same tile loop one phase apart,
// separated by workgroup barriers, so while one wave of a SIMD issues MFMAs
// (PV of tile t and QK of tile t+1) its partner runs the softmax of its tile on
// the VALU.  A K/V tile is read from LDS for three phases (its K and V^T in the
// MFMA phase before its softmax, its mask in the softmax).
//
// Direct copies: tiles rotate through four LDS slots.  In iteration t's MFMA phase every wave copies its eight rows of
// tile t+3 from memory straight into LDS (global_load_lds), into the slot of tile
// t-1, whose last reader passed an earlier barrier; each wave waits for its copies
// of the iteration before (vmcnt) ahead of each barrier, so a copy has two phases
// to land and the tile is whole before the barrier after which it is first read.
// The copies cost the MFMA wave a few dozen issue slots between its MFMAs and
// cost the softmax wave, whose phase was the longer one, nothing.
//
// Without version buffers (ROT) a version tile's rows are gathered from their
// source tokens by the same copies, with the (cos, sin) of their runs copied after
// them; in iteration t's MFMA phase each wave turns its own eight key rows of tile
// t+2 (copied in iteration t-1) in place, between the QK MFMAs, before the
// barriers after which tile t+2 is first read.
//
// The loop is unrolled over the slots so every LDS slot address is a constant.
//
// SAFE = false is the fast pass (offset 0, column sums on the matrix cores);
// SAFE = true is the lazily-rescaled softmax with per-tile range checks.
constexpr int kPPThreads = 512;
// The tile ring: four LDS slots of HPW x 16 KB (K and V of each of the workgroup's
// HPW kv heads, swizzled unpadded rows), filled by direct copies.  A wave reads the
// tiles of its own kv head (koff into each slot).
template <bool ROT, int HPW = 1>
struct PPCtx {
  static constexpr int NS = 4;
  static constexpr int KSZ = BK * D;
  static constexpr int VSZ = BK * D;
  uint16_t* lk[NS];  // K and V tiles of each slot (the first head's; the next head's KSZ / VSZ on)
  uint16_t* lv[NS];
  int koff;          // this wave's head within the slot times KSZ (0 with one head)
  int (*mtok)[BK];
  int (*mdrop)[BK];
  const uint16_t* lqw;
  const int* tiles;  // this work item's tile entries
  const uint16_t *k, *v, *kver, *vver;
  const int *tok_drop, *ver_src;
  const int* ver_run;   // ROT: run of each version row
  const float* rot_tab; // ROT: (cos, sin) per run and frequency
  int n, nvt, voff, r, tb, te, hkv, hk, q0, lq, lg, lane;  // hk: the workgroup's first kv head
  __device__ __forceinline__ TileSrc src(int ent) const { return tile_src(ent, nvt, voff, r, tb, te, k, v, kver, vver); }
  // this wave's K and V tile in slot j
  __device__ __forceinline__ uint16_t* rk(int j) const { return HPW == 1 ? lk[j] : lk[j] + koff; }
  __device__ __forceinline__ uint16_t* rv(int j) const { return HPW == 1 ? lv[j] : lv[j] + koff; }
  // entry of tile t, or of the last tile past the end (n >= 1; the caller ignores it)
  __device__ __forceinline__ int entry(int t) const { return tiles[min(t, n - 1)]; }
  __device__ __forceinline__ bool ver(int ent) const { return (ent >> 2) < nvt; }
};

// A tile copy issued from inside the MFMA phase (mfma_pv_read_k calls it).
// With HPW kv heads per workgroup, the rows of every head are copied into their
// part of the slot.
template <class Stage, int HPW = 1>
struct TileCopy {
  Stage& st;
  const TileSrc& ts;
  uint16_t *dk, *dv;
  int hkv, hk;
  static constexpr bool kActive = true;
  static constexpr int kValu = Stage::kRot ? 10 : 8;  // ALU instructions between two of its MFMAs
  __device__ __forceinline__ void operator()() const {
#pragma unroll
    for (int e = 0; e < HPW; ++e) st.dma_tile(ts, hkv, hk + e, dk + e * BK * D, dv + e * BK * D);
  }
};

// QK of the ROT kernel, which keeps Q' in the wave's LDS rows: the first two d
// slices come from PV (qf), the others are read two slices ahead of their MFMAs.
// With ROTATE the in-place rotation of a version tile's key rows is woven between
// the MFMAs: this wave's eight rows of the tile in slot lkr, copied one iteration
// ago together with their (cos, sin), are turned here; the tile is first read
// after the barriers that end this iteration.
template <bool ROTATE, int RL, class Stage>
__device__ __forceinline__ void mfma_qk_ql(WaveState& w, const KFrag& f, const bf16x8 (&qf)[2][2],
                                           const uint16_t* lqw, int lq, int lg, const Stage& st, uint16_t* lkr) {
  if (ROTATE) {
    // only this iteration's tile copies (the two latest vector-memory
    // instructions) may still be in flight; the LDS reads stay below the wait
    __builtin_amdgcn_s_waitcnt(kWaitVm2);
    asm volatile("" ::: "memory");
    st.template rotate<RL>(lkr);
  }
  const f32x16 zero = {};
  bf16x8 b[3][2];
  b[0][0] = qf[0][0];
  b[0][1] = qf[0][1];
  b[1][0] = qf[1][0];
  b[1][1] = qf[1][1];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    if (ds + 2 < 4) {
      b[(ds + 2) % 3][0] = row_frag(lqw, lq, ds + 2, lg);
      b[(ds + 2) % 3][1] = row_frag(lqw, 32 + lq, ds + 2, lg);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        w.s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ds][kb], b[ds % 3][qb], ds ? w.s[kb][qb] : zero,
                                                              0, 0, 0);
  }
}

// One iteration of the ping-pong loop for tile i held in LDS slot S; ent holds
// the entries of tiles i .. i+3 and is advanced by one.
template <bool SAFE, int S, bool ROT, int RL, int HPW = 1>
__device__ __forceinline__ void pp_step(WaveState& w, f32x4 (&ls)[2], bf16x8 sel, TileStage<kPPThreads, ROT>& st,
                                        VFrag& vf, const PPCtx<ROT, HPW>& c, int i, int (&ent)[4]) {
  constexpr int NS = PPCtx<ROT, HPW>::NS;
  // vector-memory instructions of one iteration's tile copies (two per head)
  constexpr int kWaitIter = (ROT || HPW == 2) ? kWaitVm4 : kWaitVm2;
  constexpr int S1 = (S + 1) % NS, S2 = (S + 2) % NS, S3 = (S + 3) % NS;
  // phase 1 (VALU): the softmax of tile i.  The tiles arrive by direct copies
  // issued in the MFMA phase, so this phase only moves a PARTIAL tile's mask
  // metadata (loaded into registers one iteration before it is stored) and, with
  // ROT, requests the (source, run) of tile i+3's rows for its copy (past the last
  // tile, the last tile's again).
  if (i + 2 < c.n) st.stash_mask(c.mtok[S2], c.mdrop[S2]);
  if (i + 3 < c.n) st.fetch_mask(c.src(ent[3]), (ent[3] & 3) == AKV_TILE_PARTIAL, c.tok_drop, c.ver_src);
  if (ROT) st.load_gather(c.src(ent[3]), c.ver_src, c.ver_run);
  __builtin_amdgcn_sched_barrier(0);
  // the entry the next iteration loads by, requested here: its scalar load is
  // waited for only at the barrier that ends this phase
  const int ent_next = c.entry(i + 4);
  const bool part = (ent[0] & 3) == AKV_TILE_PARTIAL;
  if (SAFE)
    tile_softmax<ROT, true>(w, part, c.mtok[S], c.mdrop[S], c.rk(S), c.lqw, c.q0, c.lq, c.lg);
  else
    tile_softmax_fast(w, part, c.mtok[S], c.mdrop[S], c.q0, c.lq, c.lg);
  if (ROT) {
    // P is complete here: the branches of this kernel's MFMA phase would otherwise
    // let the compiler sink the exps past the barrier to their use in PV, where the
    // MFMA wave would issue them itself
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 t = __builtin_bit_cast(u32x4, w.pb[kb][qb][hf]);
          asm volatile("" : "+v"(t));
          w.pb[kb][qb][hf] = __builtin_bit_cast(bf16x8, t);
        }
  }
  // the copies this wave issued two iterations ago (and earlier) have landed in
  // LDS before the barrier after which other waves may read them; the previous
  // iteration's (its last two vector-memory instructions before this phase's mask
  // loads, four with ROT when it also copied (cos, sin), or with two kv heads) may
  // stay in flight
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitIter);
  // the first PV quarter's V^T fragments; the others are read inside PV
  read_vt_part<true>(vf, c.rv(S), c.lane, 0);
  read_vt_part<true>(vf, c.rv(S), c.lane, 1);
  lds_barrier();
  // phase 2 (MFMA): PV of tile i with the K fragments of tile i+1 and tile i's own
  // V^T fragments (one quarter ahead) read between its MFMAs; QK of tile i+1, with
  // ROT and a version tile i+2 woven with that tile's rotation.  After the last
  // tile, slot S1 holds an older tile: its K reads are harmless and unused.
  __builtin_amdgcn_s_setprio(1);
  KFrag kf;
  bf16x8 qf[2][2];
  {
    // Each wave copies its rows of tile i+3 into the slot of tile i-1, whose last
    // reader (group B's softmax) passed a barrier before this phase.  The copy's
    // instructions issue between the first PV MFMAs, where this wave's issue slots
    // are free.  Past the last tile the entry is the last tile's, and its rows go
    // to a slot that is not read again (no branch: a branch here lets the compiler
    // sink the softmax's exps past the barrier into this phase).
    const TileSrc ts = c.src(ent[3]);
    const TileCopy<TileStage<kPPThreads, ROT>, HPW> copy{st, ts, c.lk[S3], c.lv[S3], c.hkv, c.hk};
    mfma_pv_read_k<!SAFE, true, TileCopy<TileStage<kPPThreads, ROT>, HPW>, ROT>(w, vf, kf, qf, ls, sel, c.rk(S1),
                                                                                 c.lqw, c.lq, c.lg, c.rv(S), c.lane,
                                                                                 copy);
  }
  __builtin_amdgcn_sched_barrier(0);
  // P of tile i is dead here, before the scores of tile i+1 are born: they share registers
  if (i + 1 < c.n) {
    if (!ROT)
      mfma_qk_lq<true>(w, kf, qf, c.lqw, c.lq, c.lg, vf, c.rv(S1), c.lane);
    else if (c.ver(ent[2]))
      mfma_qk_ql<true, RL>(w, kf, qf, c.lqw, c.lq, c.lg, st, c.lk[S2]);
    else
      mfma_qk_ql<false, RL>(w, kf, qf, c.lqw, c.lq, c.lg, st, c.lk[S2]);
  }
  // ROT: the (cos, sin) of tile i+3's version rows, for their rotation in the next
  // iteration; issued after this iteration's rotation has read the region
  const bool ver3 = ROT && c.ver(ent[3]);
  if (ver3) {
    __builtin_amdgcn_sched_barrier(0);
    st.dma_rot(c.rot_tab);
  }
  __builtin_amdgcn_s_setprio(0);
  // every wave's copies of one iteration ago (and earlier) have landed before the
  // barrier; this phase's stay in flight
  __builtin_amdgcn_sched_barrier(0);
  if (ver3)
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
  else
    __builtin_amdgcn_s_waitcnt(HPW == 2 ? kWaitVm4 : kWaitVm2);
  lds_barrier();
  ent[0] = ent[1];
  ent[1] = ent[2];
  ent[2] = ent[3];
  ent[3] = ent_next;
}

template <bool SAFE, bool ROT, int RL, int HPW = 1>
__device__ __forceinline__ void pp_pipeline(WaveState& w, f32x4 (&ls)[2], bf16x8 sel,
                                            TileStage<kPPThreads, ROT>& st, const PPCtx<ROT, HPW>& c, bool lag) {
  int ent[4] = {c.entry(0), c.entry(1), c.entry(2), c.entry(3)};
  // Tiles 0, 1 and 2 copied and tile 2's mask loaded.  With ROT the version rows of
  // tiles 0 and 1 are rotated here, one tile at a time through the wave's (cos,
  // sin) region, and tile 2's by the first iteration; tile 2 is then copied (the
  // last tile's rows past the end) even when it does not exist, as the loop does.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < c.n) {
      const TileSrc ts = c.src(ent[j]);
      st.fetch_mask(ts, (ent[j] & 3) == AKV_TILE_PARTIAL, c.tok_drop, c.ver_src);
      if (ROT) st.load_gather(ts, c.ver_src, c.ver_run);
#pragma unroll
      for (int e = 0; e < HPW; ++e) st.dma_tile(ts, c.hkv, c.hk + e, c.lk[j] + e * BK * D, c.lv[j] + e * BK * D);
      if (ROT && ts.ver) {
        st.dma_rot(c.rot_tab);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("" ::: "memory");
        st.template rotate<RL>(c.lk[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
      st.stash_mask(c.mtok[j], c.mdrop[j]);
    }
  }
  if (ROT) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    const TileSrc ts = c.src(ent[2]);
    if (c.n > 2) st.fetch_mask(ts, (ent[2] & 3) == AKV_TILE_PARTIAL, c.tok_drop, c.ver_src);
    st.load_gather(ts, c.ver_src, c.ver_run);
    st.dma_tile(ts, c.hkv, c.hk, c.lk[2], c.lv[2]);
    if (ts.ver) {
      __builtin_amdgcn_sched_barrier(0);
      st.dma_rot(c.rot_tab);
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    if (c.n > 2) {
      st.fetch_mask(c.src(ent[2]), (ent[2] & 3) == AKV_TILE_PARTIAL, c.tok_drop, c.ver_src);
#pragma unroll
      for (int e = 0; e < HPW; ++e)
        st.dma_tile(c.src(ent[2]), c.hkv, c.hk + e, c.lk[2] + e * BK * D, c.lv[2] + e * BK * D);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
  lds_barrier();
  if (lag) lds_barrier();
  tile_qk<ROT, true>(w, c.rk(0), c.lqw, c.lq, c.lg);
  VFrag vf;
  lds_barrier();
  for (int i = 0; i < c.n; i += PPCtx<ROT, HPW>::NS) {
    pp_step<SAFE, 0, ROT, RL, HPW>(w, ls, sel, st, vf, c, i, ent);
    if (i + 1 >= c.n) break;
    pp_step<SAFE, 1, ROT, RL, HPW>(w, ls, sel, st, vf, c, i + 1, ent);
    if (i + 2 >= c.n) break;
    pp_step<SAFE, 2, ROT, RL, HPW>(w, ls, sel, st, vf, c, i + 2, ent);
    if (i + 3 >= c.n) break;
    pp_step<SAFE, 3, ROT, RL, HPW>(w, ls, sel, st, vf, c, i + 3, ent);
  }
  // no copy (those past the last tile included) is still in flight when the
  // slots are next written
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (!lag) lds_barrier();
}

// Largest final column sum the fast pass accepts: P <= 2^100 keeps every fp32
// product and accumulation of the PV step far from overflow.
constexpr float kFastHi = 1.2676506002282294e30f;  // 2^100

// ROT: version rows are gathered from the source keys and values and their keys
// rotated in LDS (TileStage), with ver_run / rot_tab, instead of read from version
// buffers; RL is then the pair layout.
//
// HPW = 2 (4 query heads per kv head, no ROT): the workgroup takes two kv heads,
// group A (waves 0-3) the first one's four query heads and group B (waves 4-7) the
// second one's; each slot of the ring holds both heads' tiles, so the K/V ring
// takes 128 KB and the output is stored straight from the accumulators.
//
// M > 1 (8 / M query heads per kv head): a work item is a query tile of
// 64 M tokens (a plan built with bq = 64 M), cut into M 64-token parts; wave w runs
// part w / (8 / M) of query head w % (8 / M), so the eight waves still share every
// K/V tile.  The plan's tile classes cover the whole 64 M-row tile: a FULL tile is
// visible to every row, and each wave masks a PARTIAL tile by its own rows (a part
// past the end of the item has no rows: it computes on zero queries and stores
// nothing).
template <bool ROT, int RL = AKV_ROPE_HALF, int HPW = 1, int M = 1>
__global__ __launch_bounds__(kPPThreads) void seg_attn_bf16_pp(AKV_ATTN_PARAMS, const int* __restrict__ ver_run,
                                                               const float* __restrict__ rot_tab) {
  static_assert(HPW == 1 || (HPW == 2 && !ROT && M == 1), "two kv heads per workgroup only with version buffers");
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "1, 2, 4 or 8 query tile parts");
  constexpr int GROUP = 8 / (HPW * M);  // query heads per kv head
  using Ctx = PPCtx<ROT, HPW>;
  __shared__ __attribute__((aligned(16))) uint16_t lk[Ctx::NS][HPW * Ctx::KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t lv[Ctx::NS][HPW * Ctx::VSZ];
  __shared__ int mtok[Ctx::NS][BK], mdrop[Ctx::NS][BK];
  __shared__ __attribute__((aligned(16))) uint16_t lqs[HPW == 1 ? kPPThreads / 64 : 1][64 * KP];  // per wave
  __shared__ __attribute__((aligned(16))) float rtab[ROT ? (kPPThreads / 64) * 512 : 4];  // ROT: 2 KB per wave
  __shared__ int redo;

  const int npair = hkv / HPW;
  const int hk0 = (blockIdx.x % npair) * HPW;  // the workgroup's first kv head
  const int item = order[blockIdx.x / npair];
  const int* dsc = item_desc + item * ID_WORDS;
  const int qi0 = dsc[ID_QBEGIN], qi1 = dsc[ID_QEND], tb = dsc[ID_TB], te = dsc[ID_TE];
  const int r = dsc[ID_R], voff = dsc[ID_VEROFF], t0 = dsc[ID_TILE0], t1 = dsc[ID_TILE1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hsel = HPW == 1 ? 0 : wave >> 2;  // this wave's kv head within the workgroup
  const int hk = hk0 + hsel;
  const int h = hk * GROUP + (wave & (GROUP - 1));
  // this wave's query rows [q0, q1): the item's, or with M parts its part's
  const int q0 = M == 1 ? qi0 : qi0 + 64 * (wave / GROUP);
  const int q1 = M == 1 ? qi1 : min(qi1, q0 + 64);
  const int lq = lane & 31, lg = lane >> 5;
  uint16_t* lqw = lqs[HPW == 1 ? wave : 0];  // this wave's Q' rows (written and read by this wave only)
  const bool lag = wave >= 4;  // group B
  const int nvt = (r + BK - 1) / BK;
  const float sl2 = scale * kLog2e;
  const int n = t1 - t0;
  if (n <= 0) return;  // uniform over the workgroup; every query sees at least itself
  if (threadIdx.x == 0) redo = 0;  // published by the first barrier of the pipeline

  WaveState w;
  load_q<ROT>(w, lqw, q, q0, q1, hq, h, lq, lg, sl2, tok_pos, rq);  // ROT: Q' in LDS
  TileStage<kPPThreads, ROT> st;
  st.wave_s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.rl = rtab + (ROT ? st.wave_s * 512 : 0);
  const bf16x8 sel = colsum_selector(lane);
  f32x4 ls[2] = {};
  Ctx c;
#pragma unroll
  for (int j = 0; j < Ctx::NS; ++j) {
    c.lk[j] = lk[j];
    c.lv[j] = lv[j];
  }
  c.mtok = mtok;
  c.mdrop = mdrop;
  c.lqw = lqw;
  c.tiles = tiles + t0;
  c.k = k;
  c.v = v;
  c.kver = ROT ? k : kver;   // ROT gathers version rows from the source keys
  c.vver = ROT ? v : vver;
  c.tok_drop = tok_drop;
  c.ver_src = ver_src;
  c.ver_run = ver_run;
  c.rot_tab = rot_tab;
  c.n = n;
  c.nvt = nvt;
  c.voff = voff;
  c.r = r;
  c.tb = tb;
  c.te = te;
  c.hkv = hkv;
  c.hk = hk0;
  c.koff = hsel * Ctx::KSZ;
  c.q0 = q0;
  c.lq = lq;
  c.lg = lg;
  c.lane = lane;
  pp_pipeline<false, ROT, RL, HPW>(w, ls, sel, st, c, lag);
  // Accept the fast pass when every real query column's sum lies in [2^-40, 2^100]
  // (also false for inf/NaN); otherwise the workgroup redoes the item with the
  // rescaling softmax.
  bool bad = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = ls[qb][0];
    bad |= (q0 + qb * 32 + lq < q1) && !(l >= kSumLo && l <= kFastHi);
  }
  if (__any(bad) && lane == 0) redo = 1;
  lds_barrier();
  if (__builtin_amdgcn_readfirstlane(redo)) {
    asm volatile("");  // rare: keep the second pipeline out of the common path
    reset_acc(w);  // O, offsets and sums (Q' stays where it is)
    pp_pipeline<true, ROT, RL, HPW>(w, ls, sel, st, c, lag);
  } else {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) w.lrun[qb] = ls[qb][0];
  }
  store_out<HPW == 1>(w, out, lse, q0, q1, hq, h, lq, lg, lqw, lane);
}

// (cos, sin) of every version run's shift for every frequency: table[run][i] =
// (cos, sin)(delta_run * theta_i), evaluated as in the RoPE kernels (rope_angle.h),
// so a key rotated at staging time equals its version-buffer copy bit for bit.
__global__ __launch_bounds__(256) void rot_table_kernel(const int* __restrict__ run_delta, long long n_runs,
                                                        int half, RopeQ rq, float* __restrict__ table) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_runs * half) return;
  const long long run = t / half;
  const int i = (int)(t - run * half);
  float c, s;
  rope_angle_cs((double)run_delta[run], rq.rev[i], c, s);
  table[2 * t] = c;
  table[2 * t + 1] = s;
}

// float32 path: one thread per (query token, head), keys walked one at a time
// with an exact online softmax.  For small problems and fp32 checks.
template <int DD>
__global__ __launch_bounds__(256) void seg_attn_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ kver, const float* __restrict__ vver, const int* __restrict__ item_desc,
    const int* __restrict__ tiles, const int* __restrict__ order, const int* __restrict__ tok_drop,
    const int* __restrict__ ver_src, float* __restrict__ out, float* __restrict__ lse, int hq,
    int hkv, int bk, float scale, const int* __restrict__ tok_pos, RopeQ rq) {
  const int h = blockIdx.x % hq;
  const int item = order[blockIdx.x / hq];
  const int g = h / (hq / hkv);
  const int* dsc = item_desc + item * ID_WORDS;
  const int q0 = dsc[ID_QBEGIN], q1 = dsc[ID_QEND], tb = dsc[ID_TB], te = dsc[ID_TE];
  const int r = dsc[ID_R], voff = dsc[ID_VEROFF], t0 = dsc[ID_TILE0], t1 = dsc[ID_TILE1];
  const int tok = q0 + (int)threadIdx.x;
  if (tok >= q1) return;
  const int nvt = (r + bk - 1) / bk;
  float qv[DD], acc[DD];
  const float* qp = q + ((long long)tok * hq + h) * DD;
#pragma unroll
  for (int i = 0; i < DD; ++i) { qv[i] = qp[i]; acc[i] = 0.f; }
  if (rq.on) {  // raw query: rotate to its append position
    const double pos = (double)tok_pos[tok];
#pragma unroll
    for (int i = 0; i < DD / 2; ++i) {
      float c, s;
      rope_angle_cs(pos, rq.rev[i], c, s);
      const int ia = rq.layout == AKV_ROPE_HALF ? i : 2 * i, ib = rq.layout == AKV_ROPE_HALF ? i + DD / 2 : 2 * i + 1;
      const float a = qv[ia], b = qv[ib];
      qv[ia] = rot_first(a, b, c, s);
      qv[ib] = rot_second(a, b, c, s);
    }
  }
  float m = -INFINITY, l = 0.f;
  for (int t = t0; t < t1; ++t) {
    const int kt = tiles[t] >> 2;
    const bool ver = kt < nvt;
    const int row0 = ver ? voff + kt * bk : tb + (kt - nvt) * bk;
    const int nrows = ver ? min(bk, r - kt * bk) : min(bk, te - row0);
    for (int key = 0; key < nrows; ++key) {
      const int row = row0 + key;
      const bool vis = ver ? (tok < tok_drop[ver_src[row]]) : (row <= tok && tok < tok_drop[row]);
      if (!vis) continue;
      const float* kp = (ver ? kver : k) + ((long long)row * hkv + g) * DD;
      const float* vp = (ver ? vver : v) + ((long long)row * hkv + g) * DD;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < DD; ++i) s = fmaf(qv[i], kp[i], s);
      s *= scale;
      if (s > m) {
        const float a = expf(m - s);
        l = l * a + 1.f;
#pragma unroll
        for (int i = 0; i < DD; ++i) acc[i] = fmaf(acc[i], a, vp[i]);
        m = s;
      } else {
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int i = 0; i < DD; ++i) acc[i] = fmaf(p, vp[i], acc[i]);
      }
    }
  }
  float* op = out + ((long long)tok * hq + h) * DD;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < DD; ++i) op[i] = acc[i] * inv;
  if (lse) lse[(long long)tok * hq + h] = m + logf(l);
}

}  // namespace

int launch_segment_attention(const AttnArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.n_items == 0) return AKV_OK;
  (void)hipGetLastError();
  if (a.dtype == AKV_BF16) {
    const long long blocks = a.n_items * a.hkv;
    if (blocks > 0x7fffffffLL) return fail(AKV_EINVAL, "too many work items");
    const int grp = a.hq / a.hkv;
#define AKV_LAUNCH_BF16(G)                                                                           \
  hipLaunchKernelGGL(seg_attn_bf16<G>, dim3((unsigned)blocks), dim3(64 * G), 0, s,                  \
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,              \
                     (const uint16_t*)a.k_ver, (const uint16_t*)a.v_ver, a.item_desc, a.tiles,      \
                     a.order, a.tok_drop, a.ver_src, (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale,    \
                     a.tok_pos, a.rq)
#define AKV_LAUNCH_PARTS_ROT(M, RL)                                                                  \
  hipLaunchKernelGGL((seg_attn_bf16_pp<true, RL, 1, M>), dim3((unsigned)blocks), dim3(512), 0, s,    \
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,              \
                     (const uint16_t*)a.k_ver, (const uint16_t*)a.v_ver, a.item_desc, a.tiles,      \
                     a.order, a.tok_drop, a.ver_src, (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale,    \
                     a.tok_pos, a.rq, a.ver_run, (const float*)a.rot_tab)
#define AKV_LAUNCH_PARTS(M)                                                                          \
  hipLaunchKernelGGL((seg_attn_bf16_pp<false, AKV_ROPE_HALF, 1, M>), dim3((unsigned)blocks), dim3(512), 0, s, \
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,              \
                     (const uint16_t*)a.k_ver, (const uint16_t*)a.v_ver, a.item_desc, a.tiles,      \
                     a.order, a.tok_drop, a.ver_src, (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale,    \
                     a.tok_pos, a.rq, nullptr, nullptr)
    if (a.fused && a.n_runs > 0) {  // the (cos, sin) of every run, for the staging-time rotation
      const long long n = a.n_runs * (a.d / 2);
      hipLaunchKernelGGL(rot_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.run_delta, a.n_runs,
                         a.d / 2, a.rq, a.rot_tab);
    }
    if (a.bq != 64) {  // query tiles of 64 * 8 / grp tokens: the ping-pong pipeline with 8 / grp parts
      if (grp * a.bq != 512) return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs bq == 64 * 8 / (hq / hkv)");
      if (a.fused) {
        const bool half = a.rq.layout == AKV_ROPE_HALF;
        switch (grp) {
          case 4:
            if (half) AKV_LAUNCH_PARTS_ROT(2, AKV_ROPE_HALF);
            else AKV_LAUNCH_PARTS_ROT(2, AKV_ROPE_INTERLEAVED);
            break;
          case 2:
            if (half) AKV_LAUNCH_PARTS_ROT(4, AKV_ROPE_HALF);
            else AKV_LAUNCH_PARTS_ROT(4, AKV_ROPE_INTERLEAVED);
            break;
          case 1:
            if (half) AKV_LAUNCH_PARTS_ROT(8, AKV_ROPE_HALF);
            else AKV_LAUNCH_PARTS_ROT(8, AKV_ROPE_INTERLEAVED);
            break;
          default: return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs bq == 64 * 8 / (hq / hkv)");
        }
      } else {
        switch (grp) {
          case 4: AKV_LAUNCH_PARTS(2); break;
          case 2: AKV_LAUNCH_PARTS(4); break;
          case 1: AKV_LAUNCH_PARTS(8); break;
          default: return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs bq == 64 * 8 / (hq / hkv)");
        }
      }
    } else switch (grp) {
      case 1: AKV_LAUNCH_BF16(1); break;
      case 2: AKV_LAUNCH_BF16(2); break;
      case 4:
        if (a.hkv % 2 == 0) {  // two kv heads per workgroup: the ping-pong pipeline
          hipLaunchKernelGGL((seg_attn_bf16_pp<false, AKV_ROPE_HALF, 2>), dim3((unsigned)(blocks / 2)), dim3(512), 0, s,
                             (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                             (const uint16_t*)a.k_ver, (const uint16_t*)a.v_ver, a.item_desc, a.tiles, a.order,
                             a.tok_drop, a.ver_src, (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale, a.tok_pos, a.rq,
                             nullptr, nullptr);
        } else {
          AKV_LAUNCH_BF16(4);
        }
        break;
      case 8:
        if (a.fused) {
          auto kern = a.rq.layout == AKV_ROPE_HALF ? seg_attn_bf16_pp<true, AKV_ROPE_HALF>
                                                   : seg_attn_bf16_pp<true, AKV_ROPE_INTERLEAVED>;
          hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), 0, s, (const uint16_t*)a.q,
                             (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.k_ver,
                             (const uint16_t*)a.v_ver, a.item_desc, a.tiles, a.order, a.tok_drop, a.ver_src,
                             (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale, a.tok_pos, a.rq, a.ver_run,
                             (const float*)a.rot_tab);
        } else {
          hipLaunchKernelGGL(seg_attn_bf16_pp<false>, dim3((unsigned)blocks), dim3(512), 0, s, (const uint16_t*)a.q,
                             (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.k_ver,
                             (const uint16_t*)a.v_ver, a.item_desc, a.tiles, a.order, a.tok_drop, a.ver_src,
                             (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale, a.tok_pos, a.rq, nullptr, nullptr);
        }
        break;
      default:
        return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs hq/hkv in {1, 2, 4, 8}");
    }
#undef AKV_LAUNCH_BF16
#undef AKV_LAUNCH_PARTS
#undef AKV_LAUNCH_PARTS_ROT
  } else {
    const long long blocks = a.n_items * a.hq;
    if (blocks > 0x7fffffffLL) return fail(AKV_EINVAL, "too many work items");
    const int threads = ((a.bq + 63) / 64) * 64;
#define AKV_LAUNCH_F32(DD)                                                                           \
  hipLaunchKernelGGL(seg_attn_f32<DD>, dim3((unsigned)blocks), dim3(threads), 0, s,                 \
                     (const float*)a.q, (const float*)a.k, (const float*)a.v,                       \
                     (const float*)a.k_ver, (const float*)a.v_ver, a.item_desc, a.tiles, a.order,   \
                     a.tok_drop, a.ver_src, (float*)a.out, a.lse, a.hq, a.hkv, a.bk, a.scale,       \
                     a.tok_pos, a.rq)
    switch (a.d) {
      case 32: AKV_LAUNCH_F32(32); break;
      case 64: AKV_LAUNCH_F32(64); break;
      case 128: AKV_LAUNCH_F32(128); break;
      default: return fail(AKV_EUNSUPPORTED, "f32 segment attention needs d in {32, 64, 128}");
    }
#undef AKV_LAUNCH_F32
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("segment attention launch: ") + hipGetErrorString(e));
  return AKV_OK;
}

}  // namespace akv
