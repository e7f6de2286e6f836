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
// bf16 kernel (gfx950, wave64, MFMA 32x32x16 bf16):
//   * one workgroup = one work item (stretch, 64-token q-tile) x one kv head; its
//     GROUP waves are the GROUP query heads sharing that kv head, so each K/V tile
//     staged in LDS feeds GROUP x 64 query rows;
//   * per key tile of 64: S^T = K Q^T (keys on MFMA rows, queries on columns), so a
//     lane holds 32 scores of one query column and the running max / sum are
//     per-lane values plus one cross-half exchange (v_permlane32_swap);
//   * P^T stays in registers in exactly the layout the second MFMA wants as its B
//     operand; O^T = V^T P^T takes V^T from the row-major V tile through the
//     transposing LDS read ds_read_b64_tr_b16 (lane i of a 16-lane group gets
//     element i of 4 consecutive rows);
//   * the plan's tile list skips EMPTY tiles, FULL tiles run unmasked, PARTIAL
//     tiles build the mask from per-key (token, drop) pairs staged in LDS;
//   * blockIdx -> (item, kv head) puts consecutive workgroups on different kv heads,
//     so with 8 kv heads each XCD's L2 streams a single head's K/V.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "internal.h"

namespace akv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 64;    // head dim
constexpr int BQ = 64;   // query tokens per work item (= 2 MFMA column blocks)
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

__device__ __forceinline__ bf16x8 cat4(s16x4 a, s16x4 b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Running-max slack (log2 units): the accumulators are rescaled only when a new
// score exceeds the running max by more than this, so exp2 arguments stay <= 8
// (p <= 256, exact in fp32, no bf16 overflow) and most tiles skip the rescale.
constexpr float kRescaleSlack = 8.0f;

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

template <int GROUP>
__global__ __launch_bounds__(64 * GROUP) void seg_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ kver, const uint16_t* __restrict__ vver,
    const int* __restrict__ item_desc, const int* __restrict__ tiles, const int* __restrict__ order,
    const int* __restrict__ tok_drop, const int* __restrict__ ver_src, uint16_t* __restrict__ out,
    float* __restrict__ lse, int hq, int hkv, float scale) {
  constexpr int NT = 64 * GROUP;            // threads
  constexpr int CPT = (BK * 8 + NT - 1) / NT;  // 16-byte K (and V) chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t lk[2][BK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2][BK * VP];
  __shared__ int mtok[2][BK], mdrop[2][BK];

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

  // Q^T fragments (B operand): qf[qb][ds] = Q[q0 + 32qb + lq][h][16ds + 8lg .. +8]
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tok = q0 + qb * 32 + lq;
    const uint4* src = (const uint4*)(q + ((long long)tok * hq + h) * D);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tok < q1) x = src[ds * 2 + lg];
      qf[qb][ds] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // global -> register staging of one K/V tile (+ mask metadata), then -> LDS buffer
  uint4 kx[CPT], vx[CPT];
  int mt = INT_MAX, md = INT_MIN;
  auto fetch = [&](int ent) {
    const TileSrc ts = tile_src(ent, nvt, voff, r, tb, te, k, v, kver, vver);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + j * NT;
      const int key = c >> 3, ch = c & 7;
      kx[j] = make_uint4(0, 0, 0, 0);
      vx[j] = make_uint4(0, 0, 0, 0);
      if (c < BK * 8 && key < ts.nrows) {
        const long long off = ((long long)(ts.row0 + key) * hkv + hk) * D + ch * 8;
        kx[j] = *(const uint4*)(ts.k + off);
        vx[j] = *(const uint4*)(ts.v + off);
      }
    }
    if ((ent & 3) == AKV_TILE_PARTIAL && threadIdx.x < BK) {
      const int key = threadIdx.x;
      mt = INT_MAX;
      md = INT_MIN;
      if (key < ts.nrows) {
        mt = ts.ver ? -1 : ts.row0 + key;
        md = tok_drop[ts.ver ? ver_src[ts.row0 + key] : ts.row0 + key];
      }
    }
  };
  auto stash = [&](int buf, int ent) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + j * NT;
      if (c < BK * 8) {
        const int key = c >> 3, ch = c & 7;
        *(uint4*)(&lk[buf][key * KP + ch * 8]) = kx[j];
        *(uint4*)(&lv[buf][key * VP + ch * 8]) = vx[j];
      }
    }
    if ((ent & 3) == AKV_TILE_PARTIAL && threadIdx.x < BK) {
      mtok[buf][threadIdx.x] = mt;
      mdrop[buf][threadIdx.x] = md;
    }
  };

  f32x16 o[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
  float ms[2] = {-INFINITY, -INFINITY};  // running max, already scaled to log2 units
  float lrun[2] = {0.f, 0.f};

  if (t0 < t1) {
    fetch(tiles[t0]);
    stash(0, tiles[t0]);
  }
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const int ent = tiles[t];
    const bool has_next = t + 1 < t1;
    const int ent_next = has_next ? tiles[t + 1] : 0;
    if (has_next) fetch(ent_next);  // in flight while this tile computes

    const uint16_t* lkb = lk[buf];
    const uint16_t* lvb = lv[buf];
    // S^T[key][q]: s[kb][qb][i] is key 32kb + 8(i/4) + 4lg + i%4, query 32qb + lq
    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(lkb + (kb * 32 + lq) * KP + ds * 16 + lg * 8);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }
    if ((ent & 3) == AKV_TILE_PARTIAL) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int tok = q0 + qb * 32 + lq;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
            if (!(mtok[buf][key] <= tok && tok < mdrop[buf][key])) s[kb][qb][i] = -INFINITY;
          }
      }
    }

    // online softmax in log2 units with a lazily rescaled running max
    bf16x8 pb[2][2][2];  // [kb][qb][half]: P^T B operand
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = xhalf_max(mx) * sl2;
      const bool grow = mx > ms[qb] + kRescaleSlack;
      if (__any(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(ms[qb] - mx) : 1.f;
        ms[qb] = grow ? mx : ms[qb];
        lrun[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
      }
      const float msub = (ms[qb] == -INFINITY) ? 0.f : ms[qb];
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][i], sl2, -msub));
          s[kb][qb][i] = p;
          sum += p;
        }
      lrun[qb] += xhalf_sum(sum);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[kb][qb][hf][j] = (__bf16)s[kb][qb][8 * hf + j];
    }

    // O^T[d][q] += V^T[d][key] P^T[key][q]
    const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int key = kb * 32 + 16 * hf + 4 * (G >> 1) + (i16 >> 2);
          const int dc = db * 32 + 16 * (G & 1) + 4 * (i16 & 3);
          const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lvb + key * VP + dc));
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lvb + (key + 8) * VP + dc));
          const bf16x8 a = cat4(r0, r1);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][qb][hf], o[qb][db], 0, 0, 0);
        }

    if (has_next) stash(buf ^ 1, ent_next);
    __syncthreads();  // next buffer written; this buffer's readers done
  }

  // epilogue: O^T[d][q] / l -> out[q][h][d]; o[qb][db][i] is d = 32db + 8(i/4) + 4lg + i%4
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tok = q0 + qb * 32 + lq;
    if (tok >= q1) continue;
    const float inv = 1.f / lrun[qb];
    uint16_t* dst = out + ((long long)tok * hq + h) * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * lg;
        const __bf16 b0 = (__bf16)(o[qb][db][4 * j] * inv), b1 = (__bf16)(o[qb][db][4 * j + 1] * inv);
        const __bf16 b2 = (__bf16)(o[qb][db][4 * j + 2] * inv), b3 = (__bf16)(o[qb][db][4 * j + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *(uint2*)(dst + d0) = w;
      }
    // natural-log sum of exp(scale * score) = (ms + log2 l) / log2 e
    if (lse && lg == 0) lse[(long long)tok * hq + h] = (ms[qb] + __log2f(lrun[qb])) / kLog2e;
  }
}

// float32 path: one thread per (query token, head), keys walked one at a time
// with an exact online softmax.  For small problems and fp32 checks.
template <int DD>
__global__ __launch_bounds__(256) void seg_attn_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ kver, const float* __restrict__ vver, const int* __restrict__ item_desc,
    const int* __restrict__ tiles, const int* __restrict__ order, const int* __restrict__ tok_drop,
    const int* __restrict__ ver_src, float* __restrict__ out, float* __restrict__ lse, int hq,
    int hkv, int bk, float scale) {
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
                     a.order, a.tok_drop, a.ver_src, (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.scale)
    switch (grp) {
      case 1: AKV_LAUNCH_BF16(1); break;
      case 2: AKV_LAUNCH_BF16(2); break;
      case 4: AKV_LAUNCH_BF16(4); break;
      default: AKV_LAUNCH_BF16(8); break;
    }
#undef AKV_LAUNCH_BF16
  } else {
    const long long blocks = a.n_items * a.hq;
    if (blocks > 0x7fffffffLL) return fail(AKV_EINVAL, "too many work items");
    const int threads = ((a.bq + 63) / 64) * 64;
#define AKV_LAUNCH_F32(DD)                                                                           \
  hipLaunchKernelGGL(seg_attn_f32<DD>, dim3((unsigned)blocks), dim3(threads), 0, s,                 \
                     (const float*)a.q, (const float*)a.k, (const float*)a.v,                       \
                     (const float*)a.k_ver, (const float*)a.v_ver, a.item_desc, a.tiles, a.order,   \
                     a.tok_drop, a.ver_src, (float*)a.out, a.lse, a.hq, a.hkv, a.bk, a.scale)
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
