// Decode attention over a gathered active cache, split over the key axis.
//
// "Cache Engineering for Agents" review: decode reads only the active cache, so a
// drop cuts the KV read and the attention work of every later step (serving
// results, Fig. 12, App. A.4.1); drop/repos work at page size 1 (explainer
// section 4), i.e. a request's active cache is an arbitrary list of pool slots.
//
// HBM-bound: every gathered K and V row (1 KiB per token over 8 kv heads) is read
// once.  Kernel 1: one workgroup per (request, key chunk of 256-2048), one wave per
// kv head.  Per step of
// 32 keys it loads the K rows straight into MFMA A operands (16 B per lane),
// computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (query heads of the group on
// the 16 columns), runs the online softmax, stages the V rows in LDS and reads
// them back transposed (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T.
// The next step's rows are loaded while the current one computes.  Kernel 2
// merges the per-chunk (max, sum, acc) partials.
#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"

namespace akv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 64;
constexpr int CHUNK = 2048;  // largest key chunk per workgroup (LDS index staging)
constexpr int STEP = 32;     // keys per inner step
constexpr int VP = 80;       // LDS V row pitch (bf16): 160 B
constexpr float kLog2e = 1.4426950408889634f;

// One-wave blocks: LDS accesses of a wave complete in order, so waiting for this
// wave's own LDS traffic orders a write before other lanes' reads without a
// workgroup barrier, and unlike __syncthreads it leaves the prefetched global
// loads in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bf16x8 cat4(s16x4 a, s16x4 b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

struct StepRows {
  uint4 ka[2][2];  // [kb][ds]: K[key 16kb + lane%16][32ds + 8(lane/16) .. +8]
  uint4 vx[4];     // V[key lane/2][32(lane%2) + 8c .. +8]
};

__device__ __forceinline__ void load_step(StepRows& sr, const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v, const int* sidx, int base,
                                          int n, int g, int hkv, int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = base + kb * 16 + (lane & 15);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) sr.ka[kb][ds] = make_uint4(0, 0, 0, 0);
    if (key < n) {
      const uint16_t* row = k + ((long long)sidx[key] * hkv + g) * D + 8 * (lane >> 4);
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) sr.ka[kb][ds] = *(const uint4*)(row + 32 * ds);
    }
  }
  const int vkey = base + (lane >> 1);
#pragma unroll
  for (int c = 0; c < 4; ++c) sr.vx[c] = make_uint4(0, 0, 0, 0);
  if (vkey < n) {
    const uint16_t* row = v + ((long long)sidx[vkey] * hkv + g) * D + 32 * (lane & 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) sr.vx[c] = *(const uint4*)(row + 8 * c);
  }
}

// One workgroup per (request, key chunk): wave w handles kv head w over the same
// chunk, so the 8 waves stream the same 1 KiB pool rows together (each row read
// as one contiguous burst) and share the chunk's staged index list.
__global__ __launch_bounds__(512) void decode_split(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    const int* __restrict__ indptr,
                                                    const int* __restrict__ indices, int hq, int hkv,
                                                    int splits, int chunk, float sl2, float* __restrict__ ws) {
  __shared__ int sidx[CHUNK];
  __shared__ __attribute__((aligned(16))) uint16_t lvs[8][STEP * VP];
  const int split = blockIdx.x, b = blockIdx.y;
  const int grp = hq / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int beg = indptr[b], end = indptr[b + 1];
  const int k0 = beg + split * chunk;
  const int n = min(end - k0, chunk);
  for (int i = threadIdx.x; i < n; i += blockDim.x) sidx[i] = indices[k0 + i];
  __syncthreads();
  for (int g = wave; g < hkv; g += blockDim.x >> 6) {
    uint16_t* lv = lvs[wave];
    float* part = ws + (((long long)b * hkv + g) * splits + split) * (long long)grp * (D + 2);
    float* pm = part + grp * D;
    float* pl = pm + grp;
    if (n <= 0) {
      if (lane < grp) { pm[lane] = -INFINITY; pl[lane] = 0.f; }
      continue;
    }
    // Q^T B operand: column = query head j = lane%16 of the group, rows d = 32ds + 8(lane/16) + 0..7
    const int qj = lane & 15, G = lane >> 4;
    bf16x8 qf[2];
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qj < grp) x = *(const uint4*)(q + ((long long)b * hq + g * grp + qj) * D + 32 * ds + 8 * G);
      qf[ds] = __builtin_bit_cast(bf16x8, x);
    }

    f32x4 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    StepRows cur, nxt;
    load_step(cur, k, v, sidx, 0, n, g, hkv, lane);
    for (int base = 0; base < n; base += STEP) {
      if (base + STEP < n) load_step(nxt, k, v, sidx, base + STEP, n, g, hkv, lane);
      // stage V rows of this step
#pragma unroll
      for (int c = 0; c < 4; ++c) *(uint4*)(lv + (lane >> 1) * VP + 32 * (lane & 1) + 8 * c) = cur.vx[c];
      // S^T[key][q]: s[kb][r] is key 16kb + 4G + r, query head qj
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 2; ++ds)
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.ka[kb][ds]),
                                                          qf[ds], s[kb], 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (base + 16 * kb + 4 * G + r >= n) s[kb][r] = -INFINITY;
          mx = fmaxf(mx, s[kb][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx);  // finite: key base+0 is valid
      const float alpha = exp2f((m - mnew) * sl2);
      const float msub = mnew * sl2;
      float sum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(fmaf(s[kb][r], sl2, -msub));
          sum += p;
          pb[4 * kb + r] = (__bf16)p;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      lsum = lsum * alpha + sum;
      m = mnew;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      lds_sync();  // V rows visible to every lane of this wave
      // O^T[d][q] += V^T[d][key] P^T[key][q]; slots 8G + j: keys 4G + j (j < 4), 16 + 4G + j - 4
      const int i16 = lane & 15;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int key = 4 * G + (i16 >> 2);
        const int dc = 16 * db + 4 * (i16 & 3);
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + key * VP + dc));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + (key + 16) * VP + dc));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat4(r0, r1), pb, o[db], 0, 0, 0);
      }
      lds_sync();  // this step's LDS reads done before the next step's writes
      cur = nxt;
    }
    // partial: o[db][r] is d = 16db + 4G + r for query head qj (unnormalised), max in raw score units
    if (qj < grp) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *(float4*)(part + qj * D + 16 * db + 4 * G) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
      if (G == 0) { pm[qj] = m; pl[qj] = lsum; }
    }
  }
}

// Merge of the per-chunk partials of one (request, query head): the 64 lanes read
// the chunks' (max, sum) in parallel, reduce the max across the wave, then every
// lane (one per output dim) accumulates the rescaled chunk outputs.
__global__ __launch_bounds__(64) void decode_merge(const float* __restrict__ ws, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse, int hq, int hkv, int splits,
                                                   float scale, float sl2) {
  __shared__ float wgt[1024];
  const int b = blockIdx.x / hq, h = blockIdx.x % hq;
  const int grp = hq / hkv, g = h / grp, j = h % grp;
  const int lane = threadIdx.x;
  const long long stride = (long long)grp * (D + 2);
  const float* base = ws + ((long long)b * hkv + g) * splits * stride;
  float M = -INFINITY;
  for (int s = lane; s < splits; s += 64) {
    const float* p = base + s * stride;
    if (p[grp * D + grp + j] > 0.f) M = fmaxf(M, p[grp * D + j]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  for (int s = lane; s < splits; s += 64) {
    const float* p = base + s * stride;
    const float ls = p[grp * D + grp + j];
    const float w = ls > 0.f ? exp2f((p[grp * D + j] - M) * sl2) : 0.f;
    wgt[s] = w;
    L = fmaf(w, ls, L);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
  __syncthreads();
  float acc = 0.f;
  const float* po = base + j * D + lane;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float w = wgt[s];
    if (w != 0.f) acc = fmaf(w, po[s * stride], acc);
  }
  out[((long long)b * hq + h) * D + lane] = __builtin_bit_cast(uint16_t, (__bf16)(acc / L));
  if (lse && lane == 0) lse[(long long)b * hq + h] = M * scale + logf(L);
}

}  // namespace

// Key chunk per workgroup: the largest power of two in [256, CHUNK] that still
// yields two rounds of workgroups over the 256 CUs for this batch (long chunks
// amortise the index staging and keep the merge short; short ones fill the GPU
// when the batch is small), and never more than 1024 chunks per request (the
// merge's weight table).
int decode_split_plan(int32_t batch, int64_t max_n, int32_t* splits, int32_t* chunk) {
  if (batch < 1 || max_n < 1 || max_n > 1024LL * CHUNK) return AKV_EINVAL;
  int c = CHUNK;
  while (c > 256 && (int64_t)batch * ((max_n + c - 1) / c) < 2 * 256) c >>= 1;
  while ((max_n + c - 1) / c > 1024) c <<= 1;
  *chunk = c;
  *splits = (int32_t)((max_n + c - 1) / c);
  return AKV_OK;
}

uint64_t decode_ws_floats(int32_t batch, int32_t hq, int32_t d, int32_t splits) {
  return (uint64_t)batch * hq * splits * (uint64_t)(d + 2);
}

int launch_decode(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const float sl2 = a.scale * kLog2e;
  const int waves = a.hkv < 8 ? a.hkv : 8;
  hipLaunchKernelGGL(decode_split, dim3(a.splits, a.batch), dim3(64 * waves), 0, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.indptr, a.indices, a.hq, a.hkv,
                     a.splits, a.chunk, sl2, a.ws);
  hipLaunchKernelGGL(decode_merge, dim3(a.batch * a.hq), dim3(64), 0, s, (const float*)a.ws,
                     (uint16_t*)a.out, a.lse, a.hq, a.hkv, a.splits, a.scale, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("decode launch: ") + hipGetErrorString(e));
  return AKV_OK;
}

}  // namespace akv
