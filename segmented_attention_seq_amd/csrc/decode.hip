// Decode attention over a gathered active cache, split over the key axis.
//
// "Cache Engineering for Agents" review: decode reads only the active cache, so a
// drop cuts the KV read and the attention work of every later step (serving
// results, Fig. 12, App. A.4.1); drop/repos work at page size 1 (explainer
// section 4), i.e. a request's active cache is an arbitrary list of pool slots.
//
// HBM-bound: every gathered K and V row (1 KiB per token over 8 kv heads) is read
// once.  Kernel 1 runs one workgroup per CU (kDecodeWGs).  The batch's gathered
// keys, all requests back to back (N = indptr[batch]), are cut into kDecodeWGs
// equal ranges: workgroup w takes keys [ceil(wN/P), ceil((w+1)N/P)), so every CU
// streams the same number of rows whatever the request lengths.  A range that
// crosses request boundaries yields one partial (max, sum, unnormalised output)
// per request it touches; partial (w, b) is stored in slot w + b, which is unique
// because the (workgroup, request) overlaps form a monotone staircase.  Within a
// workgroup, wave g handles kv head g, so the 8 waves stream the same 1 KiB pool
// rows together; the range's index list is staged once in LDS.  Per step of 32
// keys a wave loads the K rows straight into MFMA A operands (16 B per lane),
// computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (query heads of the group on
// the 16 columns), runs the online softmax, stages the V rows in LDS and reads
// them back transposed (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T.
// Three steps ahead are in flight in a four-deep register ring (one workgroup per
// CU leaves the registers for it).  Kernel 2 merges each (request, query head)'s
// partials.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "internal.h"

namespace akv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 64;
constexpr int IDX = 4096;    // gathered indices staged in LDS per piece of a workgroup's range
constexpr int STEP = 32;     // keys per inner step
constexpr int VP = 80;       // LDS V row pitch (bf16): 160 B
constexpr int HG = 8;        // kv heads per workgroup (one wave each)
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

// First key of workgroup w's range: ceil(w * n / p).
__device__ __forceinline__ long long range_begin(long long w, long long n, long long p) { return (w * n + p - 1) / p; }

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

struct WaveDecode {
  bf16x8 qf[2];  // Q^T B operand: column = query head lane%16 of the group, rows d = 32ds + 8(lane/16) + 0..7
  f32x4 o[4];    // O^T: o[db][r] is d = 16db + 4(lane/16) + r for query head lane%16
  float m, lsum; // running max (raw score units) and sum
};

// One step of 32 keys [base, base + 32) of the staged piece (n keys): QK, online
// softmax, PV.  Keys at or past n are masked (their rows were not loaded).
__device__ __forceinline__ void decode_step(WaveDecode& st, const StepRows& cur, uint16_t* lv, int base, int n,
                                            float sl2, int lane) {
  const int G = lane >> 4;
#pragma unroll
  for (int c = 0; c < 4; ++c) *(uint4*)(lv + (lane >> 1) * VP + 32 * (lane & 1) + 8 * c) = cur.vx[c];
  // S^T[key][q]: s[kb][r] is key 16kb + 4G + r, query head lane%16
  f32x4 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.ka[kb][ds]), st.qf[ds], s[kb],
                                                      0, 0, 0);
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
  const float mnew = fmaxf(st.m, mx);  // finite: key base+0 is valid
  const float alpha = exp2f((st.m - mnew) * sl2);
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
  st.lsum = st.lsum * alpha + sum;
  st.m = mnew;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[db][r] *= alpha;
  lds_sync();  // V rows visible to every lane of this wave
  // O^T[d][q] += V^T[d][key] P^T[key][q]; slots 8G + j: keys 4G + j (j < 4), 16 + 4G + j - 4
  const int i16 = lane & 15;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int key = 4 * G + (i16 >> 2);
    const int dc = 16 * db + 4 * (i16 & 3);
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + key * VP + dc));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lv + (key + 16) * VP + dc));
    st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat4(r0, r1), pb, st.o[db], 0, 0, 0);
  }
  lds_sync();  // this step's LDS reads done before the next step's writes
}

// Kernel 1.  grid (kDecodeWGs, ceil(hkv / 8)), exactly; wave g of workgroup (w, y) handles
// kv head 8y + g over workgroup w's key range.
__global__ __launch_bounds__(64 * HG) void decode_split(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const int* __restrict__ indptr,
                                                        const int* __restrict__ indices, int batch, int hq,
                                                        int hkv, float sl2, float* __restrict__ ws) {
  __shared__ int sidx[IDX];
  __shared__ __attribute__((aligned(16))) uint16_t lvs[HG][STEP * VP];
  __shared__ int s_first;
  // the grid is always kDecodeWGs wide: with a power-of-two constant the range
  // bounds take shifts instead of a branching 64-bit division
  static_assert((kDecodeWGs & (kDecodeWGs - 1)) == 0, "kDecodeWGs must be a power of two");
  constexpr long long P = kDecodeWGs;
  const long long w = blockIdx.x;
  // The request bounds of the first blockDim requests are read together with N,
  // so finding the range's first request costs no round trip of its own.
  const int t = threadIdx.x;
  const int tc = t < batch ? t : batch;  // clamped, so the loads need no branch
  const int ip0 = indptr[tc], ip1 = indptr[tc < batch ? tc + 1 : batch];
  const long long N = indptr[batch];
  const long long r0 = range_begin(w, N, P), r1 = range_begin(w + 1, N, P);
  const int grp = hq / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.y * HG + wave;
  const bool active = g < hkv;  // waves past hkv still take part in the barriers
  uint16_t* lv = lvs[wave];
  const int qj = lane & 15, G = lane >> 4;
  // First request with a key in the range: the one b with indptr[b] <= r0 <
  // indptr[b + 1] (r0 < N = indptr[batch]; indptr is nondecreasing from 0).
  if (t < batch && ip0 <= r0 && r0 < ip1) s_first = t;
  for (int t0 = blockDim.x; t0 < batch; t0 += blockDim.x) {
    const int u = t0 + t;
    if (u < batch && indptr[u] <= r0 && r0 < indptr[u + 1]) s_first = u;
  }
  __syncthreads();
  if (r0 >= r1) return;  // uniform: fewer keys than workgroups (after the barrier, so the
                         // bound loads above are issued with N's)
  const int first = s_first;
  const int lo = first < 0 ? 0 : first < batch ? first : batch - 1;  // bounded for malformed indptr too
  for (int b = lo; b < batch; ++b) {
    const long long rb = indptr[b], re = indptr[b + 1];
    if (rb >= r1) break;
    const long long s0 = rb > r0 ? rb : r0, e0 = re < r1 ? re : r1;
    if (s0 >= e0) continue;  // a request with no keys (invalid input) or no overlap
    WaveDecode st;
    if (active) {
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qj < grp) x = *(const uint4*)(q + ((long long)b * hq + g * grp + qj) * D + 32 * ds + 8 * G);
        st.qf[ds] = __builtin_bit_cast(bf16x8, x);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      st.lsum = 0.f;
    }
    for (long long p0 = s0; p0 < e0; p0 += IDX) {
      const int n = (int)((e0 - p0) < IDX ? (e0 - p0) : IDX);
      __syncthreads();  // earlier readers of sidx are done
      // eight index loads per thread in flight before the first LDS write (a loop
      // storing each load before the next waits out one round trip per pass)
      for (int i0 = threadIdx.x; i0 < n; i0 += 8 * blockDim.x) {
        int ix[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i0 + j * (int)blockDim.x;
          ix[j] = indices[p0 + (i < n ? i : n - 1)];  // clamped, so the loads need no branch
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i0 + j * (int)blockDim.x;
          if (i < n) sidx[i] = ix[j];
        }
      }
      __syncthreads();
      if (!active) continue;
      // four-deep ring: steps base .. base + 96 in flight while base computes
      StepRows r[4];
      load_step(r[0], k, v, sidx, 0, n, g, hkv, lane);
      load_step(r[1], k, v, sidx, STEP, n, g, hkv, lane);
      load_step(r[2], k, v, sidx, 2 * STEP, n, g, hkv, lane);
      for (int base = 0; base < n; base += 4 * STEP) {
        load_step(r[3], k, v, sidx, base + 3 * STEP, n, g, hkv, lane);
        decode_step(st, r[0], lv, base, n, sl2, lane);
        load_step(r[0], k, v, sidx, base + 4 * STEP, n, g, hkv, lane);
        if (base + STEP < n) decode_step(st, r[1], lv, base + STEP, n, sl2, lane);
        load_step(r[1], k, v, sidx, base + 5 * STEP, n, g, hkv, lane);
        if (base + 2 * STEP < n) decode_step(st, r[2], lv, base + 2 * STEP, n, sl2, lane);
        load_step(r[2], k, v, sidx, base + 6 * STEP, n, g, hkv, lane);
        if (base + 3 * STEP < n) decode_step(st, r[3], lv, base + 3 * STEP, n, sl2, lane);
      }
    }
    if (active && qj < grp) {
      // partial slot w + b: o[db][r] is d = 16db + 4G + r (unnormalised), max in raw score units
      float* part = ws + (((w + b) * hkv + g) * grp + qj) * (long long)(D + 2);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *(float4*)(part + 16 * db + 4 * G) = make_float4(st.o[db][0], st.o[db][1], st.o[db][2], st.o[db][3]);
      if (G == 0) {
        part[D] = st.m;
        part[D + 1] = st.lsum;
      }
    }
  }
}

// Kernel 2: merge of one (request, query head)'s partials, slots w + b for the
// workgroups w whose ranges hold keys of request b.  The 64 lanes read the
// partials' (max, sum) in parallel, reduce the max across the wave, then every
// lane (one per output dim) accumulates the rescaled partial outputs.
__global__ __launch_bounds__(64) void decode_merge(const float* __restrict__ ws, const int* __restrict__ indptr,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse, int batch,
                                                   int hq, int hkv, int wgs, float scale, float sl2) {
  __shared__ float wgt[kDecodeWGs + 1];
  const int b = blockIdx.x / hq, h = blockIdx.x % hq;
  const int grp = hq / hkv, g = h / grp, j = h % grp;
  const int lane = threadIdx.x;
  const long long P = wgs, N = indptr[batch];
  const long long rb = indptr[b], re = indptr[b + 1];
  if (N <= 0 || re <= rb) {  // a request with no keys: attention over nothing is undefined
    out[((long long)b * hq + h) * D + lane] = 0x7FC0;  // bf16 quiet NaN
    if (lse && lane == 0) lse[(long long)b * hq + h] = -INFINITY;  // log of an empty sum
    return;
  }
  const long long w0 = rb * P / N, w1 = (re - 1) * P / N;  // workgroups holding the first and last key
  const int cnt = (int)(w1 - w0 + 1);
  const long long stride = (long long)hkv * grp * (D + 2);
  const float* base = ws + ((w0 + b) * hkv * grp + (long long)g * grp + j) * (D + 2);
  const float* po = base + lane;
  // The partial outputs of the first PF slots are requested first, so their latency
  // overlaps the (max, sum) loads and reductions; lane s reads slot s's (max, sum).
  constexpr int PF = 32;
  float pv[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) pv[s] = s < cnt ? po[s * stride] : 0.f;
  float ms[(kDecodeWGs + 64) / 64], lsv[(kDecodeWGs + 64) / 64];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < (kDecodeWGs + 64) / 64; ++k) {
    const int s = lane + 64 * k;
    ms[k] = -INFINITY;
    lsv[k] = 0.f;
    if (s < cnt) {
      const long long w = w0 + s;
      if (range_begin(w, N, P) < range_begin(w + 1, N, P)) {  // empty ranges wrote nothing
        ms[k] = base[s * stride + D];
        lsv[k] = base[s * stride + D + 1];
      }
    }
    M = fmaxf(M, ms[k]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < (kDecodeWGs + 64) / 64; ++k) {
    const int s = lane + 64 * k;
    const float wt = ms[k] > -INFINITY ? exp2f((ms[k] - M) * sl2) : 0.f;
    if (s < cnt) wgt[s] = wt;
    L = fmaf(wt, lsv[k], L);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    const float wt = s < cnt ? wgt[s] : 0.f;
    if (wt != 0.f) acc = fmaf(wt, pv[s], acc);  // stale slots (weight 0) may hold anything
  }
  for (int s = PF; s < cnt; ++s) {
    const float wt = wgt[s];
    if (wt != 0.f) acc = fmaf(wt, po[s * stride], acc);
  }
  out[((long long)b * hq + h) * D + lane] = __builtin_bit_cast(uint16_t, (__bf16)(acc / L));
  if (lse && lane == 0) lse[(long long)b * hq + h] = M * scale + logf(L);
}

// Scratch for callers that cannot allocate (akv_decode_attention_noalloc): one
// fixed array per device, found through hipGetSymbolAddress (in host code the
// array's name is only a stand-in for the symbol, never a device address).
constexpr uint64_t kStaticScratchFloats = 4ull << 20;  // 16 MiB
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kStaticScratchFloats];
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int decode_static_scratch(float** ptr, uint64_t* floats) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AKV_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(AKV_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = (float*)p;
  }
  *ptr = g_scratch_ptr[dev];
  *floats = kStaticScratchFloats;
  return AKV_OK;
}

uint64_t decode_ws_floats(int32_t batch, int32_t hq, int32_t d) {
  return ((uint64_t)kDecodeWGs + (uint64_t)batch) * hq * (uint64_t)(d + 2);
}

int launch_decode(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const float sl2 = a.scale * kLog2e;
  const int waves = a.hkv < HG ? a.hkv : HG;
  hipLaunchKernelGGL(decode_split, dim3(kDecodeWGs, (a.hkv + HG - 1) / HG), dim3(64 * waves), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.indptr, a.indices,
                     a.batch, a.hq, a.hkv, sl2, a.ws);
  hipLaunchKernelGGL(decode_merge, dim3(a.batch * a.hq), dim3(64), 0, s, (const float*)a.ws, a.indptr,
                     (uint16_t*)a.out, a.lse, a.batch, a.hq, a.hkv, kDecodeWGs, a.scale, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("decode launch: ") + hipGetErrorString(e));
  return AKV_OK;
}

}  // namespace akv
