// RoPE rotation kernel: repos (key re-rotation p -> q), RoPE-apply (raw -> append
// position) and the KV-version builder (rotated key + value copy).
//
// "Cache Engineering for Agents" review, "what to keep, how to align positions"
// (§3.3): moving a cached key from position p to q multiplies it by a rotation
// matrix and leaves the value untouched; "single-prefill restore" (§4.2, App.
// A.1.1): per-segment KV versions are made by key rotation and value copy.
//
// Bandwidth-bound.  For head dims 16-128 one thread writes one 16-byte output chunk
// of one head (rope_row_kernel), so stores cover whole 128-byte head rows, and the
// (cos, sin) values are shared across a group of heads by cross-lane shuffle; other
// head dims use one thread per 8-pair chunk that walks every head of the row.
#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "rope_angle.h"

namespace akv {
namespace {

// Frequencies are stored in revolutions per position, theta_i / (2 pi), in fp64; the
// angle evaluation is shared with the attention's query load (rope_angle.h).  The
// table travels as a kernel argument sized to the kernel's head dim (N = d / 2
// entries for the row kernels): a smaller argument block is a shorter dispatch,
// which shows on the 35 us repos launches.
template <int N> struct FreqsN { double rev[N]; };
using Freqs = FreqsN<128>;

__device__ __forceinline__ void angle_cs(long long delta, double rev, float& c, float& s) {
  rope_angle_cs((double)delta, rev, c, s);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 8 consecutive elements <-> float[8]
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {  // bf16 storage
  static __device__ __forceinline__ void load(const uint16_t* p, float f[8]) {
    const uint4 u = *(const uint4*)p;
    f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
    f[4] = bf_lo(u.z); f[5] = bf_hi(u.z); f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float f[8]) {
    uint4 u;
    u.x = pack_bf16(f[0], f[1]); u.y = pack_bf16(f[2], f[3]);
    u.z = pack_bf16(f[4], f[5]); u.w = pack_bf16(f[6], f[7]);
    *(uint4*)p = u;
  }
  static __device__ __forceinline__ void copy(uint16_t* d, const uint16_t* s) { *(uint4*)d = *(const uint4*)s; }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float f[8]) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float f[8]) {
    *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
  static __device__ __forceinline__ void copy(float* d, const float* s) {
    *(float4*)d = *(const float4*)s;
    *(float4*)(d + 4) = *(const float4*)(s + 4);
  }
};

typedef unsigned rs_u32x4 __attribute__((ext_vector_type(4)));
typedef float rs_f32x4 __attribute__((ext_vector_type(4)));

// 8 elements stored as streaming (nontemporal) writes
__device__ __forceinline__ void store8_nt(uint16_t* p, const float f[8]) {
  const rs_u32x4 u = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
  __builtin_nontemporal_store(u, (rs_u32x4*)p);
}
__device__ __forceinline__ void store8_nt(float* p, const float f[8]) {
  const rs_f32x4 a = {f[0], f[1], f[2], f[3]}, b = {f[4], f[5], f[6], f[7]};
  __builtin_nontemporal_store(a, (rs_f32x4*)p);
  __builtin_nontemporal_store(b, (rs_f32x4*)(p + 4));
}

// 8 consecutive elements moved bit for bit (value rows of versions and reuse)
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  rs_u32x4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *(const rs_u32x4*)p; }
  __device__ __forceinline__ void get(float f[8]) const {
    f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
    f[4] = bf_lo(u.z); f[5] = bf_hi(u.z); f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
  }
  __device__ __forceinline__ void store(uint16_t* p) const { *(rs_u32x4*)p = u; }
  __device__ __forceinline__ void store_nt(uint16_t* p) const { __builtin_nontemporal_store(u, (rs_u32x4*)p); }
};
template <> struct Raw8<float> {
  rs_f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) { a = *(const rs_f32x4*)p; b = *(const rs_f32x4*)(p + 4); }
  __device__ __forceinline__ void get(float f[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ void store(float* p) const { *(rs_f32x4*)p = a; *(rs_f32x4*)(p + 4) = b; }
  __device__ __forceinline__ void store_nt(float* p) const {
    __builtin_nontemporal_store(a, (rs_f32x4*)p);
    __builtin_nontemporal_store(b, (rs_f32x4*)(p + 4));
  }
};

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ out, const T* __restrict__ in,
                                                   T* __restrict__ vout, const T* __restrict__ vin,
                                                   long long n_rows, int heads, int d,
                                                   const int* __restrict__ gather,
                                                   const int* __restrict__ pos_from, int from_by_src,
                                                   const int* __restrict__ pos_to, Freqs fr) {
  const int cpr = d >> 4;  // 8-pair chunks per head vector
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = tid / cpr;
  const int c = (int)(tid - row * cpr);
  if (row >= n_rows) return;
  const long long src = gather ? (long long)gather[row] : row;
  const long long delta =
      (long long)pos_to[row] - (pos_from ? (long long)pos_from[from_by_src ? src : row] : 0LL);
  float cs[8], sn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) angle_cs(delta, fr.rev[c * 8 + i], cs[i], sn[i]);

  const long long stride = (long long)heads * d;
  const T* x = in + src * stride;
  T* y = out + row * stride;
  // element offsets of the chunk's two 8-element pieces within a head vector
  int oa, ob;
  if (LAYOUT == AKV_ROPE_HALF) { oa = c * 8; ob = (d >> 1) + c * 8; }
  else { oa = c * 16; ob = c * 16 + 8; }
  for (int h = 0; h < heads; ++h) {
    float a[8], b[8], ya[8], yb[8];
    Vec8<T>::load(x + h * d + oa, a);
    Vec8<T>::load(x + h * d + ob, b);
    if (LAYOUT == AKV_ROPE_HALF) {
      // pair i = (a[i], b[i])
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ya[i] = rot_first(a[i], b[i], cs[i], sn[i]);
        yb[i] = rot_second(a[i], b[i], cs[i], sn[i]);
      }
    } else {
      // pairs are adjacent: (a[0],a[1]) .. (a[6],a[7]), (b[0],b[1]) .. (b[6],b[7])
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ya[2 * i] = rot_first(a[2 * i], a[2 * i + 1], cs[i], sn[i]);
        ya[2 * i + 1] = rot_second(a[2 * i], a[2 * i + 1], cs[i], sn[i]);
        yb[2 * i] = rot_first(b[2 * i], b[2 * i + 1], cs[i + 4], sn[i + 4]);
        yb[2 * i + 1] = rot_second(b[2 * i], b[2 * i + 1], cs[i + 4], sn[i + 4]);
      }
    }
    Vec8<T>::store(y + h * d + oa, ya);
    Vec8<T>::store(y + h * d + ob, yb);
    if (vout) {
      Vec8<T>::copy(vout + row * stride + h * d + oa, vin + src * stride + h * d + oa);
      Vec8<T>::copy(vout + row * stride + h * d + ob, vin + src * stride + h * d + ob);
    }
  }
}

// Index forms of the row kernel, fixed at compile time so that independent index
// loads issue together: apply (no gather, rotation from position 0), repos and
// reuse (gather, pos_from by output row), versions (gather, pos_from by source
// row); anything else reads the pointers at run time.
enum { IX_APPLY = 0, IX_GATHER_ROW = 1, IX_GATHER_SRC = 2, IX_ANY = 3 };

// Row form for d in {16, 32, 64, 128}: one thread per 16-byte output chunk of one
// head, so each store instruction writes whole 128-byte head rows (a group of HG
// heads x 2*CPR chunks, HG = min(8, 32 / CPR), fills G <= 64 lanes).  In the half
// layout a chunk's pairs span both halves of the head vector: the two threads that
// own chunk c of the first and of the second half both load the chunk's two input
// pieces (the second load is a cache hit) and each writes its own half.  In the
// interleaved layout a chunk holds four whole pairs.  Each thread evaluates one
// angle per row, pair (lane in group) mod d/2, and fetches the ones it needs by
// shuffle.
//
// A group handles RPW consecutive rows: the index loads of all of them are issued
// together, then all their data loads, so a wave keeps RPW rows of reads in flight
// instead of paying an index-then-data round trip per row.  Rows past the end
// repeat the last row and store nothing.
template <typename T, int LAYOUT, int CPR, int IX, int RPW>
__global__ __launch_bounds__(256) void rope_row_kernel(T* __restrict__ out, const T* __restrict__ in,
                                                       T* __restrict__ vout, const T* __restrict__ vin,
                                                       long long n_rows, int heads, int n_hg,
                                                       const int* __restrict__ gather,
                                                       const int* __restrict__ pos_from, int from_by_src,
                                                       const int* __restrict__ pos_to, FreqsN<8 * CPR> fr) {
  constexpr int LPH = 2 * CPR;                      // lanes (16-byte chunks) per head
  constexpr int HG = 32 / CPR < 8 ? 32 / CPR : 8;   // heads per group
  constexpr int G = HG * LPH;
  constexpr int D = 16 * CPR;
  // With one group per wave (G == 64) the group index is the wave's, made uniform
  // by readfirstlane, so the row indices come by scalar loads.
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long grp = G == 64 ? (long long)blockIdx.x * (blockDim.x / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)
                                : tid / G;
  const int l = G == 64 ? (int)(threadIdx.x & 63) : (int)(tid - grp * G);
  const long long rb = grp / n_hg;
  if (rb * RPW >= n_rows) return;  // whole groups leave together
  const int hg = (int)(grp - rb * n_hg);
  const int hl = l / LPH, j = l - hl * LPH;
  const int h = hg * HG + hl;
  const int hc = h < heads ? h : heads - 1;   // lanes past the last head load a real row, store nothing
  const bool second = LAYOUT == AKV_ROPE_HALF && j >= CPR;
  const int c = LAYOUT == AKV_ROPE_HALF ? (second ? j - CPR : j) : j;
  const double th = fr.rev[l % (D / 2)];
  long long row[RPW], src[RPW], delta[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    row[r] = rb * RPW + r < n_rows ? rb * RPW + r : n_rows - 1;
    if constexpr (IX == IX_APPLY) {
      src[r] = row[r];
      delta[r] = pos_to[row[r]];
    } else if constexpr (IX == IX_GATHER_ROW) {
      const int g = gather[row[r]], pt = pos_to[row[r]], pf = pos_from[row[r]];
      src[r] = g;
      delta[r] = (long long)pt - pf;
    } else if constexpr (IX == IX_GATHER_SRC) {
      const int g = gather[row[r]], pt = pos_to[row[r]];
      src[r] = g;
      delta[r] = (long long)pt - pos_from[g];
    } else {
      src[r] = gather ? (long long)gather[row[r]] : row[r];
      delta[r] = (long long)pos_to[row[r]] - (pos_from ? (long long)pos_from[from_by_src ? src[r] : row[r]] : 0LL);
    }
  }
  Raw8<T> ra[RPW], rb2[RPW], vv[RPW];   // raw rows: fewer registers than converted ones
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const long long off_in = (src[r] * heads + hc) * D;
    if (LAYOUT == AKV_ROPE_HALF) {
      ra[r].load(in + off_in + 8 * c);
      rb2[r].load(in + off_in + D / 2 + 8 * c);
    } else {
      ra[r].load(in + off_in + 8 * j);
    }
    if (vout) vv[r].load(vin + off_in + 8 * j);
  }
  const int base = (int)(threadIdx.x & 63) - l;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float mc, ms;
    angle_cs(delta[r], th, mc, ms);
    float a[8], b[8], y[8];
    ra[r].get(a);
    if (LAYOUT == AKV_ROPE_HALF) rb2[r].get(b);
    if (LAYOUT == AKV_ROPE_HALF) {
      float cs[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cs[i] = __shfl(mc, base + 8 * c + i, 64);
        sn[i] = __shfl(ms, base + 8 * c + i, 64);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        y[i] = second ? rot_second(a[i], b[i], cs[i], sn[i]) : rot_first(a[i], b[i], cs[i], sn[i]);
    } else {
      float cs[4], sn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cs[i] = __shfl(mc, base + 4 * j + i, 64);
        sn[i] = __shfl(ms, base + 4 * j + i, 64);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = rot_first(a[2 * i], a[2 * i + 1], cs[i], sn[i]);
        y[2 * i + 1] = rot_second(a[2 * i], a[2 * i + 1], cs[i], sn[i]);
      }
    }
    if (h >= heads || rb * RPW + r >= n_rows) continue;
    const long long off_out = (row[r] * heads + h) * D;
    // Gathered forms write new copies once: streaming stores, so the next kernel
    // finds no dirty lines to write back.  RoPE-apply output is read right away by
    // the attention and stays cached.
    if constexpr (IX == IX_APPLY) {
      Vec8<T>::store(out + off_out + 8 * j, y);
      if (vout) vv[r].store(vout + off_out + 8 * j);
    } else {
      store8_nt(out + off_out + 8 * j, y);
      if (vout) vv[r].store_nt(vout + off_out + 8 * j);
    }
  }
}

// Rows per group of the row kernel.
constexpr int kRowsPerGroup = 3;

template <typename T, int LAYOUT, int CPR, int IX>
void launch_row_ix(const RopeArgs& a, const Freqs& all, hipStream_t s) {
  constexpr int HG = 32 / CPR < 8 ? 32 / CPR : 8;
  constexpr int RPW = kRowsPerGroup;
  FreqsN<8 * CPR> fr;  // the head dim's d / 2 = 8 CPR frequencies
  for (int i = 0; i < 8 * CPR; ++i) fr.rev[i] = all.rev[i];
  const int n_hg = (a.heads + HG - 1) / HG;
  const long long threads = (a.n_rows + RPW - 1) / RPW * n_hg * (long long)(HG * 2 * CPR);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((rope_row_kernel<T, LAYOUT, CPR, IX, RPW>), dim3(blocks), dim3(256), 0, s, (T*)a.out,
                     (const T*)a.in, (T*)a.v_out, (const T*)a.v_in, (long long)a.n_rows, a.heads, n_hg,
                     a.gather, a.pos_from, a.pos_from_by_src ? 1 : 0, a.pos_to, fr);
}

template <typename T, int LAYOUT, int CPR>
void launch_row(const RopeArgs& a, const Freqs& fr, hipStream_t s) {
  if (!a.gather && !a.pos_from) return launch_row_ix<T, LAYOUT, CPR, IX_APPLY>(a, fr, s);
  if (a.gather && a.pos_from && !a.pos_from_by_src) return launch_row_ix<T, LAYOUT, CPR, IX_GATHER_ROW>(a, fr, s);
  if (a.gather && a.pos_from && a.pos_from_by_src) return launch_row_ix<T, LAYOUT, CPR, IX_GATHER_SRC>(a, fr, s);
  launch_row_ix<T, LAYOUT, CPR, IX_ANY>(a, fr, s);
}

template <typename T, int LAYOUT>
void launch_t(const RopeArgs& a, const Freqs& fr, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_row<T, LAYOUT, 1>(a, fr, s);
    case 32: return launch_row<T, LAYOUT, 2>(a, fr, s);
    case 64: return launch_row<T, LAYOUT, 4>(a, fr, s);
    case 128: return launch_row<T, LAYOUT, 8>(a, fr, s);
    default: break;
  }
  const long long threads = a.n_rows * (a.d / 16);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((rope_kernel<T, LAYOUT>), dim3(blocks), dim3(256), 0, s, (T*)a.out, (const T*)a.in,
                     (T*)a.v_out, (const T*)a.v_in, (long long)a.n_rows, a.heads, a.d, a.gather,
                     a.pos_from, a.pos_from_by_src ? 1 : 0, a.pos_to, fr);
}

}  // namespace

int launch_rope(const RopeArgs& a, void* stream) {
  Freqs fr;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < a.d / 2; ++i) fr.rev[i] = std::pow(a.base, -2.0 * i / a.d) / two_pi;
  for (int i = a.d / 2; i < 128; ++i) fr.rev[i] = 0.0;
  const long long threads = a.n_rows * (a.heads + 7LL) * (a.d / 8);   // bound for every form
  if ((threads + 255) / 256 > 0x7fffffffLL) return fail(AKV_EINVAL, "too many rows for one launch");
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (a.dtype == AKV_BF16) {
    if (a.layout == AKV_ROPE_HALF) launch_t<uint16_t, AKV_ROPE_HALF>(a, fr, s);
    else launch_t<uint16_t, AKV_ROPE_INTERLEAVED>(a, fr, s);
  } else {
    if (a.layout == AKV_ROPE_HALF) launch_t<float, AKV_ROPE_HALF>(a, fr, s);
    else launch_t<float, AKV_ROPE_INTERLEAVED>(a, fr, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("rope launch: ") + hipGetErrorString(e));
  return AKV_OK;
}

}  // namespace akv
