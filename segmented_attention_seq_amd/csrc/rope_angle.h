// RoPE angle evaluation shared by the RoPE kernels and the attention's query load.
//
// "Cache Engineering for Agents" review, "what to keep, how to align positions"
// (§3.3): a key or query at position p is the raw vector rotated pair by pair by
// p * theta_i, theta_i = base^(-2i/d); moving it from p to q rotates by (q - p) *
// theta_i.
//
// Frequencies are held in revolutions per position, theta_i / (2 pi), in fp64.  A
// shift delta (an integer below 2^31 in magnitude, held exactly in a double) is
// reduced to its fractional revolution in fp64 (one fma of the exact product minus
// its nearest integer, rounded once), then rounded to fp32 and given to the
// hardware sine and cosine, which take revolutions (within 1.3e-7 of the exact
// value on [-0.5, 0.5]).
#pragma once

namespace akv {

__device__ __forceinline__ void rope_angle_cs(double delta, double rev, float& c, float& s) {
  const double x = delta * rev;
  const float r = (float)fma(delta, rev, -rint(x));
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

// Pair (a, b) rotated by the angle with cosine c and sine s: first member
// a c - b s, second member a s + b c.  Every kernel that rotates keys or queries
// goes through these two, with their fused multiply-adds spelled out, so a key
// rotated while a tile is staged and one rotated into a version buffer round alike.
__device__ __forceinline__ float rot_first(float a, float b, float c, float s) { return __builtin_fmaf(a, c, -(b * s)); }
__device__ __forceinline__ float rot_second(float a, float b, float c, float s) { return __builtin_fmaf(a, s, b * c); }

}  // namespace akv
