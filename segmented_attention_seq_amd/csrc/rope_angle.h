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

}  // namespace akv
