// Rotary-embedding arithmetic shared by the streaming RoPE kernel and the
// Q-tile load of the attention kernel, so that both routes round identically.
//
// Position chain ("MiniMax H3 - one transformer that denoises video and audio
// together", position-chain paragraph): coordinates (t, h, w) -> rope() ->
// rotate Q and K.  The head dim is split into contiguous t | h | w sections;
// inside section a, pair p turns dims (o_a + 2p, o_a + 2p + 1) by
// pos_a * theta_a^(-2p / d_a).  The angle is formed and reduced in binary64,
// its cos / sin taken in binary32; the rotation runs in binary32 with explicit
// fused multiply-adds and the result is rounded to bfloat16, nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

constexpr int kHeadDim = 128;
constexpr int kPairs = kHeadDim / 2;

// Inverse frequency of every pair and the pair indices where the h and w
// sections begin (pairs [0, b1) are t, [b1, b2) are h, [b2, 64) are w).
struct RopeTable {
  double freq[kPairs];
  int32_t b1;
  int32_t b2;
};

__device__ __forceinline__ int rope_axis(int pair, const RopeTable& tab) {
  return (pair >= tab.b1) + (pair >= tab.b2);
}

// cos / sin of the angle pos * freq.  The angle is formed in binary64 and reduced
// there to quarter turns, ang = q pi/2 + t with integer q and |t| <= pi/4 (the
// reduction error is about q * 1e-16).  sin t and cos t are their Taylor
// polynomials to degree 9 and 10, whose truncation error on |t| <= pi/4 is below
// 2e-9, evaluated in binary32 by Horner's rule; q mod 4 then swaps and negates
// them.  There is no branch and no large-argument path (|t| is always small),
// which keeps the code short where many rotations are unrolled.  Error against
// the binary64 angle: about 6e-8 (the binary32 rounding of t dominates).
__device__ __forceinline__ void rope_cos_sin(float pos, double freq, float& c, float& s) {
  const double ang = static_cast<double>(pos) * freq;
  const double q = __builtin_rint(ang * 0.63661977236758134);             // ang / (pi / 2)
  const float t = static_cast<float>(__builtin_fma(-q, 1.5707963267948966, ang));
  const float t2 = t * t;
  float ps = 1.0f / 362880.0f;                                             // sin: t - t^3/3! + ... + t^9/9!
  ps = __builtin_fmaf(ps, t2, -1.0f / 5040.0f);
  ps = __builtin_fmaf(ps, t2, 1.0f / 120.0f);
  ps = __builtin_fmaf(ps, t2, -1.0f / 6.0f);
  const float sn = __builtin_fmaf(ps * t2, t, t);
  float pc = -1.0f / 3628800.0f;                                           // cos: 1 - t^2/2! + ... - t^10/10!
  pc = __builtin_fmaf(pc, t2, 1.0f / 40320.0f);
  pc = __builtin_fmaf(pc, t2, -1.0f / 720.0f);
  pc = __builtin_fmaf(pc, t2, 1.0f / 24.0f);
  pc = __builtin_fmaf(pc, t2, -0.5f);
  const float cs = __builtin_fmaf(pc, t2, 1.0f);
  // cos(t + q pi/2), sin(t + q pi/2) for q mod 4 = 0, 1, 2, 3:
  // (cs, sn), (-sn, cs), (-cs, -sn), (sn, -cs)
  const int qi = static_cast<int>(q) & 3;
  const float c0 = (qi & 1) ? sn : cs;
  const float s0 = (qi & 1) ? cs : sn;
  c = ((qi + 1) & 2) ? -c0 : c0;
  s = (qi & 2) ? -s0 : s0;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t p;
  p[0] = static_cast<__bf16>(lo);   // round to nearest even
  p[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, p);
}

// Rotate one adjacent pair held as two bf16 in a 32-bit word (low half = even dim).
__device__ __forceinline__ uint32_t rope_rotate_word(uint32_t xy, float c, float s) {
  const float x = __uint_as_float(xy << 16);
  const float y = __uint_as_float(xy & 0xffff0000u);
  const float xo = __builtin_fmaf(x, c, -(y * s));
  const float yo = __builtin_fmaf(x, s, y * c);
  return pack_bf16x2(xo, yo);
}

}  // namespace h3
