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

// cos / sin of the angle pos * freq.  The angle is formed and reduced modulo
// 2 pi in binary64 (the reduction error is k * 2.4e-16 for k turns, far below
// binary32 resolution at any exact coordinate), then the binary32 sincos of the
// remainder in [-pi, pi] is taken.
__device__ __forceinline__ void rope_cos_sin(float pos, double freq, float& c, float& s) {
  const double ang = static_cast<double>(pos) * freq;
  const double turns = __builtin_rint(ang * 0.15915494309189535);       // round(ang / (2 pi))
  const float r = static_cast<float>(__builtin_fma(-turns, 6.283185307179586, ang));
  sincosf(r, &s, &c);
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
