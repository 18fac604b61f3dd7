// Internal launchers of the HIP kernels (host side).  Arguments are validated
// by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rope_math.hpp"

namespace h3 {

struct RopeArgs {
  const float* coords;
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  uint16_t* k_out;
  int32_t n;
  int32_t heads;
  int32_t stride;     // elements between rows
  RopeTable tab;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const float* coords;
  int32_t n;
  int32_t heads;
  int32_t stride_qkv;  // elements between rows of q, k, v
  int32_t stride_o;    // elements between rows of o
  float scale;         // softmax scale (natural base)
  float scale_log2;    // scale * log2(e)
  int32_t rope_q;
  int32_t pad_;
  RopeTable tab;
};

hipError_t launch_rope_qk(const RopeArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream);

}  // namespace h3
