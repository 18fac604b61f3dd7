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
  int32_t n_full;          // work units (head, query block) run over all keys, one workgroup each
  int32_t split;           // key ranges per later unit (1: no later units)
  int32_t tiles_per_split; // key tiles per range
  float* ws_o;             // partials of split units: float32 [unit * split + part][rows][128]
  float* ws_ml;            // and their (m, l) per row: float32 [unit * split + part][rows][2]
  RopeTable tab;
};

struct AdalnArgs {
  const uint16_t* x;       // bf16 [n_rows][x_stride]
  const uint16_t* y;       // bf16 [n_rows][y_stride]; null selects the plain modulation
  const int32_t* t_idx;    // per-row timestep index
  const int32_t* tags;     // per-row token tag (0 text, 1 video, 2 audio)
  const uint16_t* gate;    // bf16 table planes: entry e at plane + e * entry_stride
  const uint16_t* shift;
  const uint16_t* scale;
  uint16_t* x_out;         // bf16 residual result (residual form only)
  uint16_t* h;             // bf16 modulated norm
  int64_t x_stride;
  int64_t y_stride;
  int64_t out_stride;      // rows of x_out
  int64_t h_stride;
  int64_t entry_stride;
  int64_t n_entries;
  int64_t n_rows;
  int32_t hidden;
  int32_t norm_kind;       // 0 layer norm, 1 root-mean-square norm
  float eps;
};

struct PackArgs {
  float* latent;           // float32 sampler state (updated in place when v is set)
  const uint16_t* v;       // bf16 velocity tokens, or null (no update)
  uint16_t* tokens;        // bf16 tokens out, or null
  int64_t v_stride;        // elements between token rows
  int64_t tok_stride;
  int32_t c;               // video: channels      | audio: stereo channels
  int32_t t;               // video: latent frames | audio: steps
  int32_t h;               // video: latent rows   | audio: 1
  int32_t w;               // video: latent cols   | audio: values per frame
  float dt;
};

struct GemmArgs {
  const uint16_t* x;       // bf16 [m][x_stride]
  const uint16_t* w;       // bf16 [n_out][w_stride]
  const uint16_t* bias;    // bf16 [n_out] or null
  uint16_t* y;             // bf16 [m][y_stride]
  const float* rope_tab;   // [m][64][2] (cos, sin) of every row's rotation pairs when rope_cols > 0
  int64_t x_stride;
  int64_t w_stride;
  int64_t y_stride;
  int32_t m;
  int32_t n_out;
  int32_t k;
  int32_t rope_cols;       // leading output features rotated, in whole 128-wide heads
  int32_t tiles_f;
  int32_t tiles_t;
};

struct RopeTabArgs {
  const float* coords;     // [n][3]
  float* out;              // [n][64][2]: (cos, sin) of pair p of row i
  int32_t n;
  RopeTable tab;
};

hipError_t launch_rope_qk(const RopeArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_rope_table(const RopeTabArgs& a, hipStream_t stream);
hipError_t launch_video_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_audio_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_adaln(const AdalnArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream);
// Key-split schedule of the last, partly filled wave of attention workgroups on `cus` CUs:
// fills n_full, split, tiles_per_split and the workspace bytes it needs (0: no split).
void attn_fwd_schedule(int32_t n, int32_t heads, int32_t cus, int32_t* n_full, int32_t* split,
                       int32_t* tiles_per_split, int64_t* ws_bytes);

}  // namespace h3
