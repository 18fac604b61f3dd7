// Latent <-> token packing with the sampler's Euler step, for gfx950.
//
// "MiniMax H3 - one transformer that denoises video and audio together":
// patchify takes every non-overlapping 1 x 2 x 2 block of the video latent and
// glues its 24 x 2 x 2 channel values into one 96-value token (44 x 80 latent
// sheet -> 22 x 40 = 880 tokens per latent frame); one audio latent frame is one
// 32-value token per stereo channel; generation runs a non-learned scheduler
// step along the predicted velocity, x <- x + dt * v, and only the target rows
// move ("Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio",
// section 2).
//
// Layouts: video latent float32 [C][T][H][W]; token row (t, py, px) =
// (t * H/2 + py) * W/2 + px, value (c, iy, ix) at (c * 2 + iy) * 2 + ix.  Audio
// latent float32 [n_ch][steps][width]; token row s * n_ch + ch = latent[ch][s].
// The state stays float32 (one fused multiply-add per element); tokens are
// bfloat16, nearest even.
//
// Video: one workgroup per (latent frame, patch row).  The two latent rows of
// every channel are read coalesced into LDS, updated and emitted in token order
// (velocity reads and token writes are contiguous rows), then written back
// coalesced.  HBM-bound: 4 + 4 B of state and 2 + 2 B of tokens per element; at
// these sizes every workgroup of a launch is resident at once, so the time is the
// chain of memory round trips of one workgroup.  Audio: one thread per value
// pair.  One launch can carry both a video and an audio latent (the video
// workgroups first), which saves the audio launch of a sampler step.
#include "launch.hpp"

namespace h3 {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kPackThreads = 256;

__device__ __forceinline__ f32x2_t bf16x2_to_f32(uint32_t w) {
  return f32x2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}

__device__ __forceinline__ void video_pack(const PackArgs& a, int blk, float* tile) {
  const int hp = a.h >> 1, wp = a.w >> 1;
  const int t = blk / hp, py = blk - t * hp;
  const int two_w = 2 * a.w;
  const int n = a.c * two_w;        // elements of the two latent rows, all channels
  const int64_t plane = int64_t(a.t) * a.h * a.w;
  float* lat = a.latent + (int64_t(t) * a.h + 2 * py) * a.w;   // channel 0, row 2 py

  // latent rows -> LDS (pairs along x)
  for (int e = 2 * threadIdx.x; e < n; e += 2 * kPackThreads) {
    const int c = e / two_w, rem = e - c * two_w;   // rem = iy * W + x, x even
    *reinterpret_cast<f32x2_t*>(tile + e) = *reinterpret_cast<const f32x2_t*>(lat + c * plane + rem);
  }
  __syncthreads();

  // token order: pair p of token px covers values 2 jp, 2 jp + 1 = (c, iy, ix = 0 / 1)
  const int64_t row0 = int64_t(blk) * wp;
  const int pairs_per_token = 2 * a.c;
  for (int p = threadIdx.x; p < a.c * a.w; p += kPackThreads) {
    const int px = p / pairs_per_token, jp = p - px * pairs_per_token;
    const int c = jp >> 1, iy = jp & 1;
    float* cell = tile + c * two_w + iy * a.w + 2 * px;
    f32x2_t v = *reinterpret_cast<f32x2_t*>(cell);
    if (a.v != nullptr) {
      const f32x2_t d = bf16x2_to_f32(*reinterpret_cast<const uint32_t*>(a.v + (row0 + px) * a.v_stride + 2 * jp));
      v = f32x2_t{__builtin_fmaf(a.dt, d[0], v[0]), __builtin_fmaf(a.dt, d[1], v[1])};
      *reinterpret_cast<f32x2_t*>(cell) = v;
    }
    if (a.tokens != nullptr)
      *reinterpret_cast<uint32_t*>(a.tokens + (row0 + px) * a.tok_stride + 2 * jp) = pack_bf16x2(v[0], v[1]);
  }

  if (a.v == nullptr) return;
  __syncthreads();
  for (int e = 2 * threadIdx.x; e < n; e += 2 * kPackThreads) {
    const int c = e / two_w, rem = e - c * two_w;
    *reinterpret_cast<f32x2_t*>(lat + c * plane + rem) = *reinterpret_cast<const f32x2_t*>(tile + e);
  }
}

// audio: a = (n_ch, steps, width) in (c, t, w); one thread per value pair
__device__ __forceinline__ void audio_pack(const PackArgs& a, int blk) {
  const int half = a.w >> 1;
  const int64_t total = int64_t(a.t) * a.c * half;
  const int64_t p = int64_t(blk) * kPackThreads + threadIdx.x;
  if (p >= total) return;
  const int64_t row = p / half;                      // token row s * n_ch + ch
  const int j = 2 * int(p - row * half);
  const int64_t s = row / a.c, ch = row - s * a.c;
  float* cell = a.latent + (ch * a.t + s) * a.w + j;
  f32x2_t v = *reinterpret_cast<f32x2_t*>(cell);
  if (a.v != nullptr) {
    const f32x2_t d = bf16x2_to_f32(*reinterpret_cast<const uint32_t*>(a.v + row * a.v_stride + j));
    v = f32x2_t{__builtin_fmaf(a.dt, d[0], v[0]), __builtin_fmaf(a.dt, d[1], v[1])};
    *reinterpret_cast<f32x2_t*>(cell) = v;
  }
  if (a.tokens != nullptr) *reinterpret_cast<uint32_t*>(a.tokens + row * a.tok_stride + j) = pack_bf16x2(v[0], v[1]);
}

// workgroups [0, video_blocks) pack the video latent, the rest the audio latent
__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackArgs video, PackArgs audio, int video_blocks) {
  extern __shared__ float tile[];   // [C][2][W] of the video latent
  if (static_cast<int>(blockIdx.x) < video_blocks) {
    video_pack(video, blockIdx.x, tile);
  } else {
    audio_pack(audio, blockIdx.x - video_blocks);
  }
}

}  // namespace

namespace {

int video_blocks(const PackArgs* v) { return v != nullptr ? v->t * (v->h >> 1) : 0; }
int audio_blocks(const PackArgs* a) {
  return a != nullptr ? static_cast<int>((int64_t(a->t) * a->c * (a->w >> 1) + kPackThreads - 1) / kPackThreads) : 0;
}

}  // namespace

hipError_t launch_av_pack(const PackArgs* video, const PackArgs* audio, hipStream_t stream) {
  PackArgs none;
  __builtin_memset(&none, 0, sizeof(none));
  PackArgs v = video != nullptr ? *video : none, au = audio != nullptr ? *audio : none;
  int vb = video_blocks(video);
  const int ab = audio_blocks(audio);
  void* args[] = {&v, &au, &vb};
  const size_t lds = video != nullptr ? size_t(video->c) * 2 * video->w * sizeof(float) : 0;
  return hipLaunchKernel(reinterpret_cast<const void*>(&pack_kernel), dim3(vb + ab), dim3(kPackThreads), args, lds,
                         stream);
}

hipError_t launch_video_pack(const PackArgs& a, hipStream_t stream) { return launch_av_pack(&a, nullptr, stream); }

hipError_t launch_audio_pack(const PackArgs& a, hipStream_t stream) { return launch_av_pack(nullptr, &a, stream); }

}  // namespace h3
