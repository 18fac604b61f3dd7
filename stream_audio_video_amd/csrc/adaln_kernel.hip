// Indexed AdaLN modulation around attention, for gfx950.
//
// Every row of the packed sequence picks its own modulation entry,
// e = timestep_index * 3 + token_tag ("MiniMax H3 - one transformer that
// denoises video and audio together", AdaLN paragraphs; "Inside MiniMax H3: One
// DiT Stream for Text, Video, and Stereo Audio", section 5: shift, scale and
// gate per block for the attention and MLP paths, gathered per row).
//
//   modulate:  h = norm(x) * (1 + scale[e]) + shift[e]
//   residual:  x' = bf16(x + gate[e] * y);  h = norm(x') * (1 + scale[e]) + shift[e]
//
// norm is a layer norm without affine ((x - mean) / sqrt(var + eps), biased
// variance) or, on request, a root-mean-square norm (x / sqrt(mean(x^2) + eps)):
// the same code with the mean held at zero.
//
// One wave owns one row (HBM-bound: 2 B read and 2 B written per element and
// tensor) and is a workgroup of its own.  Lane l holds the 16-byte chunks l,
// l + 64, ... of the row, so every load and store instruction of the wave covers
// 1 KB of contiguous memory, and the row statistics reduce inside the wave with
// no LDS and no barrier.  The streamed tensors (x, y in; x_out, h out) are read
// and written non-temporally, so they do not displace the table in the caches;
// the table planes are read normally (every row of a segment shares an entry).  The
// residual row stays in registers as the bfloat16 values that are stored, which
// are exactly what the norm reads; the shift / scale chunks are requested while
// the statistics are reduced.  Arithmetic is float32 with one rounding to
// bfloat16 (nearest even) per output.
#include "launch.hpp"

namespace h3 {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWavesPerGroup = 1;
constexpr uint32_t kNaN2 = 0x7fc07fc0u;   // two bfloat16 quiet NaNs

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// J = 16-byte chunks per lane (hidden <= 512 * J); kRes selects the gated residual
template <int J, bool kRes>
__global__ __launch_bounds__(64 * kWavesPerGroup) void adaln_kernel(AdalnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kWavesPerGroup + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  const int nchunk = a.hidden >> 3;
  const int t = a.t_idx[row], tag = a.tags[row];
  const int64_t e = int64_t(t) * 3 + tag;
  uint16_t* hr = a.h + row * a.h_stride;
  uint16_t* xo = kRes ? a.x_out + row * a.out_stride : nullptr;

  if (t < 0 || tag < 0 || tag >= 3 || e >= a.n_entries) {
    // an index outside the table: the row's outputs become NaN, nothing is read
    const u32x4_t nan = {kNaN2, kNaN2, kNaN2, kNaN2};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 64 * j + lane;
      if (c < nchunk) {
        st16(hr + 8 * c, nan);
        if (kRes) st16(xo + 8 * c, nan);
      }
    }
    return;
  }

  const uint16_t* xr = a.x + row * a.x_stride;
  u32x4_t r[J];
  if constexpr (kRes) {
    const uint16_t* yr = a.y + row * a.y_stride;
    const uint16_t* gr = a.gate + e * a.entry_stride;
    u32x4_t xv[J], yv[J], gv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 64 * j + lane;
      if (c < nchunk) {
        xv[j] = ld16_stream(xr + 8 * c);
        yv[j] = ld16_stream(yr + 8 * c);
        gv[j] = ld16(gr + 8 * c);
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 64 * j + lane;
      if (c < nchunk) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          r[j][w] = pack_bf16x2(__builtin_fmaf(lo_f(gv[j][w]), lo_f(yv[j][w]), lo_f(xv[j][w])),
                                __builtin_fmaf(hi_f(gv[j][w]), hi_f(yv[j][w]), hi_f(xv[j][w])));
        st16(xo + 8 * c, r[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 64 * j + lane;
      if (c < nchunk) r[j] = ld16_stream(xr + 8 * c);
    }
  }

  // modulation chunks, requested before the statistics are reduced
  const uint16_t* shr = a.shift + e * a.entry_stride;
  const uint16_t* scr = a.scale + e * a.entry_stride;
  u32x4_t sh[J], sc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = 64 * j + lane;
    if (c < nchunk) {
      sh[j] = ld16(shr + 8 * c);
      sc[j] = ld16(scr + 8 * c);
    }
  }

  // statistics: two passes over the register-resident row
  const float inv_c = 1.0f / static_cast<float>(a.hidden);
  float mean = 0.0f;
  if (a.norm_kind == 0) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (64 * j + lane < nchunk)
#pragma unroll
        for (int w = 0; w < 4; ++w) s += lo_f(r[j][w]) + hi_f(r[j][w]);
    mean = wave_sum(s) * inv_c;
  }
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (64 * j + lane < nchunk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float d0 = lo_f(r[j][w]) - mean, d1 = hi_f(r[j][w]) - mean;
        q = __builtin_fmaf(d0, d0, q);
        q = __builtin_fmaf(d1, d1, q);
      }
  const float rstd = 1.0f / __builtin_sqrtf(wave_sum(q) * inv_c + a.eps);

  // h = n * (1 + scale) + shift, n = (x - mean) * rstd
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = 64 * j + lane;
    if (c < nchunk) {
      u32x4_t o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float n0 = (lo_f(r[j][w]) - mean) * rstd, n1 = (hi_f(r[j][w]) - mean) * rstd;
        o[w] = pack_bf16x2(__builtin_fmaf(n0, lo_f(sc[j][w]), n0) + lo_f(sh[j][w]),
                           __builtin_fmaf(n1, hi_f(sc[j][w]), n1) + hi_f(sh[j][w]));
      }
      st16(hr + 8 * c, o);
    }
  }
}

template <bool kRes>
hipError_t launch_j(const AdalnArgs& a, hipStream_t stream) {
  const int nchunk = a.hidden >> 3;
  const dim3 grid(static_cast<unsigned>((a.n_rows + kWavesPerGroup - 1) / kWavesPerGroup));
  const dim3 block(64 * kWavesPerGroup);
  void* args[] = {const_cast<AdalnArgs*>(&a)};
  const void* k;
  if (nchunk <= 64 * 2)
    k = reinterpret_cast<const void*>(&adaln_kernel<2, kRes>);
  else if (nchunk <= 64 * 4)
    k = reinterpret_cast<const void*>(&adaln_kernel<4, kRes>);
  else if (nchunk <= 64 * 8)
    k = reinterpret_cast<const void*>(&adaln_kernel<8, kRes>);
  else if (nchunk <= 64 * 11)
    k = reinterpret_cast<const void*>(&adaln_kernel<11, kRes>);
  else
    k = reinterpret_cast<const void*>(&adaln_kernel<16, kRes>);
  return hipLaunchKernel(k, grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_adaln(const AdalnArgs& a, hipStream_t stream) {
  return a.y != nullptr ? launch_j<true>(a, stream) : launch_j<false>(a, stream);
}

}  // namespace h3
