// Attention projections y = x W^T (+ b) with the rotary embedding of Q and K in
// the epilogue, for gfx950.
//
// Text, reference media and noisy latents share one set of attention
// projections ("Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo
// Audio", section 2), and positions reach attention only through rope()
// rotating Q and K ("MiniMax H3 - one transformer that denoises video and audio
// together", position-chain paragraph).  Rotating the projection's float32
// accumulators before the single rounding to bfloat16 removes the separate
// RoPE pass over Q and K.
//
// Transposed product, C^T[feature][token] = W . x^T on v_mfma_f32_32x32x16_bf16
// (A = W rows, B = x rows, both k-contiguous).  Each lane then holds one token
// and, in consecutive accumulator registers, consecutive output features: the
// rotation pairs (2p, 2p + 1) of a head are neighbouring registers of one lane.
//
// A workgroup of 8 waves computes 256 features x 256 tokens; wave (wf, wt) owns
// features [128 wf, +128) (one whole head) and tokens [64 wt, +64).  k advances
// 64 at a time through double-buffered LDS tiles whose 144-byte rows make the
// 16-byte operand reads bank-conflict-free; the next stage's global loads are in
// flight while the current one is multiplied.  Workgroups are ordered in groups
// of 8 token tiles so that the tiles in flight share x and W in the caches.
// Rows of x past m read as zero (buffer loads with a clamped descriptor) and
// their outputs are not stored.
#include "launch.hpp"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;                    // features and tokens per workgroup
constexpr int kBK = 64;                       // k per stage
constexpr int kStr = kBK + 8;                 // LDS row stride, elements (144 B)
constexpr int kBuf = kTile * kStr;            // elements per operand buffer
constexpr int kLoads = kTile * kBK / 8 / kThreads;   // 16-byte chunks per thread, operand and stage (4)
constexpr int kGroup = 8;                     // token tiles per ordering group
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t as[2 * kBuf];   // W tile [feature][k]
  __shared__ __attribute__((aligned(16))) uint16_t bs[2 * kBuf];   // x tile [token][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, hf = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  // grouped tile order: kGroup token tiles sweep all feature tiles together
  const int pid = blockIdx.x;
  const int group_size = kGroup * a.tiles_f;
  const int first_t = (pid / group_size) * kGroup;
  const int gsz = min(a.tiles_t - first_t, kGroup);
  const int in_group = pid - (pid / group_size) * group_size;
  const int tt = first_t + in_group % gsz;
  const int tf = in_group / gsz;
  const int f0 = tf * kTile, t0 = tt * kTile;

  // global -> register staging: chunk q = tid + kThreads i is row q / 8, k columns 8 (q % 8) ..
  const int xrow_bytes = static_cast<int>(a.x_stride * 2), wrow_bytes = static_cast<int>(a.w_stride * 2);
  const int64_t x_left = (int64_t(a.m) - t0) * a.x_stride * 2;
  const __amdgpu_buffer_rsrc_t xd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.x + int64_t(t0) * a.x_stride), 0, static_cast<int>(static_cast<uint32_t>(x_left)), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t wd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w + int64_t(f0) * a.w_stride), 0, kTile * wrow_bytes, kRsrcFlags);
  int xoff[kLoads], woff[kLoads], lds_st[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int q = tid + kThreads * i, row = q >> 3, c8 = q & 7;
    xoff[i] = row * xrow_bytes + c8 * 16;
    woff[i] = row * wrow_bytes + c8 * 16;
    lds_st[i] = row * kStr + c8 * 8;
  }
  u32x4_t xr[kLoads], wr[kLoads];
  auto load = [&](int s) {
    const int kb = s * kBK * 2;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      wr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wd, woff[i] + kb, 0, 0));
      xr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xd, xoff[i] + kb, 0, 0));
    }
  };
  lds_u16* asl = (lds_u16*)as;
  lds_u16* bsl = (lds_u16*)bs;
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      *reinterpret_cast<lds_u32x4*>(asl + buf * kBuf + lds_st[i]) = wr[i];
      *reinterpret_cast<lds_u32x4*>(bsl + buf * kBuf + lds_st[i]) = xr[i];
    }
  };

  // operand reads: A (W) rows 128 wf + 32 fb + col, B (x) rows 64 wt + 32 tb + col, k 16 kk + 8 hf
  const int a_rd = (wf * 128 + col) * kStr + 8 * hf;
  const int b_rd = (wt * 64 + col) * kStr + 8 * hf;
  f32x16_t acc[4][2];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = f32x16_t{};

  auto compute = [&](int buf) {
    const lds_u16* at = asl + buf * kBuf + a_rd;
    const lds_u16* bt = bsl + buf * kBuf + b_rd;
    bf16x8_t af[2][4], bf[2][2];
    auto read = [&](int kk, int slot) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) af[slot][fb] = *reinterpret_cast<const lds_bf16x8*>(at + fb * 32 * kStr + 16 * kk);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) bf[slot][tb] = *reinterpret_cast<const lds_bf16x8*>(bt + tb * 32 * kStr + 16 * kk);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) read(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = mfma(af[kk & 1][fb], bf[kk & 1][tb], acc[fb][tb]);
    }
  };

  const int nst = a.k / kBK;
  load(0);
  store(0);
  __syncthreads();
  if (nst > 1) load(1);
  for (int s = 0; s < nst; ++s) {
    compute(s & 1);
    if (s + 1 < nst) store((s + 1) & 1);
    if (s + 2 < nst) load(s + 2);
    __syncthreads();
  }

  // epilogue: bias, rotation of whole-head slabs, one rounding to bf16
  const int fw0 = f0 + wf * 128;                       // first feature of this wave: a head boundary
  const bool rotate = fw0 < a.rope_cols;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int token = t0 + wt * 64 + tb * 32 + col;
    const bool valid = token < a.m;
    float pos0 = 0.0f, pos1 = 0.0f, pos2 = 0.0f;
    if (rotate && valid) {
      pos0 = a.coords[3 * int64_t(token) + 0];
      pos1 = a.coords[3 * int64_t(token) + 1];
      pos2 = a.coords[3 * int64_t(token) + 2];
    }
    uint16_t* yrow = a.y + int64_t(valid ? token : 0) * a.y_stride + fw0;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x16_t v = acc[fb][tb];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = fb * 32 + 8 * g + 4 * hf;       // head-dim index of register 4 g
        if (a.bias != nullptr) {
          const uint2 bw = *reinterpret_cast<const uint2*>(a.bias + fw0 + d0);
          v[4 * g + 0] += __uint_as_float(bw.x << 16);
          v[4 * g + 1] += __uint_as_float(bw.x & 0xffff0000u);
          v[4 * g + 2] += __uint_as_float(bw.y << 16);
          v[4 * g + 3] += __uint_as_float(bw.y & 0xffff0000u);
        }
        if (rotate) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int pair = (d0 >> 1) + h;
            const int ax = rope_axis(pair, a.tab);
            float cs, sn;
            rope_cos_sin(ax == 0 ? pos0 : (ax == 1 ? pos1 : pos2), a.tab.freq[pair], cs, sn);
            const float x = v[4 * g + 2 * h], y = v[4 * g + 2 * h + 1];
            v[4 * g + 2 * h] = __builtin_fmaf(x, cs, -(y * sn));
            v[4 * g + 2 * h + 1] = __builtin_fmaf(x, sn, y * cs);
          }
        }
        if (valid)
          *reinterpret_cast<uint2*>(yrow + d0) = make_uint2(pack_bf16x2(v[4 * g + 0], v[4 * g + 1]),
                                                            pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel), dim3(a.tiles_f * a.tiles_t), dim3(kThreads),
                         args, 0, stream);
}

}  // namespace h3
