// Streaming MM-RoPE pass over Q and/or K (HBM-bound).
//
// A workgroup owns kTok consecutive rows.  It first forms the cos / sin of the
// 64 pair angles of each of its rows (once per row, in LDS), then streams the
// rows' heads in 16-byte chunks (4 adjacent pairs = 8 bf16), rotating each chunk
// with the shared table.  Every chunk is read once and written once: the
// algorithmic traffic is 2 x 2 bytes per element per rotated tensor plus 12
// bytes of coordinates per row.
#include "launch.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 4;          // rows per workgroup
constexpr int kUnroll = 4;       // chunks in flight per thread

__device__ __forceinline__ uint4 rotate_chunk(uint4 x, const float2* cs) {
  x.x = rope_rotate_word(x.x, cs[0].x, cs[0].y);
  x.y = rope_rotate_word(x.y, cs[1].x, cs[1].y);
  x.z = rope_rotate_word(x.z, cs[2].x, cs[2].y);
  x.w = rope_rotate_word(x.w, cs[3].x, cs[3].y);
  return x;
}

__global__ __launch_bounds__(kThreads) void rope_qk_kernel(RopeArgs a) {
  __shared__ float2 cs[kTok * kPairs];
  const int tok0 = blockIdx.x * kTok;
  for (int i = threadIdx.x; i < kTok * kPairs; i += kThreads) {
    const int row = tok0 + i / kPairs;
    const int pair = i % kPairs;
    float c = 1.0f, s = 0.0f;
    if (row < a.n) {
      const float pos = a.coords[3 * row + rope_axis(pair, a.tab)];
      rope_cos_sin(pos, a.tab.freq[pair], c, s);
    }
    cs[i] = make_float2(c, s);
  }
  __syncthreads();

  const int rows = min(kTok, a.n - tok0);
  const int per_row = a.heads * (kHeadDim / 8);
  const int total = rows * per_row;
  for (int base = 0; base < total; base += kThreads * kUnroll) {
    uint4 xq[kUnroll], xk[kUnroll];
    int off[kUnroll], tab[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int idx = base + threadIdx.x + u * kThreads;
      ok[u] = idx < total;
      const int r = ok[u] ? idx / per_row : 0;
      const int rem = ok[u] ? idx - r * per_row : 0;
      const int head = rem >> 4, dc = rem & 15;
      off[u] = (tok0 + r) * a.stride + head * kHeadDim + dc * 8;
      tab[u] = r * kPairs + dc * 4;
      if (ok[u]) {
        if (a.q_in) xq[u] = *reinterpret_cast<const uint4*>(a.q_in + off[u]);
        if (a.k_in) xk[u] = *reinterpret_cast<const uint4*>(a.k_in + off[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!ok[u]) continue;
      if (a.q_in) *reinterpret_cast<uint4*>(a.q_out + off[u]) = rotate_chunk(xq[u], cs + tab[u]);
      if (a.k_in) *reinterpret_cast<uint4*>(a.k_out + off[u]) = rotate_chunk(xk[u], cs + tab[u]);
    }
  }
}

}  // namespace

hipError_t launch_rope_qk(const RopeArgs& a, hipStream_t stream) {
  const dim3 grid((a.n + kTok - 1) / kTok), block(kThreads);
  void* args[] = {const_cast<RopeArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rope_qk_kernel), grid, block, args, 0, stream);
}

}  // namespace h3
