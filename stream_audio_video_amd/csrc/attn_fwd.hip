// Full bidirectional attention forward with MM-RoPE on Q, for gfx950.
//
// Per head: O = softmax(Q~ K~^T * scale) V over all rows, no mask (the open
// release runs full attention: "Inside MiniMax H3: One DiT Stream for Text,
// Video, and Stereo Audio", section 6).  K arrives already rotated; Q is rotated
// in registers while its tile is loaded (or arrives rotated, rope_q == 0).
//
// Work split.  A workgroup of kWaves waves owns kBM = 32 * kWaves query rows of
// one head; each wave owns 32 query rows and keeps their rotated Q in
// registers for the whole kernel.  The workgroup streams the head's K and V in
// tiles of kBN keys through LDS (double-buffered, one barrier per tile; the
// next tile's global loads are in flight while the current one is computed).
//
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form so that a
// query is a column of every accumulator:
//   S^T[key][query] = K~ . Q~^T   (A = K tile rows from LDS, B = Q~ registers)
//   O^T[d][query]  += V^T . P^T    (A = V^T from LDS, B = P straight from the
//                                   S^T accumulators, converted to bf16)
// With queries in columns, every lane holds one query and 16 of its scores, so
// the row max is an in-lane max plus one exchange with the lane 32 away, and
// the row sum needs no exchange until the end.  The contraction order of the PV
// product is free, so the keys are numbered to match the accumulator layout;
// V is written transposed into LDS in that key order.
//
// Online softmax in base 2 with a lazy rescale: the running reference max of a
// row is raised (and O, l rescaled) only when a tile's max exceeds it by more
// than 2^8 in probability, so the rescale is skipped on almost every tile and
// exp2 arguments stay <= 8.  The result is exact up to rounding either way.
#include "launch.hpp"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;     // query rows per workgroup
constexpr int kBN = 64;              // keys per tile
constexpr int kKStr = kHeadDim + 8;  // LDS row stride of the K tile, elements (272 B)
constexpr int kVStr = kBN + 8;       // LDS row stride of the V^T tile, elements (144 B)
constexpr float kLazyLog2 = 8.0f;    // rescale only when the max grows by more than 2^8

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position inside a 16-key group of the V^T tile for the 4-key run starting at
// key 4r (r = 0..3): runs are stored in the order 0, 2, 1, 3 so that the 8 keys
// one lane feeds to a PV step (keys 4h..4h+3 and 8+4h..8+4h+3) are contiguous.
__device__ __forceinline__ int vt_run_slot(int r) { return ((r & 1) << 1) | (r >> 1); }

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * kKStr];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kHeadDim * kVStr];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column / A-operand row of this lane
  const int hf = lane >> 5;    // which 8-element half of a 16-deep k chunk
  const int nqb = (a.n + kBM - 1) / kBM;
  const int head = blockIdx.x / nqb;
  const int qb = blockIdx.x - head * nqb;
  const int qrow = qb * kBM + wave * 32 + col;
  const bool qvalid = qrow < a.n;

  // ---- Q~ fragment: B operand of S^T, lane holds dims 16c + 8hf .. +7 of its query
  bf16x8_t qf[8];
  {
    const uint16_t* qp = a.q + (qvalid ? qrow : 0) * a.stride_qkv + head * kHeadDim + 8 * hf;
    float pos[3] = {0.0f, 0.0f, 0.0f};
    if (a.rope_q && qvalid) {
      pos[0] = a.coords[3 * qrow + 0];
      pos[1] = a.coords[3 * qrow + 1];
      pos[2] = a.coords[3 * qrow + 2];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qvalid) x = *reinterpret_cast<const uint4*>(qp + 16 * c);
      if (a.rope_q) {
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pair = 8 * c + 4 * hf + p;
          float cs, sn;
          rope_cos_sin(pos[rope_axis(pair, a.tab)], a.tab.freq[pair], cs, sn);
          w[p] = rope_rotate_word(w[p], cs, sn);
        }
        x = make_uint4(w[0], w[1], w[2], w[3]);
      }
      qf[c] = as_bf16x8(x);
    }
  }

  // ---- K / V tile loaders
  const uint16_t* kbase_p = a.k + head * kHeadDim;
  const uint16_t* vbase_p = a.v + head * kHeadDim;
  const int kd = (tid & 15) * 8;      // K: 16-byte chunk of a key row
  const int krow = tid >> 4;          // K: key rows krow + 16 r
  const int vd = (tid & 15) * 8;      // V: dims vd .. vd+7
  const int vg = tid >> 4;            // V: keys 4vg .. 4vg+3
  uint4 kr[4], vr[4];

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + krow + 16 * r;
      kr[r] = key < a.n ? *reinterpret_cast<const uint4*>(kbase_p + key * a.stride_qkv + kd)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * vg + i;
      vr[i] = key < a.n ? *reinterpret_cast<const uint4*>(vbase_p + key * a.stride_qkv + vd)
                        : make_uint4(0, 0, 0, 0);
    }
  };

  const int vslot = 16 * (vg >> 2) + 4 * vt_run_slot(vg & 3);
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<uint4*>(&ks[buf][(krow + 16 * r) * kKStr + kd]) = kr[r];
    const uint32_t v0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
    const uint32_t v1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
    const uint32_t v2[4] = {vr[2].x, vr[2].y, vr[2].z, vr[2].w};
    const uint32_t v3[4] = {vr[3].x, vr[3].y, vr[3].z, vr[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dim vd + 2w: low halves of the four keys; dim vd + 2w + 1: high halves
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u),
                                  __builtin_amdgcn_perm(v3[w], v2[w], 0x05040100u));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u),
                                  __builtin_amdgcn_perm(v3[w], v2[w], 0x07060302u));
      *reinterpret_cast<uint2*>(&vt[buf][(vd + 2 * w) * kVStr + vslot]) = lo;
      *reinterpret_cast<uint2*>(&vt[buf][(vd + 2 * w + 1) * kVStr + vslot]) = hi;
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  float m_ref = -__builtin_inff();
  float l_part = 0.0f;
  const float c2 = a.scale_log2;

  const int ntiles = (a.n + kBN - 1) / kBN;
  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < ntiles) load_tile((t + 1) * kBN);

    // S^T = K~ Q~^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16_t{};
      const uint16_t* kp = &ks[buf][(32 * b + col) * kKStr + 8 * hf];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        s[b] = mfma32(*reinterpret_cast<const bf16x8_t*>(kp + 16 * c), qf[c], s[b]);
    }

    // keys past the end of the sequence (last tile only) take no weight
    const int key0 = t * kBN;
    if (key0 + kBN > a.n) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= a.n) s[b][r] = -__builtin_inff();
        }
    }

    float mt = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[b][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));

    const bool need = (mt - m_ref) * c2 > kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }
    const float nm = -m_ref * c2;

    // P = exp2(S * c - m * c) -> bf16, the B operand of the PV product
    bf16x8_t pb[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c2, nm));
        l_part += p;
        pb[b][r >> 3][r & 7] = static_cast<__bf16>(p);
      }

    // O^T += V^T P^T over four 16-key chunks, four 32-dim blocks
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t va =
            *reinterpret_cast<const bf16x8_t*>(&vt[buf][(32 * db + col) * kVStr + 16 * kc + 8 * hf]);
        oacc[db] = mfma32(va, pb[kc >> 1][kc & 1], oacc[db]);
      }
    }
  }

  // ---- epilogue: O = O^T / l, LSE = m * scale + ln l
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = a.o + qrow * a.stride_o + head * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * hf;
        const uint2 w = make_uint2(pack_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
    if (a.lse != nullptr && hf == 0) a.lse[head * a.n + qrow] = m_ref * a.scale + logf(l_tot);
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.n + kBM - 1) / kBM;
  const dim3 grid(nqb * a.heads), block(kThreads);
  void* args[] = {const_cast<FwdArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel), grid, block, args, 0, stream);
}

}  // namespace h3
