// Attention projections y = x W^T (+ b) with the rotary embedding of Q and K in
// the epilogue, for gfx950.
//
// Text, reference media and noisy latents share one set of attention
// projections ("Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo
// Audio", section 2), and positions reach attention only through rope()
// rotating Q and K ("MiniMax H3 - one transformer that denoises video and audio
// together", position-chain paragraph).  Rotating the projection's float32
// accumulators before the single rounding to bfloat16 removes the separate
// RoPE pass over Q and K.  The (cos, sin) of every row's 64 rotation pairs come
// from a per-sequence table (rope_table_kernel below): the same pairs serve all
// heads of Q and K, every block and every sampler step, so the epilogue reads
// them instead of recomputing them per head.
//
// Transposed product, C^T[feature][token] = W . x^T on v_mfma_f32_32x32x16_bf16
// (A = W rows, B = x rows, both k-contiguous).  Each lane then holds one token
// and, in consecutive accumulator registers, consecutive output features: the
// rotation pairs (2p, 2p + 1) of a head are neighbouring registers of one lane.
//
// A workgroup of 4 waves (one per SIMD) computes 256 features x 256 tokens;
// wave (wf, wt) owns features [128 wf, +128) (one whole head) and tokens
// [128 wt, +128): 16 accumulator blocks (in AGPRs), so every 16-byte LDS operand
// read feeds four MFMAs.  k advances 64 at a time through two LDS stages filled
// by direct-to-LDS buffer loads (no staging registers).  Each wave load
// instruction writes 1 KB = 8 rows of 128 B, and a row's 16-byte chunk c is
// stored at slot c ^ ((row >> 1) & 7), which keeps the operand reads of 16 rows
// on disjoint banks.
//
// Schedule.  With one wave per SIMD nothing else hides a wave's own stalls, so
// every MFMA is followed by at most two other memory instructions: in each
// k-step of 16 MFMAs, MFMAs 0..7 each cover one operand read of the next k-step
// and every odd MFMA covers one load of a later stage.  The barrier of stage s
// sits before its last k-step, whose MFMAs then hide the reads of the next
// stage's first k-step.  Workgroups are ordered in groups of kGroup token tiles
// so that the tiles in flight share x and W in the caches.  Rows of x past m
// read as zero (clamped buffer descriptor) and their outputs are not stored.
//
// The loads are written in inline assembly: issued through the compiler's
// buffer-to-LDS builtin, every operand read of one stage would wait for the
// loads in flight into the other stage (the compiler cannot tell the two LDS
// stages apart), which serialises the pipeline.  The assembly has no register
// outputs; it sets M0 (the LDS destination), which no compiler-generated
// instruction of this kernel uses on gfx950, and the waits for the loads are
// explicit (vmcnt(0) before each barrier; none is outstanding at the epilogue).
#include "launch.hpp"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;                    // features and tokens per workgroup
constexpr int kBK = 64;                       // k per stage (128 B per row)
constexpr int kBuf = kTile * kBK;             // elements per operand stage
constexpr int kRowsPerWave = kTile / kWaves;  // rows of each operand a wave loads per stage (64)
constexpr int kEarly = 8;                     // loads of a stage issued as soon as its buffer is free
constexpr int kGroup = 4;                     // token tiles per ordering group
constexpr int kAhead = 4;                     // epilogue table loads in flight, in (token, feature) block steps
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format
static_assert(kEarly >= 0 && kEarly <= 8, "at most one load per MFMA");

struct True { static constexpr bool value = true; };
struct False { static constexpr bool value = false; };

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// raw buffer descriptor in scalar registers: base, no stride, `bytes` readable
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = kRsrcFlags;
  return r;
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds_addr + 16 * lane.  M0 carries
// the LDS address; one wait state separates its write from the load.
__device__ __forceinline__ void load_lds(i32x4_t rsrc, int voff, uint32_t lds_addr, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)

__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t as[2 * kBuf];   // W stages [feature][k], swizzled
  __shared__ __attribute__((aligned(1024))) uint16_t bs[2 * kBuf];   // x stages [token][k], swizzled
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // direct-to-LDS loads: instruction i of this wave fills rows 64 wave + 8 i .. +7 (1 KB); lane l
  // writes slot l & 7 of row 64 wave + 8 i + (l >> 3), which holds source chunk
  // (l & 7) ^ ((row >> 1) & 7) = (l & 7) ^ ((4 i + (l >> 4)) & 7).  The stage's k offset goes in
  // the scalar offset.
  const int xrow_bytes = static_cast<int>(a.x_stride * 2), wrow_bytes = static_cast<int>(a.w_stride * 2);
  const int64_t x_left = (int64_t(a.m) - t0) * a.x_stride * 2;
  const i32x4_t xd = make_rsrc(a.x + int64_t(t0) * a.x_stride, static_cast<uint32_t>(x_left));
  const i32x4_t wd = make_rsrc(a.w + int64_t(f0) * a.w_stride, static_cast<uint32_t>(kTile * wrow_bytes));
  const int lrow = lane >> 3, lpos = lane & 7;
  int voff[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = j & 7;
    const int c = lpos ^ ((4 * i + (lane >> 4)) & 7);
    const int rb = j < 8 ? wrow_bytes : xrow_bytes;
    voff[j] = (kRowsPerWave * wave + 8 * i + lrow) * rb + c * 16;
  }
  const uint32_t as_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)as));
  const uint32_t bs_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)bs));
  // load j = 0..15 of stage s into buffer buf: j < 8 are W rows, j >= 8 are x rows
  auto load_one = [&](int s, int buf, int j) {
    const int i = j & 7;
    const uint32_t lds = (j < 8 ? as_addr : bs_addr) +
                         static_cast<uint32_t>((buf * kBuf + (kRowsPerWave * wave + 8 * i) * kBK) * 2);
    load_lds(j < 8 ? wd : xd, voff[j], __builtin_amdgcn_readfirstlane(lds), s * kBK * 2);
  };

  // operand reads: A rows 128 wf + 32 fb + col, B rows 128 wt + 32 tb + col; chunk 2 kk + hf.
  const int a_row = wf * 128 + col, b_row = wt * 128 + col;
  const int a_sw = (a_row >> 1) & 7, b_sw = (b_row >> 1) & 7;
  const lds_u16* asl = (const lds_u16*)as;
  const lds_u16* bsl = (const lds_u16*)bs;
  f32x16_t acc[4][4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[fb][tb] = f32x16_t{};

  bf16x8_t op[2][8];   // [slot][0..3 = A fb, 4..7 = B tb]
  auto read_one = [&](int buf, int kk, int slot, int e) {
    if (e < 4)
      op[slot][e] = *reinterpret_cast<const lds_bf16x8*>(asl + buf * kBuf + (a_row + 32 * e) * kBK +
                                                         ((2 * kk + hf) ^ a_sw) * 8);
    else
      op[slot][e] = *reinterpret_cast<const lds_bf16x8*>(bsl + buf * kBuf + (b_row + 32 * (e - 4)) * kBK +
                                                         ((2 * kk + hf) ^ b_sw) * 8);
  };

  // One k-step: 16 MFMAs on operand slot `slot`.  After MFMA q < 8 read operand q of k-step rkk
  // of buffer rbuf into the other slot (if do_read); after each odd MFMA q issue load
  // j0 + (q >> 1) of stage lstage into buffer lbuf (if (q >> 1) < nload), so that the four waves'
  // loads reach the memory pipeline spread out rather than in bursts.  The scheduling barriers
  // keep that order.
  auto kstep = [&](int slot, bool do_read, int rbuf, int rkk, int nload, int lstage, int lbuf, int j0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int fb = q >> 2, tb = q & 3;
      acc[fb][tb] = mfma(op[slot][fb], op[slot][4 + tb], acc[fb][tb]);
      __builtin_amdgcn_sched_barrier(0);
      if (q < 8 && do_read) read_one(rbuf, rkk, slot ^ 1, q);
      if ((q & 1) && (q >> 1) < nload) load_one(lstage, lbuf, j0 + (q >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Stage s lives in buffer s & 1.  Loads of stage s + 1: the W half (loads 0..7) right after the
  // barrier that frees its buffer (during k-step 3 of stage s - 1), the x half during k-step 0 of
  // stage s; all land before the barrier ahead of k-step 3 of stage s.
  const int nst = a.k / kBK;
#pragma unroll
  for (int j = 0; j < 16; ++j) load_one(0, 0, j);
  wait_vm0();
  __syncthreads();
  if (nst > 1) {
#pragma unroll
    for (int j = 0; j < kEarly; ++j) load_one(1, 1, j);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) read_one(0, 0, 0, e);
  // one stage; more1 / more2: stages s + 1 / s + 2 exist (compile-time, so the steady state has no
  // branches)
  auto stage = [&](int s, auto more1_t, auto more2_t) {
    constexpr bool more1 = decltype(more1_t)::value, more2 = decltype(more2_t)::value;
    const int buf = s & 1;
    kstep(0, true, buf, 1, more1 ? 16 - kEarly : 0, s + 1, buf ^ 1, kEarly);
    __builtin_amdgcn_sched_barrier(0);
    kstep(1, true, buf, 2, 0, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep(0, true, buf, 3, 0, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm0();        // this wave's loads of stage s + 1 are in LDS
    __syncthreads();   // ... and every wave's; every wave is done reading stage s's buffer
    kstep(1, more1, buf ^ 1, 0, more2 ? kEarly : 0, s + 2, buf, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + 2 < nst; ++s) stage(s, True{}, True{});
  if (s + 1 < nst) stage(s++, True{}, False{});
  stage(s, False{}, False{});

  // epilogue: bias, rotation of whole-head slabs by the rows' (cos, sin) from the table, one rounding
  // to bf16.  The lane's 64 bias values are the same for every token block and are requested first.
  const int fw0 = f0 + wf * 128;                       // first feature of this wave: a head boundary
  const bool rotate = fw0 < a.rope_cols;
  // Every epilogue load is unconditional (a missing bias, or a slab without rotation, reads zeros
  // through an empty descriptor), so the waits before their uses are counted, never a vmcnt(0) at a
  // branch merge.
  const __amdgpu_buffer_rsrc_t bd = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.bias != nullptr ? a.bias + fw0 : a.y), 0, a.bias != nullptr ? 256 : 0, kRsrcFlags);
  uint2 bw[4][4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bw[fb][g] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(bd, (fb * 32 + 8 * g + 4 * hf) * 2, 0, 0));
  // the output through a descriptor over this wave's token rows (rows past m: stores dropped), and
  // the rotation table through one over the same rows (rows past m read as zero)
  const int tw0 = t0 + wt * 128;
  const int rows = min(a.m - tw0, 128);                // may be <= 0 on the last token tile
  const int yrow_bytes = static_cast<int>(a.y_stride * 2);
  const __amdgpu_buffer_rsrc_t yd = __builtin_amdgcn_make_buffer_rsrc(
      a.y + int64_t(tw0) * a.y_stride + fw0, 0, rows > 0 ? (rows - 1) * yrow_bytes + 256 : 0, kRsrcFlags);
  const bool table = rotate && rows > 0;               // a NULL table (no rotation) is never offset
  const __amdgpu_buffer_rsrc_t td = __builtin_amdgcn_make_buffer_rsrc(
      table ? const_cast<float*>(a.rope_tab) + int64_t(tw0) * (2 * kPairs) : reinterpret_cast<float*>(a.y), 0,
      table ? rows * kPairs * 8 : 0, kRsrcFlags);
  // (cos, sin) of the lane's pairs fb 16 + 4 g + 2 hf and the next one, token block tb: 16 bytes
  auto rot4 = [&](int tb, int fb, int g) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                          td, ((tb * 32 + col) * kPairs + fb * 16 + 4 * g + 2 * hf) * 8, 0, 0));
  };
  // The bf16 results go through this wave's 32 KB of LDS (free once every wave is past the last
  // barrier: the final k-step reads only registers), token-major with 256 B per token, so that
  // each store instruction then writes four whole output rows instead of 16 B of 32 rows.  The
  // 16-byte chunk c of token row r sits at slot c ^ (r & 15), which keeps the row-segment reads
  // on disjoint banks.
  lds_u16* eb = (wave < 2 ? (lds_u16*)as : (lds_u16*)bs) + (wave & 1) * (128 * 128);
  // The table loads run kAhead (token block, feature block) steps ahead of their use.
  float4 rt[kAhead + 1][4];
  auto fetch = [&](int i) {                            // step i = 4 tb + fb
#pragma unroll
    for (int g = 0; g < 4; ++g) rt[i % (kAhead + 1)][g] = rot4(i >> 2, i & 3, g);
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fetch(i);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tb = i >> 2, fb = i & 3;
    if (i + kAhead < 16) fetch(i + kAhead);
    const int erow = tb * 32 + col;
    f32x16_t v = acc[fb][tb];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = fb * 32 + 8 * g + 4 * hf;         // head-dim index of register 4 g
      v[4 * g + 0] += __uint_as_float(bw[fb][g].x << 16);
      v[4 * g + 1] += __uint_as_float(bw[fb][g].x & 0xffff0000u);
      v[4 * g + 2] += __uint_as_float(bw[fb][g].y << 16);
      v[4 * g + 3] += __uint_as_float(bw[fb][g].y & 0xffff0000u);
      if (rotate) {
        const float4 r = rt[i % (kAhead + 1)][g];
        const float cs[2] = {r.x, r.z}, sn[2] = {r.y, r.w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float x = v[4 * g + 2 * h], y = v[4 * g + 2 * h + 1];
          v[4 * g + 2 * h] = __builtin_fmaf(x, cs[h], -(y * sn[h]));
          v[4 * g + 2 * h + 1] = __builtin_fmaf(x, sn[h], y * cs[h]);
        }
      }
      const uint2 w = make_uint2(pack_bf16x2(v[4 * g + 0], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
      const int slot = (d0 >> 3) ^ (erow & 15);
      *reinterpret_cast<lds_u32x2*>(eb + erow * 128 + slot * 8 + 4 * hf) = u32x2_t{w.x, w.y};
    }
  }
  // row segments out: instruction j covers token rows 4 j .. 4 j + 3, lane l the 16-byte chunk l & 15
  // of row 4 j + (l >> 4); a wave's LDS writes complete in order before its reads
  const int sc = lane & 15;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int r = 4 * j + (lane >> 4);
    const u32x4_t w = *reinterpret_cast<const lds_u32x4*>(eb + r * 128 + (sc ^ (r & 15)) * 8);
    __builtin_amdgcn_raw_buffer_store_b128(w, yd, r * yrow_bytes + sc * 16, 0, 0);
  }
}

// (cos, sin) of pair p of row i, one thread per (row, pair), with the rotation arithmetic every RoPE
// route shares (rope_math.hpp): the values the streaming pass and the attention's Q load use.
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTabArgs a) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(a.n) * kPairs) return;
  const int row = static_cast<int>(i / kPairs), pair = static_cast<int>(i - int64_t(row) * kPairs);
  float c, s;
  rope_cos_sin(a.coords[3 * int64_t(row) + rope_axis(pair, a.tab)], a.tab.freq[pair], c, s);
  reinterpret_cast<float2*>(a.out)[i] = make_float2(c, s);
}

}  // namespace

hipError_t launch_rope_table(const RopeTabArgs& a, hipStream_t stream) {
  const int64_t total = int64_t(a.n) * kPairs;
  void* args[] = {const_cast<RopeTabArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rope_table_kernel),
                         dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), args, 0, stream);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel), dim3(a.tiles_f * a.tiles_t), dim3(kThreads),
                         args, 0, stream);
}

}  // namespace h3
