// Full bidirectional attention forward with MM-RoPE on Q, for gfx950.
//
// Per head: O = softmax(Q~ K~^T * scale) V over all rows, no mask (the open
// release runs full attention: "Inside MiniMax H3: One DiT Stream for Text,
// Video, and Stereo Audio", section 6).  K arrives already rotated; Q is rotated
// in registers while its tile is loaded (or arrives rotated, rope_q == 0).
//
// Work split.  A workgroup of kWaves waves owns kBM = 32 * kQB * kWaves query
// rows of one head; each wave owns kQB blocks of 32 query rows and keeps their
// rotated Q in registers for the whole kernel.  Every K or V operand a wave
// reads from LDS feeds kQB MFMAs (one per query block).  The build uses kQB = 1
// and eight waves (256 rows, two waves per SIMD); kQB = 2 (one wave per SIMD,
// half the LDS traffic per MFMA) still compiles but runs slower, because a
// wave's own exponentials then stall its MFMAs and the compiler shuffles the
// accumulators between register files.  The workgroup streams the head's K and V in
// tiles of kBN keys through three LDS buffers with one barrier per tile: the
// next tile's loads are in flight while the current tile is computed, and the
// two waves on each SIMD work half a tile apart (see the tile loop).  The
// loads use a buffer descriptor rebased on every tile, so rows past the end of
// the sequence read as zero without any per-lane test.
//
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form so that a
// query is a column of every accumulator:
//   S^T[key][query] = K~ . Q~^T   (A = K tile rows from LDS, B = Q~ registers)
//   O^T[d][query]  += V^T . P^T    (A = V^T read from the row-major V tile with
//                                   ds_read_b64_tr_b16, B = P taken straight
//                                   from the S^T accumulators as bf16)
// With queries in columns, every lane holds one query and 16 of its scores per
// 32-key block, so a row max is an in-lane max plus one exchange with the lane
// 32 away, and the row sum stays per lane until the end.  The contraction order
// of the PV product is free, so the keys fed to each PV step are the ones the
// S^T accumulator layout leaves in that lane.
//
// Online softmax in base 2, biased.  Q~ is pre-scaled by scale * log2(e): with
// rope_q set, Q is rotated and scaled in binary32 and rounded to bf16 once; a
// Q~ that arrives rotated (and so already rounded) is rounded again after the
// scaling.  Every score chain starts from an accumulator holding -m, the row's running
// reference max in those units: the MFMA itself returns s - m, so P = exp2 of
// the accumulator with no per-score arithmetic.  The reference is raised only
// when a tile's probabilities get large: each lane sums its tile's P (v_dot2 on
// the bf16 P, i.e. exactly the weights that multiply V); if any lane's sum
// exceeds 2^8 - which bounds every single P - the wave takes a rare slow path
// that raises the reference to the new max, rescales O and l, and recomputes
// the tile.  So every P is <= 2^8 and the result is exact up to rounding.
#include "launch.hpp"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

#ifndef H3_ATTN_WAVES
#define H3_ATTN_WAVES 8
#endif
#ifndef H3_ATTN_QB
#define H3_ATTN_QB 1
#endif
#ifndef H3_ATTN_BN
#define H3_ATTN_BN 64
#endif
#ifndef H3_ATTN_VSTR
#define H3_ATTN_VSTR (kHeadDim + 32)
#endif

constexpr int kWaves = H3_ATTN_WAVES;
constexpr int kQB = H3_ATTN_QB;              // 32-row query blocks per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kQB * kWaves;       // query rows per workgroup
constexpr int kBN = H3_ATTN_BN;              // keys per tile (multiple of 32)
constexpr int kKB = kBN / 32;                // 32-key blocks per tile
constexpr int kKStr = kHeadDim + 8;          // LDS row stride of the K tile, elements (272 B)
// LDS row stride of the V tile, elements: 320 B puts the four rows and two
// column halves of each transpose read on disjoint banks
constexpr int kVStr = H3_ATTN_VSTR;
constexpr int kKTile = kBN * kKStr;          // elements per K buffer
constexpr int kVTile = kBN * kVStr;          // elements per V buffer
constexpr int kChunks = kBN * 16 / kThreads; // 16-byte chunks per thread per tensor per tile
constexpr int kRowsPerPass = kThreads / 16;  // rows covered by one pass of all threads
constexpr int kNBuf = 3;                     // K/V tile buffers
constexpr float kMaxTileSum = 256.0f;        // a lane's tile sum of P above 2^8 raises the reference
constexpr int kRsrcFlags = 0x00020000;       // raw buffer, 32-bit data format
static_assert(kBN % 32 == 0 && kChunks >= 1 && kBN * 16 == kChunks * kThreads, "tile shape");

struct True { static constexpr bool value = true; };
struct False { static constexpr bool value = false; };

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two bf16 (low, high) times f, rounded back to bf16
__device__ __forceinline__ uint32_t scale_word(uint32_t w, float f) {
  return pack_bf16x2(__uint_as_float(w << 16) * f, __uint_as_float(w & 0xffff0000u) * f);
}

// max / sum over the two lanes that hold the same query (l and l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  const u32x2_t r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const u32x2_t r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Unit run by full-unit workgroup i of g.  Workgroups are dispatched to the chip's eight
// XCDs round-robin (workgroup i on XCD i mod 8), and each XCD has its own L2.  XCD x gets the
// contiguous units [start_x, start_x + cnt_x) in order, so the workgroups resident on one XCD
// at a time are consecutive query blocks of one head: they read the same K and V tiles, which
// its L2 then fetches once for all of them.  A bijection on [0, g) for any g.
__device__ __forceinline__ int xcd_unit(int i, int g) {
  const int x = i & 7, k = i >> 3;
  return x * (g >> 3) + min(x, g & 7) + k;
}

__global__ __launch_bounds__(kThreads, kQB == 1 ? 2 : 1) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kNBuf * kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kNBuf * kVTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column / A-operand row of this lane
  const int hf = lane >> 5;    // which 8-element half of a 16-deep k chunk
  const int nqb = (a.n + kBM - 1) / kBM;
  const int ntiles = (a.n + kBN - 1) / kBN;
  // work unit = (head, query block).  The first n_full workgroups take one unit each over all
  // keys; each later unit is split over `split` workgroups, part p taking key tiles
  // [p * tiles_per_split, ...), and leaves an unnormalised partial result for the merge.
  int unit = blockIdx.x, part = -1, t_begin = 0, t_end = ntiles;
  if (unit < a.n_full) {
    unit = xcd_unit(unit, a.n_full);
  } else {
    const int r = unit - a.n_full;
    unit = a.n_full + r / a.split;
    part = r - (r / a.split) * a.split;
    t_begin = part * a.tiles_per_split;
    t_end = min(t_begin + a.tiles_per_split, ntiles);
  }
  const int head = unit / nqb;
  const int qblk = unit - head * nqb;
  const float qscale = a.scale_log2;

  // ---- Q~ fragments: B operand of S^T; lane holds dims 16c + 8hf .. +7 of its query
  int qrow[kQB];
  bf16x8_t qf[kQB][8];
#pragma unroll
  for (int i = 0; i < kQB; ++i) {
    qrow[i] = qblk * kBM + (wave * kQB + i) * 32 + col;
    const bool qvalid = qrow[i] < a.n;
    const uint16_t* qp = a.q + (qvalid ? qrow[i] : 0) * a.stride_qkv + head * kHeadDim + 8 * hf;
    // the row's (t, h, w), picked per pair by selects (an indexed array would be placed in LDS)
    float pt = 0.0f, ph = 0.0f, pw = 0.0f;
    if (a.rope_q && qvalid) {
      pt = a.coords[3 * qrow[i] + 0];
      ph = a.coords[3 * qrow[i] + 1];
      pw = a.coords[3 * qrow[i] + 2];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qvalid) x = *reinterpret_cast<const uint4*>(qp + 16 * c);
      if (a.rope_q) {
        // rotation and the pre-scale by scale * log2(e) in binary32, then one bf16 rounding
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pair = 8 * c + 4 * hf + p;
          float cs, sn;
          const int ax = rope_axis(pair, a.tab);
          rope_cos_sin(ax == 0 ? pt : (ax == 1 ? ph : pw), a.tab.freq[pair], cs, sn);
          w[p] = rope_rotate_word(w[p], cs * qscale, sn * qscale);
        }
        x = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        // Q~ arrives rotated and rounded: pre-scale by scale * log2(e), rounding once more
        x = make_uint4(scale_word(x.x, qscale), scale_word(x.y, qscale), scale_word(x.z, qscale),
                       scale_word(x.w, qscale));
      }
      qf[i][c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- K / V tile loads: thread covers rows (tid >> 4) + kRowsPerPass * r, bytes 16 * (tid & 15)
  const int row_bytes = a.stride_qkv * 2;
  const int64_t head_off = int64_t(head) * kHeadDim * 2;
  const int64_t span = int64_t(a.n - 1) * row_bytes + kHeadDim * 2;   // bytes from the head base to its last byte
  const char* kbase = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v) + head_off;
  int voff[kChunks];
  int lds_k_st[kChunks], lds_v_st[kChunks];
#pragma unroll
  for (int r = 0; r < kChunks; ++r) {
    const int row = (tid >> 4) + kRowsPerPass * r;
    voff[r] = row * row_bytes + (tid & 15) * 16;
    lds_k_st[r] = row * kKStr + (tid & 15) * 8;
    lds_v_st[r] = row * kVStr + (tid & 15) * 8;
  }
  u32x4_t kr[kChunks], vr[kChunks];
  auto rsrc = [&](const char* base, int t) {
    const int64_t off = int64_t(t) * kBN * row_bytes;
    // bytes left from this tile's first row; the check on the tensor size keeps it below 2^32
    const int64_t left = span - off > 0 ? span - off : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), 0, static_cast<int>(static_cast<uint32_t>(left)),
                                             kRsrcFlags);
  };
  auto load_tile = [&](int t) {
    const __amdgpu_buffer_rsrc_t kd = rsrc(kbase, t);
    const __amdgpu_buffer_rsrc_t vd = rsrc(vbase, t);
#pragma unroll
    for (int r = 0; r < kChunks; ++r)
      kr[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kd, voff[r], 0, 0));
#pragma unroll
    for (int r = 0; r < kChunks; ++r)
      vr[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vd, voff[r], 0, 0));
  };
  lds_u16* ksl = (lds_u16*)ks;
  lds_u16* vsl = (lds_u16*)vs;
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < kChunks; ++r)
      *reinterpret_cast<lds_u32x4*>(ksl + buf * kKTile + lds_k_st[r]) = kr[r];
#pragma unroll
    for (int r = 0; r < kChunks; ++r)
      *reinterpret_cast<lds_u32x4*>(vsl + buf * kVTile + lds_v_st[r]) = vr[r];
  };

  // per-lane LDS read bases
  // K (A of S^T): row = key 32b + col, elements 16c + 8hf
  const int k_rd = col * kKStr + 8 * hf;
  // V^T (A of O^T) via transpose reads: in each 16-lane group g, lanes 4r + j
  // address row (16kc + 8c + 4(g >> 1) + r), columns 32db + 16(g & 1) + 4j; lane i
  // of the group receives column i of the four rows.
  const int g = lane >> 4;
  const int v_rd = (4 * (g >> 1) + ((lane >> 2) & 3)) * kVStr + 16 * (g & 1) + 4 * (lane & 3);

  f32x16_t oacc[kQB][4];
  f32x16_t cinit[kQB];   // -m_ref in every entry: the start of each score chain
  float m_ref[kQB];      // running reference max of the row, log2 units
  float l_part[kQB];
#pragma unroll
  for (int i = 0; i < kQB; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[i][d] = f32x16_t{};
    cinit[i] = f32x16_t{};
    m_ref[i] = 0.0f;
    l_part[i] = 0.0f;
  }
  const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // S^T (scaled, biased) for every query block and 32-key block of K buffer `buf`
  auto scores = [&](int buf, f32x16_t (&s)[kQB][kKB]) {
    const lds_u16* kt = ksl + buf * kKTile + k_rd;
    // all K operands of the tile first, so the LDS reads overlap the MFMA chains
    bf16x8_t kop[kKB][8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int b = 0; b < kKB; ++b) kop[b][c] = *reinterpret_cast<const lds_bf16x8*>(kt + 32 * b * kKStr + 16 * c);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int b = 0; b < kKB; ++b)
#pragma unroll
        for (int i = 0; i < kQB; ++i) s[i][b] = mfma32(kop[b][c], qf[i][c], c == 0 ? cinit[i] : s[i][b]);
  };

  // P = exp2(S) as bf16 (pb[b][half] is the B operand of PV chunk 2b + half);
  // returns this lane's sum of the block's P
  auto probs = [&](const f32x16_t (&s)[kKB], bf16x8_t (&pb)[kKB][2]) {
    float lt = 0.0f;
#pragma unroll
    for (int b = 0; b < kKB; ++b)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        bf16x2_t p;
        p[0] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[b][r]));
        p[1] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[b][r + 1]));
        lt = __builtin_amdgcn_fdot2_f32_bf16(p, ones, lt, false);
        pb[b][r >> 3][r & 7] = p[0];
        pb[b][r >> 3][(r & 7) + 1] = p[1];
      }
    return lt;
  };

  // row max of one query block's tile over both lanes of each query
  auto tile_max = [&](const f32x16_t (&s)[kKB]) {
    // NaN-propagating maximum: lowers to v_maximum3_f32 with no input canonicalisation
    float mt = s[0][0];
#pragma unroll
    for (int b = 0; b < kKB; ++b)
#pragma unroll
      for (int r = (b == 0 ? 1 : 0); r < 16; ++r) mt = __builtin_elementwise_maximum(mt, s[b][r]);
    return pair_max(mt);
  };

  // V^T operand of 16-key chunk kc and 32-dim block db of V buffer `buf`
  auto vread = [&](int buf, int kc, int db) {
    const lds_u16* vt = vsl + buf * kVTile + v_rd + (16 * kc) * kVStr + 32 * db;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(const_cast<lds_u16*>(vt)));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4*>(const_cast<lds_u16*>(vt + 8 * kVStr)));
    const i16x4_t both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, both);
  };
  // O^T += V^T P^T over the tile's 16-key chunks and four 32-dim blocks of V buffer `buf`; the
  // operands of the first kVPre chunks may have been read already (pre).  The lagging waves read
  // all of them while they wait at the barrier.
  constexpr int kVPre = 2 * kKB;
  auto pv_pre = [&](int buf, const bf16x8_t (&pb)[kQB][kKB][2], const bf16x8_t (&pre)[kVPre][4], auto use_pre) {
#pragma unroll
    for (int kc = 0; kc < 2 * kKB; ++kc)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        bf16x8_t vop;
        if constexpr (decltype(use_pre)::value) {
          vop = kc < kVPre ? pre[kc < kVPre ? kc : 0][db] : vread(buf, kc, db);
        } else {
          vop = vread(buf, kc, db);
        }
#pragma unroll
        for (int i = 0; i < kQB; ++i) oacc[i][db] = mfma32(vop, pb[i][kc >> 1][kc & 1], oacc[i][db]);
      }
  };
  auto pv = [&](int buf, const bf16x8_t (&pb)[kQB][kKB][2]) {
    bf16x8_t none[kVPre][4];
    pv_pre(buf, pb, none, False{});
  };

  // keys past the end of the sequence take no weight (last tile only)
  auto mask_tail = [&](f32x16_t (&s)[kQB][kKB], int key0) {
#pragma unroll
    for (int b = 0; b < kKB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= a.n) {
#pragma unroll
          for (int i = 0; i < kQB; ++i) s[i][b][r] = -__builtin_inff();
        }
      }
  };

  // One tile: scores, softmax, PV.  The first tile sets the reference max (O and
  // l are still zero); the last one masks keys >= n.
  auto softmax_step = [&](int t, auto first, auto last, bf16x8_t (&pb)[kQB][kKB][2]) {
    f32x16_t s[kQB][kKB];
    scores(t % kNBuf, s);
    if constexpr (decltype(last)::value) mask_tail(s, t * kBN);
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int i = 0; i < kQB; ++i) {
        const float mt = tile_max(s[i]);
#pragma unroll
        for (int b = 0; b < kKB; ++b) s[i][b] -= mt;
        cinit[i] -= mt;
        m_ref[i] = mt;
      }
    }
    float lt[kQB];
#pragma unroll
    for (int i = 0; i < kQB; ++i) lt[i] = probs(s[i], pb[i]);
    if constexpr (!decltype(first)::value) {
      bool big = false;
#pragma unroll
      for (int i = 0; i < kQB; ++i) big = big || lt[i] > kMaxTileSum;
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        // raise each reference by the tile's excess (never lower it), rescale, redo the tile
#pragma unroll
        for (int i = 0; i < kQB; ++i) {
          const float delta = __builtin_elementwise_maximum(tile_max(s[i]), 0.0f);
#pragma unroll
          for (int b = 0; b < kKB; ++b) s[i][b] -= delta;
          cinit[i] -= delta;
          m_ref[i] += delta;
          const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
          for (int d = 0; d < 4; ++d) oacc[i][d] *= alpha;
          l_part[i] *= alpha;
          lt[i] = probs(s[i], pb[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kQB; ++i) l_part[i] += lt[i];
  };
  auto step = [&](int t, auto first, auto last) {
    bf16x8_t pb[kQB][kKB][2];
    softmax_step(t, first, last, pb);
    pv(t % kNBuf, pb);
  };


  // Tiles over [t_begin, t_end) in three LDS buffers (tile t in buffer t % 3), one barrier per
  // tile.  Each wave loads its share of tile t + 1 into registers and stores it between the
  // barriers that open tiles t and t + 1.  The two waves that share a SIMD are kept half a tile
  // apart, so that one's softmax runs under the other's MFMAs instead of both competing for the
  // matrix pipe and then both leaving it idle: the leading half (waves 0 .. kWaves/2 - 1) runs
  // scores, softmax and PV of tile t after barrier t; the lagging half runs PV of tile t - 1 and
  // then scores and softmax of tile t, keeping P in registers across the barrier.  The lagging
  // half issues its reads of V of tile t - 1 while it waits at barrier t and they may complete
  // after it, hence the third buffer.  Each wave's own arithmetic is the same in both halves, so
  // the result does not depend on the half.  The last step masks keys >= n, which only bites on
  // the sequence's last tile.
  load_tile(t_begin);
  store_tile(t_begin % kNBuf);
  __syncthreads();
  // waves w and w + kWaves / 2 share a SIMD; the second half runs half a tile behind
  const bool lag = wave >= kWaves / 2;
  if (!lag) {
    if (t_end - t_begin == 1) {
      step(t_begin, True{}, True{});
    } else {
      load_tile(t_begin + 1);
      step(t_begin, True{}, False{});
      store_tile((t_begin + 1) % kNBuf);
      for (int t = t_begin + 1; t + 1 < t_end; ++t) {
        __syncthreads();
        load_tile(t + 1);
        step(t, False{}, False{});
        store_tile((t + 1) % kNBuf);
      }
      __syncthreads();
      step(t_end - 1, False{}, True{});
    }
  } else {
    bf16x8_t pb[kQB][kKB][2];
    if (t_end - t_begin == 1) {
      softmax_step(t_begin, True{}, True{}, pb);
      pv(t_begin % kNBuf, pb);
    } else {
      load_tile(t_begin + 1);
      softmax_step(t_begin, True{}, False{}, pb);
      store_tile((t_begin + 1) % kNBuf);
      for (int t = t_begin + 1; t + 1 < t_end; ++t) {
        // V of tile t - 1 has been visible since barrier t - 1.  Barrier t is taken in two
        // halves (release, then wait and acquire) so that the PV operands are read while this
        // wave waits for the others.
        bf16x8_t pre[kVPre][4];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
#pragma unroll
        for (int kc = 0; kc < kVPre; ++kc)
#pragma unroll
          for (int db = 0; db < 4; ++db) pre[kc][db] = vread((t - 1) % kNBuf, kc, db);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        load_tile(t + 1);
        pv_pre((t - 1) % kNBuf, pb, pre, True{});
        softmax_step(t, False{}, False{}, pb);
        store_tile((t + 1) % kNBuf);
      }
      __syncthreads();
      pv((t_end - 2) % kNBuf, pb);
      softmax_step(t_end - 1, False{}, True{}, pb);
      pv((t_end - 1) % kNBuf, pb);
    }
  }

  if (part >= 0) {
    // partial result of one key range: O^T unnormalised (float32) and (m, l) per query row
    const int slot = blockIdx.x - a.n_full;
#pragma unroll
    for (int i = 0; i < kQB; ++i) {
      const float l_tot = pair_sum(l_part[i]);
      const int rloc = (wave * kQB + i) * 32 + col;
      float* po = a.ws_o + (int64_t(slot) * kBM + rloc) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(po + 32 * db + 8 * r + 4 * hf) =
              make_float4(oacc[i][db][4 * r + 0], oacc[i][db][4 * r + 1], oacc[i][db][4 * r + 2],
                          oacc[i][db][4 * r + 3]);
      if (hf == 0)
        *reinterpret_cast<float2*>(a.ws_ml + (int64_t(slot) * kBM + rloc) * 2) = make_float2(m_ref[i], l_tot);
    }
    return;
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int i = 0; i < kQB; ++i) {
    const float l_tot = pair_sum(l_part[i]);
    if (qrow[i] < a.n) {
      const float inv = 1.0f / l_tot;
      uint16_t* op = a.o + qrow[i] * a.stride_o + head * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * db + 8 * r + 4 * hf;
          const uint2 w = make_uint2(pack_bf16x2(oacc[i][db][4 * r + 0] * inv, oacc[i][db][4 * r + 1] * inv),
                                     pack_bf16x2(oacc[i][db][4 * r + 2] * inv, oacc[i][db][4 * r + 3] * inv));
          *reinterpret_cast<uint2*>(op + d) = w;
        }
      if (a.lse != nullptr && hf == 0)
        a.lse[head * a.n + qrow[i]] = (m_ref[i] + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

// Merge of the key-range partials of split units: per query row, with m = max_p m_p and
// w_p = 2^(m_p - m), O = sum_p w_p O_p / sum_p w_p l_p and LSE = (m + log2 sum_p w_p l_p) ln 2.
// Block: 8 rows x 16 lanes of 8 head-dim values; grid (rows / 8, split units).
__global__ __launch_bounds__(128) void attn_merge_kernel(FwdArgs a) {
  const int nqb = (a.n + kBM - 1) / kBM;
  const int su = blockIdx.y;                               // split unit
  const int unit = a.n_full + su;
  const int head = unit / nqb, qblk = unit - head * nqb;
  const int rloc = blockIdx.x * 8 + (threadIdx.x >> 4), d0 = 8 * (threadIdx.x & 15);
  const int row = qblk * kBM + rloc;
  if (row >= a.n) return;
  float m = -__builtin_inff();
  for (int p = 0; p < a.split; ++p) m = fmaxf(m, a.ws_ml[(int64_t(su * a.split + p) * kBM + rloc) * 2]);
  float l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int p = 0; p < a.split; ++p) {
    const int64_t slot = int64_t(su * a.split + p) * kBM + rloc;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + slot * 2);
    const float w = __builtin_amdgcn_exp2f(ml.x - m);
    l = __builtin_fmaf(w, ml.y, l);
    const float4 x0 = *reinterpret_cast<const float4*>(a.ws_o + slot * kHeadDim + d0);
    const float4 x1 = *reinterpret_cast<const float4*>(a.ws_o + slot * kHeadDim + d0 + 4);
    o[0] = __builtin_fmaf(w, x0.x, o[0]); o[1] = __builtin_fmaf(w, x0.y, o[1]);
    o[2] = __builtin_fmaf(w, x0.z, o[2]); o[3] = __builtin_fmaf(w, x0.w, o[3]);
    o[4] = __builtin_fmaf(w, x1.x, o[4]); o[5] = __builtin_fmaf(w, x1.y, o[5]);
    o[6] = __builtin_fmaf(w, x1.z, o[6]); o[7] = __builtin_fmaf(w, x1.w, o[7]);
  }
  const float inv = 1.0f / l;
  uint4 out;
  out.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  out.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  out.z = pack_bf16x2(o[4] * inv, o[5] * inv);
  out.w = pack_bf16x2(o[6] * inv, o[7] * inv);
  *reinterpret_cast<uint4*>(a.o + int64_t(row) * a.stride_o + head * kHeadDim + d0) = out;
  if (a.lse != nullptr && d0 == 0) a.lse[head * a.n + row] = (m + __log2f(l)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.n + kBM - 1) / kBM;
  const int units = nqb * a.heads;
  const int split_units = units - a.n_full;
  const dim3 grid(a.n_full + split_units * a.split), block(kThreads);
  FwdArgs b = a;
  if (split_units > 0) b.ws_ml = b.ws_o + int64_t(split_units) * a.split * kBM * kHeadDim;
  void* args[] = {&b};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel), grid, block, args, 0, stream);
  if (e != hipSuccess || split_units == 0) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_merge_kernel), dim3(kBM / 8, split_units), dim3(128),
                         args, 0, stream);
}

void attn_fwd_schedule(int32_t n, int32_t heads, int32_t cus, int32_t* n_full, int32_t* split,
                       int32_t* tiles_per_split, int64_t* ws_bytes) {
  const int nqb = (n + kBM - 1) / kBM;
  const int ntiles = (n + kBN - 1) / kBN;
  const int units = nqb * heads;
  *n_full = units;
  *split = 1;
  *tiles_per_split = ntiles;
  *ws_bytes = 0;
  // One workgroup per CU: the last wave holds rem = units mod cus units and the other CUs idle
  // for the rest of it.  Cutting those units into s key ranges of tps tiles makes the last
  // stretch ceil(rem s / cus) waves of tps / ntiles of a unit each, plus the merge, which reads
  // and writes the partials (about rem s 133 KB at ~4 TB/s, against ~1.75 us per key tile of a
  // unit).  Take the s in 2 .. 8 (parts of at least 4 tiles) that minimises that, and split only
  // if it saves at least a tenth of a unit.
  const int rem = cus > 0 ? units % cus : 0;
  if (units < cus || rem == 0 || ntiles < 8) return;
  const double part_bytes = double(kBM) * (kHeadDim + 2) * 4;
  double best = 0.9;
  int best_s = 1, best_tps = ntiles;
  for (int s = 2; s <= 8 && 4 * s <= ntiles; ++s) {
    const int tps = (ntiles + s - 1) / s;
    const int parts = (ntiles + tps - 1) / tps;        // every part non-empty
    const int waves = (rem * parts + cus - 1) / cus;
    const double merge = double(rem) * parts * part_bytes / 4.0e12 / (ntiles * 1.75e-6);
    const double t = double(waves) * tps / ntiles + merge;
    if (t < best - 1e-9) {
      best = t;
      best_s = parts;
      best_tps = tps;
    }
  }
  if (best_s < 2) return;
  *n_full = units - rem;
  *split = best_s;
  *tiles_per_split = best_tps;
  *ws_bytes = int64_t(rem) * best_s * kBM * (kHeadDim + 2) * 4;
}

}  // namespace h3
