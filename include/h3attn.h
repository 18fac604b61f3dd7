/*
 * h3attn.h - C ABI of the MI355X (gfx950) library for MM-RoPE + full
 * bidirectional attention over one packed text / video / stereo-audio sequence.
 *
 * The operation is the attention of the single-stream Omni-Transformer
 * described in "Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo
 * Audio" (section 2: text, reference media, noisy video latents and noisy audio
 * latents share one attention sequence; section 4: RoPE coordinates on a shared
 * physical timeline; section 6: full attention) and in "MiniMax H3 - one
 * transformer that denoises video and audio together" (latent frames and the
 * 1x2x2 patch grid, the 40 Hz clock and the 5/3 frame rescale, text as 1-D RoPE,
 * position_ids -> rope() -> rotate Q and K, the normalised spatial grid).
 *
 * Conventions for every call:
 *  - All buffers are owned by the caller.  The library allocates no device
 *    memory at run time and keeps no state beyond a per-device cache of device
 *    properties; the one exception is the static scratch array of
 *    h3attn_forward_noalloc (H3ATTN_NOALLOC_SCRATCH_BYTES per device, part of
 *    the loaded code object).
 *  - Device calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the default stream) and never synchronise.
 *  - Arguments are validated before any write or launch: on error nothing has
 *    been written and nothing has been launched.
 *  - Return value: H3ATTN_OK (0) or one of the negative codes below.  No C++
 *    exception crosses this boundary.  The calls are thread-safe.
 *  - Q, K, V, O tensors are bfloat16, row-major [n_tokens][n_heads][head_dim]
 *    with a row stride given in elements (>= n_heads * head_dim, a multiple of
 *    8), base pointers 16-byte aligned.  head_dim must be 128.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  H3ATTN_OK = 0,
  H3ATTN_EINVAL = -1,       /* null pointer, bad size, bad config, misalignment */
  H3ATTN_ERANGE = -2,       /* capacity too small; coordinate or size out of exact range */
  H3ATTN_EUNSUPPORTED = -3, /* current device is not gfx950 */
  H3ATTN_EHIP = -4,         /* HIP runtime or launch error */
  H3ATTN_ESCRATCH = -5      /* shape needs more than h3attn_forward_noalloc's static scratch */
};

/* Segment kinds of the packed sequence. */
enum { H3_SEG_TEXT = 0, H3_SEG_VIDEO = 1, H3_SEG_AUDIO = 2 };

/*
 * One segment of the packed sequence.  Times are integers in thirds of one
 * clock unit (one audio latent, 1/40 s), so that the video advance of
 * 4 source frames x 5/3 = 20/3 units per latent frame is exact.
 *
 *   kind      H3_SEG_TEXT | H3_SEG_VIDEO | H3_SEG_AUDIO
 *   frames    TEXT: tokens | VIDEO: latent frames (1 = still or reference image)
 *             | AUDIO: 40 Hz steps.  0 is allowed (no rows).
 *   grid_h    VIDEO: patch rows (22 for a 44x80 latent sheet) | TEXT, AUDIO: 1
 *   grid_w    VIDEO: patch columns (40) | AUDIO: channels (2) | TEXT: 1
 *   t0_thirds time of the first frame / token / step, in thirds
 *   dt_thirds advance per frame: VIDEO 20, AUDIO 3, TEXT 3 (any value allowed)
 */
typedef struct {
  int32_t kind;
  int32_t frames;
  int32_t grid_h;
  int32_t grid_w;
  int32_t t0_thirds;
  int32_t dt_thirds;
} h3attn_segment;

/*
 * Rotary configuration: head_dim (must be 128) is split into three contiguous
 * sections for the t, h and w axes (sec[0] + sec[1] + sec[2] == head_dim, each
 * even and >= 0).  Inside section a, pair p rotates dims (o_a + 2p, o_a + 2p + 1)
 * by pos_a * theta[a]^(-2p / sec[a]); theta[a] > 0.  The inverse frequencies
 * are computed, not loaded ("MiniMax H3 - one transformer that denoises video
 * and audio together", inv_freq paragraph).  The workloads here use
 * {128, {32, 48, 48}, {1e4, 1e4, 1e4}}.
 */
typedef struct {
  int32_t head_dim;
  int32_t sec[3];
  double theta[3];
} h3attn_rope_cfg;

/*
 * Host call.  Builds the (t, h, w) coordinate of every packed row.
 *   Rows follow the segment order.  VIDEO rows are frame-major, then row-major
 *   (r, c); AUDIO rows step-major, channel-minor; TEXT rows in order.
 *   t = RN32(t3 / 3) with t3 = t0_thirds + f * dt_thirds (exact, round to
 *   nearest even).  TEXT: h = w = 0.  AUDIO: h = 0, w = channel (left and right
 *   share t: section 4 of the thread).  VIDEO: the patch grid normalised by
 *   sqrt(grid_h * grid_w) and centred on the [0, 32) canvas with the aspect kept:
 *   s = 16 / sqrt(gh * gw); h_r = RN32(16 + (2r + 1 - gh) * s),
 *   w_c = RN32(16 + (2c + 1 - gw) * s), evaluated in binary64 without fusion.
 * Arguments:
 *   segs, n_segs     segment table (n_segs >= 0; segs may be NULL iff n_segs == 0)
 *   coords           host float32 [capacity_rows][3], or NULL to only count
 *   capacity_rows    rows available in coords
 *   n_tokens         out: number of rows (always written on success)
 * Errors: EINVAL (bad kind or sizes, null n_tokens), ERANGE (|t3| >= 2^24,
 *   rows >= 2^31, or capacity too small; *n_tokens still holds the count when
 *   only the capacity is short).
 */
int h3attn_build_coords(const h3attn_segment* segs, int32_t n_segs, float* coords,
                        int64_t capacity_rows, int64_t* n_tokens);

/*
 * Device call.  Rotates Q and/or K by the rows' coordinates (the rope() step of
 * the position chain; V is never rotated).  Out-of-place, or in place when
 * the output pointer equals the input pointer.  Apart from that exact in-place
 * case, an output shares no byte with another output, an input or the
 * coordinates (EINVAL); views that interleave rows of one buffer without
 * sharing bytes, such as the Q and K slots of a [N][3][H][128] projection
 * output, are accepted.  The cos/sin of each
 * (row, pair) angle are formed once per row from a binary64 angle and reused
 * over all heads; the rotation runs in float32 and rounds to bfloat16 (nearest
 * even).
 *   cfg            rotary configuration (host pointer)
 *   coords_dev     device float32 [n_tokens][3]
 *   q_in, q_out    bf16 [n_tokens][n_heads][128]; both NULL to skip Q
 *   k_in, k_out    same for K; both NULL to skip K
 *   row_stride     elements between rows, for all four tensors
 * n_tokens == 0 is a no-op.  Errors: EINVAL, ERANGE (n_tokens * row_stride
 *   >= 2^31), EUNSUPPORTED, EHIP.
 */
int h3attn_rope_qk(const h3attn_rope_cfg* cfg, const float* coords_dev,
                   const void* q_in, void* q_out, const void* k_in, void* k_out,
                   int64_t n_tokens, int32_t n_heads, int64_t row_stride, void* stream);

/*
 * Device call.  Per head, O = softmax(Q~ K^T * scale) V over all n_tokens rows:
 * full bidirectional attention with no mask (section 6 of the thread; the open
 * release runs full attention).  K must already be rotated (h3attn_rope_qk with
 * q = NULL).  Q is rotated inside the kernel's Q-tile load when rope_q != 0,
 * or used as given when rope_q == 0 (already rotated).  The kernel multiplies
 * Q~ by scale * log2(e) and rounds it to bf16 for the matrix cores: with
 * rope_q != 0 the rotation and that scaling run in float32 and round once;
 * a pre-rotated Q~ (already rounded by h3attn_rope_qk) is rounded once more,
 * so the fused route is the more accurate of the two.
 *   cfg, coords_dev   as above (coords_dev may be NULL when rope_q == 0)
 *   q, k, v           bf16 [n_tokens][n_heads][128], row stride row_stride_qkv
 *   o                 out: bf16 [n_tokens][n_heads][128], row stride row_stride_o
 *   lse               out (optional, may be NULL): float32 [n_heads][n_tokens],
 *                     natural log of sum_j exp(scale * q~.k_j)
 *   scale             softmax scale; <= 0 selects 1/sqrt(128)
 * o must not alias q, k or v.  n_tokens == 0 is a no-op.  Errors: EINVAL,
 *   ERANGE, EUNSUPPORTED, EHIP.
 */
int h3attn_forward(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                   const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                   int64_t row_stride_o, float scale, void* stream);

/*
 * ---- Indexed AdaLN modulation around attention ----
 *
 * Sources: "MiniMax H3 - one transformer that denoises video and audio
 * together", AdaLN paragraphs (a sublayer input becomes norm(x) * (1 + scale) +
 * shift; H3 keeps a table indexed by (noise level, modality) and every row looks
 * up entry timestep_index * 3 + token_tag); "Inside MiniMax H3: One DiT Stream
 * for Text, Video, and Stereo Audio", section 5 (each block produces shift,
 * scale and gate for its attention and MLP paths, gathered per row).
 *
 * Readings where the pages are silent: norm is a layer norm without affine
 * ((x - mean) / sqrt(var + eps), biased variance over the row) or, on request, a
 * root-mean-square norm (x / sqrt(mean(x^2) + eps)); a gate scales the sublayer
 * output before it joins the residual stream (x + gate * y); token tags are
 * 0 text, 1 video, 2 audio.
 *
 * Conventions of both calls:
 *   x, y, h, x_out   bf16, row-major [n_rows][stride], 16-byte aligned, stride in
 *                    elements (>= hidden, multiple of 8)
 *   t_idx, tags      device int32 [n_rows]: entry e = t_idx * 3 + tags
 *   gate/shift/scale device bf16 table planes: entry e starts at plane + e * entry_stride
 *                    elements (for an [E][6][hidden] table in the order
 *                    shift_attn, scale_attn, gate_attn, shift_mlp, scale_mlp, gate_mlp,
 *                    pass table + k * hidden and entry_stride = 6 * hidden)
 *   n_entries        entries in the table (> 0)
 *   hidden           8 <= hidden <= H3ATTN_ADALN_MAX_HIDDEN, multiple of 8 (5,376 here)
 *   norm_kind        H3ATTN_LAYER_NORM or H3ATTN_RMS_NORM;  eps >= 0
 * Arithmetic is float32, each output rounded once to bf16 (nearest even).  A row
 * whose t_idx < 0, tag outside [0, 3) or entry >= n_entries reads no table entry;
 * its outputs are written as bf16 NaN.  n_rows == 0 is a no-op.  Errors: EINVAL
 * (sizes, alignment, overlaps, null pointers), ERANGE (n_rows >= 2^31),
 * EUNSUPPORTED, EHIP.
 */
#define H3ATTN_ADALN_MAX_HIDDEN 8192
enum { H3ATTN_LAYER_NORM = 0, H3ATTN_RMS_NORM = 1 };

/*
 * Device call.  h = norm(x) * (1 + scale[e]) + shift[e] per row (the modulated
 * input of a sublayer).  h may be x itself (in place); otherwise they must not
 * overlap.
 */
int h3attn_adaln_modulate(const void* x, int64_t x_stride, const int32_t* t_idx, const int32_t* tags,
                          const void* shift, const void* scale, int64_t entry_stride, int32_t n_entries,
                          void* h, int64_t h_stride, int64_t n_rows, int32_t hidden,
                          int32_t norm_kind, float eps, void* stream);

/*
 * Device call.  The gated residual of one sublayer fused with the modulated
 * norm of the next:
 *   x_out = bf16(x + gate[e] * y)
 *   h     = norm(x_out) * (1 + scale[e]) + shift[e]      (norm of the stored bf16 row)
 * x and y share xy_stride; x_out and h share out_stride.  x_out may be x itself
 * (in place, then out_stride == xy_stride); no other buffers may overlap.
 */
int h3attn_adaln_residual(const void* x, const void* y, int64_t xy_stride, const int32_t* t_idx,
                          const int32_t* tags, const void* gate, const void* shift, const void* scale,
                          int64_t entry_stride, int32_t n_entries, void* x_out, void* h,
                          int64_t out_stride, int64_t n_rows, int32_t hidden, int32_t norm_kind,
                          float eps, void* stream);

/*
 * ---- Attention projections with the rotary embedding in the epilogue ----
 *
 * Sources: "Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo
 * Audio", section 2 (every row shares one set of attention projections); "MiniMax
 * H3 - one transformer that denoises video and audio together", position-chain
 * paragraph (rope() rotates Q and K, V is not rotated).
 *
 * Device call.  y = x W^T (+ bias), then, for the leading rope_cols output
 * features (whole 128-wide heads), the rotation of h3attn_rope_qk applied to the
 * float32 results with each row's (cos, sin) from a table made by
 * h3attn_rope_table, then one rounding to bf16 (nearest even).  For the fused
 * QKV projection of H heads: W is [3 H 128][k] (Q rows, then K, then V),
 * rope_cols = 2 H 128, and y = [m][3][H][128] feeds h3attn_forward with
 * rope_q = 0 through strided views (row stride 3 H 128).
 * Readings: no bias unless given; W is stored [n_out][k] (row = output feature).
 *   x          bf16 [m][x_stride], w bf16 [n_out][w_stride], bias bf16 [n_out] or NULL
 *   y          out: bf16 [m][y_stride]; must not overlap x, w or bias
 *   n_out      multiple of H3ATTN_LINEAR_TILE (256);  k multiple of H3ATTN_LINEAR_KSTEP (64)
 *   rope_table_dev  device float32 [m][64][2] from h3attn_rope_table over the
 *              rows of x, 16-byte aligned; read only when rope_cols > 0 (else may
 *              be NULL); must not overlap y
 *   rope_cols  0 <= rope_cols <= n_out, multiple of 128
 * Strides are in elements, multiples of 8 (x, w >= k; y >= n_out); pointers
 * 16-byte aligned.  Arithmetic: float32 accumulation of exact bf16 products.
 * m == 0 is a no-op.  Errors: EINVAL, ERANGE (m >= 2^31, 256 rows of x, w or y
 * spanning 2^31 bytes, x spanning 2^32 bytes, 2^30 or more 256 x 256 tiles),
 * EUNSUPPORTED, EHIP.
 */
#define H3ATTN_LINEAR_TILE 256
#define H3ATTN_LINEAR_KSTEP 64
int h3attn_linear(const void* x, int64_t x_stride, const void* w, int64_t w_stride, const void* bias,
                  void* y, int64_t y_stride, int64_t m, int32_t n_out, int32_t k,
                  const float* rope_table_dev, int32_t rope_cols, void* stream);

/*
 * Device call.  The rotation table of a packed sequence: table[i][p] = (cos phi,
 * sin phi) of pair p of row i, phi = pos_a(i) * theta_a^(-2 p' / d_a) as in
 * h3attn_rope_qk (same arithmetic, same float32 values), for all 64 pairs of a
 * 128-wide head.  Every head of Q and K, every block and every sampler step
 * shares it, so a sequence builds it once (512 B per row, 14.4 MB at 28,192
 * rows) and h3attn_linear reads it instead of recomputing it per head.
 *   cfg, coords_dev   as for h3attn_rope_qk
 *   table_dev         out: device float32 [n_tokens][64][2], 16-byte aligned, not
 *                     overlapping the coordinates
 * n_tokens == 0 is a no-op.  Errors: EINVAL, ERANGE (n_tokens * 64 >= 2^31),
 * EUNSUPPORTED, EHIP.
 */
int h3attn_rope_table(const h3attn_rope_cfg* cfg, const float* coords_dev, int64_t n_tokens, float* table_dev,
                      void* stream);

/*
 * ---- Latent <-> token packing with the sampler's Euler step ----
 *
 * Sources: "MiniMax H3 - one transformer that denoises video and audio
 * together": patchify paragraph (every non-overlapping 1 x 2 x 2 block of the
 * video latent becomes one token of 24 x 2 x 2 = 96 values), latent-frame
 * paragraph (44 x 80 sheet -> 22 x 40 = 880 tokens; one audio latent frame = one
 * 32-value token per stereo channel), flow-matching paragraphs (x_t = t x0 +
 * (1 - t) noise; a non-learned scheduler steps along the predicted velocity);
 * "Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio",
 * section 2 (only target rows are updated).
 *
 * Readings where the pages are silent: the sampler state is float32, tokens
 * bf16 (nearest even); one step is x <- x + dt * v with dt = t_next - t; the
 * video latent is [C][T][H][W] and its token rows run (t, patch row, patch
 * column) with values (c, iy, ix) at (c * 2 + iy) * 2 + ix; the audio latent is
 * [n_ch][steps][width] and token row s * n_ch + ch holds latent[ch][s][:].
 *
 * Both calls: latent is device float32 (8-byte aligned), updated in place when
 * v_tokens is not NULL (latent += dt * unpack(v_tokens)); tokens, when not NULL,
 * receive the packed (updated) latent as bf16.  At least one of v_tokens and
 * tokens must be given.  Token buffers are row-major with a stride in elements
 * (even, >= the token width), 4-byte aligned, and overlap neither each other
 * nor the latent.  Zero frames / steps is a no-op.  Errors: EINVAL, ERANGE (more
 * than 2^31 - 1 latent values; video rows wider than LDS allows:
 * channels * lat_w > 8192), EUNSUPPORTED, EHIP.
 */

/* Video: latent [channels][frames][lat_h][lat_w] (lat_h, lat_w even); tokens
 * [frames * lat_h/2 * lat_w/2][4 * channels]. */
int h3attn_video_euler_pack(float* latent, int32_t channels, int32_t frames, int32_t lat_h, int32_t lat_w,
                            const void* v_tokens, int64_t v_stride, float dt, void* tokens,
                            int64_t tokens_stride, void* stream);

/* Audio: latent [n_ch][steps][width] (width even); tokens [steps * n_ch][width]. */
int h3attn_audio_euler_pack(float* latent, int32_t n_ch, int32_t steps, int32_t width,
                            const void* v_tokens, int64_t v_stride, float dt, void* tokens,
                            int64_t tokens_stride, void* stream);

/* Both target latents of one sampler step, video and audio, in one launch: the
 * same result as h3attn_video_euler_pack followed by h3attn_audio_euler_pack
 * with the same dt, each argument group checked as there.  A part with zero
 * frames / steps is skipped.  No buffer that one part writes (its latent when
 * it has velocities, its tokens) may share a byte with a buffer of the other
 * part (EINVAL). */
int h3attn_av_euler_pack(float* video_latent, int32_t channels, int32_t frames, int32_t lat_h, int32_t lat_w,
                         const void* video_v, int64_t video_v_stride, void* video_tokens,
                         int64_t video_tokens_stride, float* audio_latent, int32_t n_ch, int32_t steps,
                         int32_t width, const void* audio_v, int64_t audio_v_stride, void* audio_tokens,
                         int64_t audio_tokens_stride, float dt, void* stream);

/*
 * Device call.  h3attn_forward with a caller-owned scratch workspace (device
 * memory, 16-byte aligned, not overlapping any tensor argument).  The attention
 * runs one workgroup per (head, 256-row query block) on each compute unit in
 * waves; the units of the last, partly filled wave may be split along the keys
 * over several workgroups that leave float32 partial results (unnormalised O
 * and the row's max / sum) in the workspace, merged by a second kernel with the
 * same max-and-rescale rule.  A cost model of that last stretch (the waves of
 * parts it takes, plus the merge's traffic) picks the number of parts, 2 to 8,
 * and splits only when that saves at least a tenth of a unit's time.  The
 * result equals h3attn_forward up to the rounding order of the split rows.  A
 * NULL or too small workspace runs the unsplit schedule (h3attn_forward); the
 * library still allocates nothing.  The workspace must not be shared by calls
 * in flight at once.
 */
int h3attn_forward_ws(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                      const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                      int64_t row_stride_o, float scale, void* workspace, int64_t workspace_bytes,
                      void* stream);

/*
 * Host call.  Workspace bytes h3attn_forward_ws uses for this shape on the
 * current device (0 when no split pays off, or no gfx950 device is current).
 */
int64_t h3attn_forward_workspace_bytes(int64_t n_tokens, int32_t n_heads);

/*
 * Device call for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, checks and result are those of h3attn_forward_ws given the full
 * workspace it asks for (the same schedule and kernels, hence the same bits),
 * but the key-split partials go to a static device array of
 * H3ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends; the call allocates nothing.  A shape whose
 * partials need more (h3attn_forward_workspace_bytes above the limit; the five
 * 42-head workloads need at most 64.0 MiB) returns H3ATTN_ESCRATCH before
 * anything runs.  Every call on one device shares that device's array and
 * leaves its partials there; nothing in it needs clearing between calls, but
 * calls in flight at the same time on one device (several streams or host
 * threads) race on it and must be serialised by the caller.
 */
#define H3ATTN_NOALLOC_SCRATCH_BYTES (64LL << 20)
int h3attn_forward_noalloc(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                           int64_t row_stride_o, float scale, void* stream);

/* Static description of an error code (never NULL). */
const char* h3attn_strerror(int code);

/* Library version string, e.g. "h3attn 0.2.0 gfx950". */
const char* h3attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
