// Host-side coordinate builder of the packed sequence: segment table -> (t, h, w)
// per row.  Plain C++ (no HIP); compiled with -ffp-contract=off so that the
// binary64 spatial formula is evaluated as separate IEEE operations.
//
// Rules ("Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio",
// section 4; "MiniMax H3 - one transformer that denoises video and audio
// together", paragraphs on the clock unit, text positions and the spatial grid):
//  - the clock unit is one 40 Hz audio latent; a 24 fps frame is 5/3 units, so a
//    latent frame (4 source frames) advances 20/3 units; times are carried as
//    integers in thirds and rounded once to binary32;
//  - left / right audio share t and differ on w; text is 1-D (h = w = 0);
//  - the video patch grid is normalised by sqrt(rows * cols), centred on the
//    [0, 32) canvas, aspect ratio kept.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "h3attn.h"

namespace {

constexpr int64_t kMaxThirds = int64_t(1) << 24;   // |t3| below this is exact in binary32
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

// t3 / 3 rounded to nearest-even binary32.  Both operands are exact binary32
// values (|t3| < 2^24), so one IEEE division is the correctly rounded quotient.
inline float thirds_to_f32(int64_t t3) {
  volatile float num = static_cast<float>(t3);
  volatile float den = 3.0f;
  return num / den;
}

int segment_rows(const h3attn_segment& s, int64_t* rows) {
  if (s.frames < 0 || s.grid_h < 1 || s.grid_w < 1) return H3ATTN_EINVAL;
  switch (s.kind) {
    case H3_SEG_TEXT:
      if (s.grid_h != 1 || s.grid_w != 1) return H3ATTN_EINVAL;
      break;
    case H3_SEG_AUDIO:
      if (s.grid_h != 1) return H3ATTN_EINVAL;
      break;
    case H3_SEG_VIDEO:
      break;
    default:
      return H3ATTN_EINVAL;
  }
  *rows = int64_t(s.frames) * s.grid_h * s.grid_w;
  if (s.frames > 0) {
    int64_t first = s.t0_thirds;
    int64_t last = int64_t(s.t0_thirds) + int64_t(s.frames - 1) * s.dt_thirds;
    if (first <= -kMaxThirds || first >= kMaxThirds || last <= -kMaxThirds || last >= kMaxThirds)
      return H3ATTN_ERANGE;
  }
  return H3ATTN_OK;
}

}  // namespace

extern "C" int h3attn_build_coords(const h3attn_segment* segs, int32_t n_segs, float* coords,
                                   int64_t capacity_rows, int64_t* n_tokens) {
  if (n_tokens == nullptr || n_segs < 0 || (n_segs > 0 && segs == nullptr) || capacity_rows < 0)
    return H3ATTN_EINVAL;
  int64_t total = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    int64_t rows = 0;
    int rc = segment_rows(segs[i], &rows);
    if (rc != H3ATTN_OK) return rc;
    total += rows;
    if (total > kMaxRows) return H3ATTN_ERANGE;
  }
  *n_tokens = total;
  if (coords == nullptr) return H3ATTN_OK;
  if (capacity_rows < total) return H3ATTN_ERANGE;

  float* out = coords;
  for (int32_t i = 0; i < n_segs; ++i) {
    const h3attn_segment& s = segs[i];
    if (s.frames == 0) continue;
    if (s.kind == H3_SEG_TEXT) {
      for (int32_t f = 0; f < s.frames; ++f) {
        out[0] = thirds_to_f32(int64_t(s.t0_thirds) + int64_t(f) * s.dt_thirds);
        out[1] = 0.0f;
        out[2] = 0.0f;
        out += 3;
      }
    } else if (s.kind == H3_SEG_AUDIO) {
      for (int32_t f = 0; f < s.frames; ++f) {
        const float t = thirds_to_f32(int64_t(s.t0_thirds) + int64_t(f) * s.dt_thirds);
        for (int32_t ch = 0; ch < s.grid_w; ++ch) {
          out[0] = t;
          out[1] = 0.0f;
          out[2] = static_cast<float>(ch);
          out += 3;
        }
      }
    } else {  // H3_SEG_VIDEO
      const int32_t gh = s.grid_h, gw = s.grid_w;
      const double step = 16.0 / std::sqrt(static_cast<double>(int64_t(gh) * gw));
      for (int32_t f = 0; f < s.frames; ++f) {
        const float t = thirds_to_f32(int64_t(s.t0_thirds) + int64_t(f) * s.dt_thirds);
        for (int32_t r = 0; r < gh; ++r) {
          const double hr = 16.0 + static_cast<double>(2 * int64_t(r) + 1 - gh) * step;
          const float h = static_cast<float>(hr);
          for (int32_t c = 0; c < gw; ++c) {
            const double wc = 16.0 + static_cast<double>(2 * int64_t(c) + 1 - gw) * step;
            out[0] = t;
            out[1] = h;
            out[2] = static_cast<float>(wc);
            out += 3;
          }
        }
      }
    }
  }
  return H3ATTN_OK;
}
