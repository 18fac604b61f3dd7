// C ABI of the library: argument validation, device check and dispatch to the
// kernel launchers.  Every check runs before any launch, so an error leaves
// all outputs untouched.
#include <atomic>
#include <cmath>
#include <cstring>

#include "h3attn.h"
#include "launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_device_kind[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return H3ATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return H3ATTN_EUNSUPPORTED;
  int kind = g_device_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return H3ATTN_EHIP;
    kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? H3ATTN_OK : H3ATTN_EUNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int make_table(const h3attn_rope_cfg* cfg, h3::RopeTable* tab) {
  if (cfg == nullptr || cfg->head_dim != h3::kHeadDim) return H3ATTN_EINVAL;
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (cfg->sec[a] < 0 || (cfg->sec[a] & 1)) return H3ATTN_EINVAL;
    if (!(cfg->theta[a] > 0.0) || !std::isfinite(cfg->theta[a])) return H3ATTN_EINVAL;
    sum += cfg->sec[a];
  }
  if (sum != h3::kHeadDim) return H3ATTN_EINVAL;
  int pair = 0;
  for (int a = 0; a < 3; ++a) {
    const int d = cfg->sec[a];
    for (int p = 0; p < d / 2; ++p)
      tab->freq[pair++] = std::pow(cfg->theta[a], -(2.0 * p) / static_cast<double>(d));
  }
  tab->b1 = cfg->sec[0] / 2;
  tab->b2 = (cfg->sec[0] + cfg->sec[1]) / 2;
  return H3ATTN_OK;
}

int check_tensor_geometry(int64_t n_tokens, int32_t n_heads, int64_t stride) {
  if (n_tokens < 0 || n_heads <= 0) return H3ATTN_EINVAL;
  if (stride < int64_t(n_heads) * h3::kHeadDim || (stride & 7) != 0) return H3ATTN_EINVAL;
  // element offsets are 32-bit inside the kernels
  if (n_tokens > 0 && n_tokens * stride >= (int64_t(1) << 31)) return H3ATTN_ERANGE;
  return H3ATTN_OK;
}

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + uintptr_t(b_bytes) && b0 < a0 + uintptr_t(a_bytes);
}

// Whether two row views with the same row pitch share a byte: rows r of view x cover
// [x + r * pitch, x + r * pitch + width) for r < rows, with width <= pitch.  Rows r1 of a and
// r2 of b meet iff |d - j * pitch| < width for d = b - a and j = r1 - r2 in (-rows, rows); only
// the two j next to d / pitch can come that close.  Views of one fused buffer that interleave
// rows without sharing bytes (Q and K slots of a [N][3][H][D] projection output) do not overlap.
bool views_overlap(const void* a, const void* b, int64_t rows, int64_t pitch, int64_t width) {
  const int64_t d = static_cast<int64_t>(reinterpret_cast<uintptr_t>(b) - reinterpret_cast<uintptr_t>(a));
  int64_t j = d / pitch;
  if (d < 0 && j * pitch != d) --j;   // floor
  for (int64_t jj = j; jj <= j + 1; ++jj) {
    if (jj <= -rows || jj >= rows) continue;
    const int64_t gap = d - jj * pitch;
    if (gap > -width && gap < width) return true;
  }
  return false;
}

}  // namespace

extern "C" int h3attn_rope_qk(const h3attn_rope_cfg* cfg, const float* coords_dev,
                              const void* q_in, void* q_out, const void* k_in, void* k_out,
                              int64_t n_tokens, int32_t n_heads, int64_t row_stride,
                              void* stream) {
  h3::RopeArgs a;
  int rc = make_table(cfg, &a.tab);
  if (rc != H3ATTN_OK) return rc;
  if ((q_in == nullptr) != (q_out == nullptr) || (k_in == nullptr) != (k_out == nullptr))
    return H3ATTN_EINVAL;
  if (q_in == nullptr && k_in == nullptr) return H3ATTN_EINVAL;
  for (const void* p : {q_in, static_cast<const void*>(q_out), k_in, static_cast<const void*>(k_out)})
    if (p != nullptr && !aligned16(p)) return H3ATTN_EINVAL;
  rc = check_tensor_geometry(n_tokens, n_heads, row_stride);
  if (rc != H3ATTN_OK) return rc;
  if (n_tokens == 0) return H3ATTN_OK;
  if (coords_dev == nullptr) return H3ATTN_EINVAL;
  // an output may be its own input exactly (in place); it shares no byte with any other tensor
  {
    const int64_t pitch = row_stride * 2, width = int64_t(n_heads) * h3::kHeadDim * 2;
    const int64_t span = (n_tokens - 1) * pitch + width;
    const void* ins[2] = {q_in, k_in};
    const void* outs[2] = {q_out, k_out};
    for (int o = 0; o < 2; ++o) {
      if (outs[o] == nullptr) continue;
      if (overlaps(outs[o], span, coords_dev, n_tokens * 12)) return H3ATTN_EINVAL;
      for (int i = 0; i < 2; ++i)
        if (ins[i] != nullptr && !(i == o && ins[i] == outs[o]) &&
            views_overlap(ins[i], outs[o], n_tokens, pitch, width))
          return H3ATTN_EINVAL;
      if (o == 1 && outs[0] != nullptr && views_overlap(outs[0], outs[1], n_tokens, pitch, width))
        return H3ATTN_EINVAL;
    }
  }
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  a.coords = coords_dev;
  a.q_in = static_cast<const uint16_t*>(q_in);
  a.q_out = static_cast<uint16_t*>(q_out);
  a.k_in = static_cast<const uint16_t*>(k_in);
  a.k_out = static_cast<uint16_t*>(k_out);
  a.n = static_cast<int32_t>(n_tokens);
  a.heads = n_heads;
  a.stride = static_cast<int32_t>(row_stride);
  return h3::launch_rope_qk(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK
                                                                               : H3ATTN_EHIP;
}

namespace {

std::atomic<int> g_device_cus[kMaxDevices];

// compute units of the current device (cached), or 0 when it cannot be read
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = g_device_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_device_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int forward_impl(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q, const void* q, const void* k,
                 const void* v, void* o, float* lse, int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                 int64_t row_stride_o, float scale, void* workspace, int64_t workspace_bytes, bool noalloc, void* stream);

// Scratch of h3attn_forward_noalloc: the key-split partials live in this file-scope device array
// instead of a caller workspace.  Each device holds its own copy for the life of the process.  In
// host code the name is only a stand-in for the symbol: kernels receive the device address that
// hipGetSymbolAddress returns, resolved once per device with that device current.
static __device__ __align__(256) unsigned char scratch[H3ATTN_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// device address of the current device's scratch array, or nullptr when it cannot be resolved
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int64_t h3attn_forward_workspace_bytes(int64_t n_tokens, int32_t n_heads) {
  if (n_tokens <= 0 || n_heads <= 0 || n_tokens >= (int64_t(1) << 31)) return 0;
  if (check_device() != H3ATTN_OK) return 0;
  int32_t n_full, split, tps;
  int64_t bytes;
  h3::attn_fwd_schedule(static_cast<int32_t>(n_tokens), n_heads, device_cus(), &n_full, &split, &tps, &bytes);
  return bytes;
}

extern "C" int h3attn_forward(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                              int64_t row_stride_o, float scale, void* stream) {
  return forward_impl(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
                      scale, nullptr, 0, false, stream);
}

extern "C" int h3attn_forward_ws(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                                 const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                                 int64_t row_stride_o, float scale, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  if (workspace_bytes < 0 || (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0))
    return H3ATTN_EINVAL;
  return forward_impl(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
                      scale, workspace, workspace_bytes, false, stream);
}

extern "C" int h3attn_forward_noalloc(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q,
                                      const void* q, const void* k, const void* v, void* o, float* lse,
                                      int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                                      int64_t row_stride_o, float scale, void* stream) {
  return forward_impl(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
                      scale, nullptr, 0, true, stream);
}

namespace {

int forward_impl(const h3attn_rope_cfg* cfg, const float* coords_dev, int32_t rope_q, const void* q, const void* k,
                 const void* v, void* o, float* lse, int64_t n_tokens, int32_t n_heads, int64_t row_stride_qkv,
                 int64_t row_stride_o, float scale, void* workspace, int64_t workspace_bytes, bool noalloc, void* stream) {
  h3::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  int rc = make_table(cfg, &a.tab);
  if (rc != H3ATTN_OK) return rc;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return H3ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return H3ATTN_EINVAL;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return H3ATTN_EINVAL;
  if (!std::isfinite(scale)) return H3ATTN_EINVAL;
  rc = check_tensor_geometry(n_tokens, n_heads, row_stride_qkv);
  if (rc != H3ATTN_OK) return rc;
  rc = check_tensor_geometry(n_tokens, n_heads, row_stride_o);
  if (rc != H3ATTN_OK) return rc;
  if (n_tokens > 0 && int64_t(n_heads) * n_tokens >= (int64_t(1) << 31)) return H3ATTN_ERANGE;
  if (n_tokens == 0) return H3ATTN_OK;
  if (rope_q && coords_dev == nullptr) return H3ATTN_EINVAL;
  const int64_t in_bytes = ((n_tokens - 1) * row_stride_qkv + int64_t(n_heads) * h3::kHeadDim) * 2;
  const int64_t out_bytes = ((n_tokens - 1) * row_stride_o + int64_t(n_heads) * h3::kHeadDim) * 2;
  if (overlaps(o, out_bytes, q, in_bytes) || overlaps(o, out_bytes, k, in_bytes) ||
      overlaps(o, out_bytes, v, in_bytes))
    return H3ATTN_EINVAL;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  if (scale <= 0.0f) scale = 1.0f / std::sqrt(static_cast<float>(h3::kHeadDim));
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.coords = coords_dev;
  a.n = static_cast<int32_t>(n_tokens);
  a.heads = n_heads;
  a.stride_qkv = static_cast<int32_t>(row_stride_qkv);
  a.stride_o = static_cast<int32_t>(row_stride_o);
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rope_q = rope_q ? 1 : 0;
  if (noalloc) {
    // the schedule of h3attn_forward_ws with a full workspace; shapes whose partials exceed the
    // static scratch are refused before anything runs
    int32_t nf, sp, tps;
    int64_t need = 0;
    h3::attn_fwd_schedule(a.n, a.heads, device_cus(), &nf, &sp, &tps, &need);
    if (need > H3ATTN_NOALLOC_SCRATCH_BYTES) return H3ATTN_ESCRATCH;
    if (need > 0) {
      workspace = device_scratch();
      if (workspace == nullptr) return H3ATTN_EHIP;
      workspace_bytes = H3ATTN_NOALLOC_SCRATCH_BYTES;
    }
  }
  // the key-split tail runs only with a workspace that holds its partials, disjoint from the tensors
  int64_t ws_need = 0;
  h3::attn_fwd_schedule(a.n, a.heads, workspace != nullptr ? device_cus() : 0, &a.n_full, &a.split,
                        &a.tiles_per_split, &ws_need);
  if (ws_need > 0 && (workspace_bytes < ws_need || overlaps(workspace, ws_need, o, out_bytes) ||
                      overlaps(workspace, ws_need, q, in_bytes) || overlaps(workspace, ws_need, k, in_bytes) ||
                      overlaps(workspace, ws_need, v, in_bytes) ||
                      (lse != nullptr && overlaps(workspace, ws_need, lse, int64_t(n_heads) * n_tokens * 4)))) {
    if (workspace_bytes < ws_need) {
      h3::attn_fwd_schedule(a.n, a.heads, 0, &a.n_full, &a.split, &a.tiles_per_split, &ws_need);
    } else {
      return H3ATTN_EINVAL;
    }
  }
  if (ws_need > 0) a.ws_o = static_cast<float*>(workspace);   // the launcher lays out the partials
  return h3::launch_attn_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK
                                                                                : H3ATTN_EHIP;
}

}  // namespace

namespace {

// Shared checks of the two AdaLN entry points; fills everything but y / gate / x_out.
int adaln_common(const void* x, int64_t x_stride, const int32_t* t_idx, const int32_t* tags,
                 const void* shift, const void* scale, int64_t entry_stride, int32_t n_entries, void* h,
                 int64_t h_stride, int64_t n_rows, int32_t hidden, int32_t norm_kind, float eps,
                 h3::AdalnArgs* a) {
  if (n_rows < 0 || n_rows >= (int64_t(1) << 31)) return n_rows < 0 ? H3ATTN_EINVAL : H3ATTN_ERANGE;
  if (hidden < 8 || hidden > H3ATTN_ADALN_MAX_HIDDEN || (hidden & 7) != 0) return H3ATTN_EINVAL;
  if (norm_kind != H3ATTN_LAYER_NORM && norm_kind != H3ATTN_RMS_NORM) return H3ATTN_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3ATTN_EINVAL;
  if (n_entries <= 0 || entry_stride < 0 || (entry_stride & 7) != 0) return H3ATTN_EINVAL;
  if (x_stride < hidden || (x_stride & 7) != 0 || h_stride < hidden || (h_stride & 7) != 0) return H3ATTN_EINVAL;
  if (x == nullptr || h == nullptr || t_idx == nullptr || tags == nullptr || shift == nullptr || scale == nullptr)
    return H3ATTN_EINVAL;
  for (const void* p : {x, static_cast<const void*>(h), shift, scale})
    if (!aligned16(p)) return H3ATTN_EINVAL;
  if ((reinterpret_cast<uintptr_t>(t_idx) & 3u) != 0 || (reinterpret_cast<uintptr_t>(tags) & 3u) != 0)
    return H3ATTN_EINVAL;
  a->x = static_cast<const uint16_t*>(x);
  a->t_idx = t_idx;
  a->tags = tags;
  a->shift = static_cast<const uint16_t*>(shift);
  a->scale = static_cast<const uint16_t*>(scale);
  a->h = static_cast<uint16_t*>(h);
  a->x_stride = x_stride;
  a->h_stride = h_stride;
  a->entry_stride = entry_stride;
  a->n_entries = n_entries;
  a->n_rows = n_rows;
  a->hidden = hidden;
  a->norm_kind = norm_kind;
  a->eps = eps;
  return H3ATTN_OK;
}

int64_t span_bytes(int64_t rows, int64_t stride, int64_t width) { return ((rows - 1) * stride + width) * 2; }

}  // namespace

extern "C" int h3attn_adaln_modulate(const void* x, int64_t x_stride, const int32_t* t_idx, const int32_t* tags,
                                     const void* shift, const void* scale, int64_t entry_stride,
                                     int32_t n_entries, void* h, int64_t h_stride, int64_t n_rows,
                                     int32_t hidden, int32_t norm_kind, float eps, void* stream) {
  h3::AdalnArgs a;
  std::memset(&a, 0, sizeof(a));
  int rc = adaln_common(x, x_stride, t_idx, tags, shift, scale, entry_stride, n_entries, h, h_stride, n_rows,
                        hidden, norm_kind, eps, &a);
  if (rc != H3ATTN_OK) return rc;
  if (n_rows == 0) return H3ATTN_OK;
  // h may be x itself (each row is read whole before it is written), nothing else
  const int64_t hb = span_bytes(n_rows, h_stride, hidden), xb = span_bytes(n_rows, x_stride, hidden);
  if (h != x && overlaps(h, hb, x, xb)) return H3ATTN_EINVAL;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  return h3::launch_adaln(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

extern "C" int h3attn_adaln_residual(const void* x, const void* y, int64_t xy_stride, const int32_t* t_idx,
                                     const int32_t* tags, const void* gate, const void* shift, const void* scale,
                                     int64_t entry_stride, int32_t n_entries, void* x_out, void* h,
                                     int64_t out_stride, int64_t n_rows, int32_t hidden, int32_t norm_kind,
                                     float eps, void* stream) {
  h3::AdalnArgs a;
  std::memset(&a, 0, sizeof(a));
  int rc = adaln_common(x, xy_stride, t_idx, tags, shift, scale, entry_stride, n_entries, h, out_stride, n_rows,
                        hidden, norm_kind, eps, &a);
  if (rc != H3ATTN_OK) return rc;
  if (y == nullptr || gate == nullptr || x_out == nullptr) return H3ATTN_EINVAL;
  if (!aligned16(y) || !aligned16(gate) || !aligned16(x_out)) return H3ATTN_EINVAL;
  if (n_rows == 0) return H3ATTN_OK;
  // x_out may be x itself; h overlaps nothing; x_out overlaps neither y nor h
  const int64_t ib = span_bytes(n_rows, xy_stride, hidden), ob = span_bytes(n_rows, out_stride, hidden);
  if (overlaps(h, ob, x, ib) || overlaps(h, ob, y, ib) || overlaps(h, ob, x_out, ob)) return H3ATTN_EINVAL;
  if (overlaps(x_out, ob, y, ib)) return H3ATTN_EINVAL;
  if (x_out != x && overlaps(x_out, ob, x, ib)) return H3ATTN_EINVAL;
  if (x_out == x && out_stride != xy_stride) return H3ATTN_EINVAL;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  a.y = static_cast<const uint16_t*>(y);
  a.y_stride = xy_stride;
  a.gate = static_cast<const uint16_t*>(gate);
  a.x_out = static_cast<uint16_t*>(x_out);
  a.out_stride = out_stride;
  return h3::launch_adaln(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

namespace {

// Shared argument checks of the packing calls (sizes already checked by the caller); the device
// check comes after every argument check.
int pack_common(float* latent, int64_t elems, const void* v, int64_t v_stride, void* tokens, int64_t tok_stride,
                int64_t rows, int64_t width, float dt) {
  if (latent == nullptr || (reinterpret_cast<uintptr_t>(latent) & 7u) != 0) return H3ATTN_EINVAL;
  if (v == nullptr && tokens == nullptr) return H3ATTN_EINVAL;
  if (!std::isfinite(dt)) return H3ATTN_EINVAL;
  if (elems >= (int64_t(1) << 31)) return H3ATTN_ERANGE;
  if (v != nullptr && ((reinterpret_cast<uintptr_t>(v) & 3u) != 0 || v_stride < width || (v_stride & 1) != 0))
    return H3ATTN_EINVAL;
  if (tokens != nullptr &&
      ((reinterpret_cast<uintptr_t>(tokens) & 3u) != 0 || tok_stride < width || (tok_stride & 1) != 0))
    return H3ATTN_EINVAL;
  if (rows == 0) return H3ATTN_OK;
  const int64_t lat_bytes = elems * 4;
  if (v != nullptr && overlaps(v, span_bytes(rows, v_stride, width), latent, lat_bytes)) return H3ATTN_EINVAL;
  if (tokens != nullptr) {
    const int64_t tb = span_bytes(rows, tok_stride, width);
    if (overlaps(tokens, tb, latent, lat_bytes)) return H3ATTN_EINVAL;
    if (v != nullptr && overlaps(tokens, tb, v, span_bytes(rows, v_stride, width))) return H3ATTN_EINVAL;
  }
  return H3ATTN_OK;
}

}  // namespace

namespace h3 {
// one launch for a video and an audio latent (either may be null); pack_kernel.hip
hipError_t launch_av_pack(const PackArgs* video, const PackArgs* audio, hipStream_t stream);
}  // namespace h3

namespace {

// Checks of the video packing call; fills a and the byte spans of its buffers.  *rows_out = 0: nothing to do.
int video_pack_args(float* latent, int32_t channels, int32_t frames, int32_t lat_h, int32_t lat_w,
                    const void* v_tokens, int64_t v_stride, float dt, void* tokens, int64_t tokens_stride,
                    h3::PackArgs* a, int64_t* rows_out) {
  *rows_out = 0;
  if (channels < 1 || frames < 0 || lat_h < 2 || lat_w < 2 || (lat_h & 1) != 0 || (lat_w & 1) != 0)
    return H3ATTN_EINVAL;
  if (int64_t(channels) * 2 * lat_w * 4 > 65536) return H3ATTN_ERANGE;   // two latent rows of every channel in LDS
  const int64_t elems = int64_t(channels) * frames * lat_h * lat_w;
  const int64_t rows = int64_t(frames) * (lat_h / 2) * (lat_w / 2);
  int rc = pack_common(latent, elems, v_tokens, v_stride, tokens, tokens_stride, rows, 4 * int64_t(channels), dt);
  if (rc != H3ATTN_OK || rows == 0) return rc;
  std::memset(a, 0, sizeof(*a));
  a->latent = latent;
  a->v = static_cast<const uint16_t*>(v_tokens);
  a->tokens = static_cast<uint16_t*>(tokens);
  a->v_stride = v_stride;
  a->tok_stride = tokens_stride;
  a->c = channels;
  a->t = frames;
  a->h = lat_h;
  a->w = lat_w;
  a->dt = dt;
  *rows_out = rows;
  return H3ATTN_OK;
}

// Checks of the audio packing call; fills a.  *rows_out = 0: nothing to do.
int audio_pack_args(float* latent, int32_t n_ch, int32_t steps, int32_t width, const void* v_tokens,
                    int64_t v_stride, float dt, void* tokens, int64_t tokens_stride, h3::PackArgs* a,
                    int64_t* rows_out) {
  *rows_out = 0;
  if (n_ch < 1 || steps < 0 || width < 2 || (width & 1) != 0) return H3ATTN_EINVAL;
  const int64_t elems = int64_t(n_ch) * steps * width;
  const int64_t rows = int64_t(n_ch) * steps;
  int rc = pack_common(latent, elems, v_tokens, v_stride, tokens, tokens_stride, rows, width, dt);
  if (rc != H3ATTN_OK || rows == 0) return rc;
  std::memset(a, 0, sizeof(*a));
  a->latent = latent;
  a->v = static_cast<const uint16_t*>(v_tokens);
  a->tokens = static_cast<uint16_t*>(tokens);
  a->v_stride = v_stride;
  a->tok_stride = tokens_stride;
  a->c = n_ch;
  a->t = steps;
  a->h = 1;
  a->w = width;
  a->dt = dt;
  *rows_out = rows;
  return H3ATTN_OK;
}

// byte spans of a packing call's latent, velocity and token buffers (0 where absent)
void pack_spans(const h3::PackArgs& a, int64_t rows, int64_t width, int64_t elems, int64_t* lat, int64_t* v,
                int64_t* tok) {
  *lat = elems * 4;
  *v = a.v != nullptr ? span_bytes(rows, a.v_stride, width) : 0;
  *tok = a.tokens != nullptr ? span_bytes(rows, a.tok_stride, width) : 0;
}

}  // namespace

extern "C" int h3attn_video_euler_pack(float* latent, int32_t channels, int32_t frames, int32_t lat_h, int32_t lat_w,
                                       const void* v_tokens, int64_t v_stride, float dt, void* tokens,
                                       int64_t tokens_stride, void* stream) {
  h3::PackArgs a;
  int64_t rows = 0;
  int rc = video_pack_args(latent, channels, frames, lat_h, lat_w, v_tokens, v_stride, dt, tokens, tokens_stride, &a,
                           &rows);
  if (rc != H3ATTN_OK || rows == 0) return rc;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  return h3::launch_video_pack(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

extern "C" int h3attn_audio_euler_pack(float* latent, int32_t n_ch, int32_t steps, int32_t width,
                                       const void* v_tokens, int64_t v_stride, float dt, void* tokens,
                                       int64_t tokens_stride, void* stream) {
  h3::PackArgs a;
  int64_t rows = 0;
  int rc = audio_pack_args(latent, n_ch, steps, width, v_tokens, v_stride, dt, tokens, tokens_stride, &a, &rows);
  if (rc != H3ATTN_OK || rows == 0) return rc;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  return h3::launch_audio_pack(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

extern "C" int h3attn_av_euler_pack(float* video_latent, int32_t channels, int32_t frames, int32_t lat_h,
                                    int32_t lat_w, const void* video_v, int64_t video_v_stride, void* video_tokens,
                                    int64_t video_tokens_stride, float* audio_latent, int32_t n_ch, int32_t steps,
                                    int32_t width, const void* audio_v, int64_t audio_v_stride, void* audio_tokens,
                                    int64_t audio_tokens_stride, float dt, void* stream) {
  h3::PackArgs va, aa;
  int64_t vrows = 0, arows = 0;
  int rc = video_pack_args(video_latent, channels, frames, lat_h, lat_w, video_v, video_v_stride, dt, video_tokens,
                           video_tokens_stride, &va, &vrows);
  if (rc != H3ATTN_OK) return rc;
  rc = audio_pack_args(audio_latent, n_ch, steps, width, audio_v, audio_v_stride, dt, audio_tokens,
                       audio_tokens_stride, &aa, &arows);
  if (rc != H3ATTN_OK) return rc;
  if (vrows == 0 && arows == 0) return H3ATTN_OK;
  if (vrows > 0 && arows > 0) {
    // the buffers one part writes (latent, tokens) share no byte with any buffer of the other part
    int64_t vl, vv, vt, al, av, at;
    pack_spans(va, vrows, 4 * int64_t(channels), int64_t(channels) * frames * lat_h * lat_w, &vl, &vv, &vt);
    pack_spans(aa, arows, width, int64_t(n_ch) * steps * width, &al, &av, &at);
    const void* vb[3] = {va.latent, va.v, va.tokens};
    const int64_t vn[3] = {vl, vv, vt};
    const void* ab[3] = {aa.latent, aa.v, aa.tokens};
    const int64_t an[3] = {al, av, at};
    const bool v_written[3] = {va.v != nullptr, false, true};   // the latent is written only with velocities
    const bool a_written[3] = {aa.v != nullptr, false, true};
    for (int i = 0; i < 3; ++i)
      for (int j = 0; j < 3; ++j)
        if (vb[i] != nullptr && ab[j] != nullptr && (v_written[i] || a_written[j]) &&
            overlaps(vb[i], vn[i], ab[j], an[j]))
          return H3ATTN_EINVAL;
  }
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  return h3::launch_av_pack(vrows > 0 ? &va : nullptr, arows > 0 ? &aa : nullptr, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? H3ATTN_OK
             : H3ATTN_EHIP;
}

extern "C" int h3attn_rope_table(const h3attn_rope_cfg* cfg, const float* coords_dev, int64_t n_tokens,
                                 float* table_dev, void* stream) {
  h3::RopeTabArgs a;
  std::memset(&a, 0, sizeof(a));
  int rc = make_table(cfg, &a.tab);
  if (rc != H3ATTN_OK) return rc;
  if (n_tokens < 0) return H3ATTN_EINVAL;
  if (n_tokens >= (int64_t(1) << 31) / h3::kPairs) return H3ATTN_ERANGE;
  if (n_tokens == 0) return H3ATTN_OK;
  if (coords_dev == nullptr || table_dev == nullptr || !aligned16(table_dev) ||
      (reinterpret_cast<uintptr_t>(coords_dev) & 3u) != 0)
    return H3ATTN_EINVAL;
  if (overlaps(table_dev, n_tokens * h3::kPairs * 8, coords_dev, n_tokens * 12)) return H3ATTN_EINVAL;
  rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  a.coords = coords_dev;
  a.out = table_dev;
  a.n = static_cast<int32_t>(n_tokens);
  return h3::launch_rope_table(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

extern "C" int h3attn_linear(const void* x, int64_t x_stride, const void* w, int64_t w_stride, const void* bias,
                             void* y, int64_t y_stride, int64_t m, int32_t n_out, int32_t k,
                             const float* rope_table_dev, int32_t rope_cols, void* stream) {
  h3::GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  if (x == nullptr || w == nullptr || y == nullptr) return H3ATTN_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias != nullptr && !aligned16(bias))) return H3ATTN_EINVAL;
  if (m < 0 || n_out <= 0 || (n_out % H3ATTN_LINEAR_TILE) != 0 || k <= 0 || (k % H3ATTN_LINEAR_KSTEP) != 0)
    return H3ATTN_EINVAL;
  if (x_stride < k || (x_stride & 7) != 0 || w_stride < k || (w_stride & 7) != 0 || y_stride < n_out ||
      (y_stride & 7) != 0)
    return H3ATTN_EINVAL;
  if (rope_cols < 0 || rope_cols > n_out || (rope_cols % h3::kHeadDim) != 0) return H3ATTN_EINVAL;
  if (rope_cols > 0 && (rope_table_dev == nullptr || !aligned16(rope_table_dev))) return H3ATTN_EINVAL;
  // byte offsets inside a 256-row tile and over x are 32-bit
  if (m >= (int64_t(1) << 31) || int64_t(H3ATTN_LINEAR_TILE) * x_stride * 2 >= (int64_t(1) << 31) ||
      int64_t(H3ATTN_LINEAR_TILE) * w_stride * 2 >= (int64_t(1) << 31) ||
      int64_t(H3ATTN_LINEAR_TILE) * y_stride * 2 >= (int64_t(1) << 31) || m * x_stride * 2 >= (int64_t(1) << 32) ||
      int64_t(n_out / H3ATTN_LINEAR_TILE) * ((m + H3ATTN_LINEAR_TILE - 1) / H3ATTN_LINEAR_TILE) >= (int64_t(1) << 30))
    return H3ATTN_ERANGE;
  if (m == 0) return H3ATTN_OK;
  const int64_t yb = span_bytes(m, y_stride, n_out);
  if (overlaps(y, yb, x, span_bytes(m, x_stride, k)) || overlaps(y, yb, w, span_bytes(n_out, w_stride, k)) ||
      (bias != nullptr && overlaps(y, yb, bias, int64_t(n_out) * 2)) ||
      (rope_cols > 0 && overlaps(y, yb, rope_table_dev, m * h3::kPairs * 8)))
    return H3ATTN_EINVAL;
  int rc = check_device();
  if (rc != H3ATTN_OK) return rc;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.rope_tab = rope_table_dev;
  a.x_stride = x_stride;
  a.w_stride = w_stride;
  a.y_stride = y_stride;
  a.m = static_cast<int32_t>(m);
  a.n_out = n_out;
  a.k = k;
  a.rope_cols = rope_cols;
  a.tiles_f = n_out / H3ATTN_LINEAR_TILE;
  a.tiles_t = static_cast<int32_t>((m + H3ATTN_LINEAR_TILE - 1) / H3ATTN_LINEAR_TILE);
  return h3::launch_gemm(a, static_cast<hipStream_t>(stream)) == hipSuccess ? H3ATTN_OK : H3ATTN_EHIP;
}

extern "C" const char* h3attn_strerror(int code) {
  switch (code) {
    case H3ATTN_OK: return "ok";
    case H3ATTN_EINVAL: return "invalid argument";
    case H3ATTN_ERANGE: return "size or coordinate out of range";
    case H3ATTN_EUNSUPPORTED: return "device is not gfx950";
    case H3ATTN_EHIP: return "HIP runtime error";
    case H3ATTN_ESCRATCH: return "shape needs more key-split scratch than h3attn_forward_noalloc holds";
    default: return "unknown error";
  }
}

extern "C" const char* h3attn_version(void) { return "h3attn 0.2.0 gfx950"; }
