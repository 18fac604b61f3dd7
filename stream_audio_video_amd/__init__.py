"""Python binding of libh3attn (MM-RoPE + full attention over one packed sequence, gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels (or, for the coordinate table, its host C++ builder).  PyTorch supplies
device memory and the current stream.  The functions keep the C names:

  build_coords(segments)                          -> float32 [N, 3] numpy array
  rope_qk(cfg, coords_dev, q_in, q_out, k_in, k_out, n_tokens, n_heads, row_stride, stream=None)
  forward(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads,
          row_stride_qkv, row_stride_o, scale=0.0, stream=None)
  adaln_modulate(x, x_stride, t_idx, tags, shift, scale, entry_stride, n_entries, h, h_stride,
                 n_rows, hidden, norm_kind=LAYER_NORM, eps=1e-6, stream=None)
  adaln_residual(x, y, xy_stride, t_idx, tags, gate, shift, scale, entry_stride, n_entries,
                 x_out, h, out_stride, n_rows, hidden, norm_kind=LAYER_NORM, eps=1e-6, stream=None)
  video_euler_pack(latent, channels, frames, lat_h, lat_w, v_tokens, v_stride, dt, tokens, tokens_stride,
                   stream=None)
  audio_euler_pack(latent, n_ch, steps, width, v_tokens, v_stride, dt, tokens, tokens_stride, stream=None)
  av_euler_pack(video_latent, channels, frames, lat_h, lat_w, video_v, video_v_stride, video_tokens,
                video_tokens_stride, audio_latent, n_ch, steps, width, audio_v, audio_v_stride, audio_tokens,
                audio_tokens_stride, dt, stream=None)
  linear(x, x_stride, w, w_stride, bias, y, y_stride, m, n_out, k, rope_table=None, rope_cols=0, stream=None)
  rope_table(cfg, coords_dev, n_tokens, table, stream=None)
  forward_ws(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
             scale, workspace, workspace_bytes, stream=None)
  forward_workspace_bytes(n_tokens, n_heads)
  forward_noalloc(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
                  scale=0.0, stream=None)
  strerror(code), version()

Tensor arguments may be torch tensors (their data_ptr is passed) or raw
integer addresses; None passes NULL.  Errors raise H3AttnError.
"""
import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh3attn.so")
_lib = None

H3ATTN_OK, H3ATTN_EINVAL, H3ATTN_ERANGE, H3ATTN_EUNSUPPORTED, H3ATTN_EHIP, H3ATTN_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20
SEG_TEXT, SEG_VIDEO, SEG_AUDIO = 0, 1, 2
LAYER_NORM, RMS_NORM = 0, 1
ADALN_MAX_HIDDEN = 8192

EXPORTED = ("h3attn_build_coords", "h3attn_rope_qk", "h3attn_forward", "h3attn_adaln_modulate",
            "h3attn_adaln_residual", "h3attn_video_euler_pack", "h3attn_audio_euler_pack", "h3attn_strerror",
            "h3attn_linear", "h3attn_forward_ws", "h3attn_forward_workspace_bytes", "h3attn_version",
            "h3attn_forward_noalloc", "h3attn_av_euler_pack", "h3attn_rope_table")


class H3AttnError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (fn, strerror(code) if _lib else "?", code))


class Segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("frames", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("t0_thirds", ctypes.c_int32), ("dt_thirds", ctypes.c_int32)]


class RopeCfg(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("sec", ctypes.c_int32 * 3), ("theta", ctypes.c_double * 3)]


def rope_cfg(sections=(32, 48, 48), thetas=(10000.0, 10000.0, 10000.0), head_dim=128):
    return RopeCfg(head_dim, (ctypes.c_int32 * 3)(*sections), (ctypes.c_double * 3)(*thetas))


def load_library(path=None):
    """Load libh3attn.so; raises if it is not built (there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libh3attn.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.h3attn_build_coords.argtypes = [ctypes.POINTER(Segment), i32, ctypes.POINTER(ctypes.c_float), i64,
                                        ctypes.POINTER(i64)]
    lib.h3attn_build_coords.restype = ctypes.c_int
    lib.h3attn_rope_qk.argtypes = [ctypes.POINTER(RopeCfg), vp, vp, vp, vp, vp, i64, i32, i64, vp]
    lib.h3attn_rope_qk.restype = ctypes.c_int
    lib.h3attn_forward.argtypes = [ctypes.POINTER(RopeCfg), vp, i32, vp, vp, vp, vp, vp, i64, i32, i64, i64,
                                   ctypes.c_float, vp]
    lib.h3attn_forward.restype = ctypes.c_int
    lib.h3attn_adaln_modulate.argtypes = [vp, i64, vp, vp, vp, vp, i64, i32, vp, i64, i64, i32, i32,
                                          ctypes.c_float, vp]
    lib.h3attn_adaln_modulate.restype = ctypes.c_int
    lib.h3attn_adaln_residual.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, i64, i32, vp, vp, i64, i64, i32, i32,
                                          ctypes.c_float, vp]
    lib.h3attn_adaln_residual.restype = ctypes.c_int
    lib.h3attn_video_euler_pack.argtypes = [vp, i32, i32, i32, i32, vp, i64, ctypes.c_float, vp, i64, vp]
    lib.h3attn_video_euler_pack.restype = ctypes.c_int
    lib.h3attn_audio_euler_pack.argtypes = [vp, i32, i32, i32, vp, i64, ctypes.c_float, vp, i64, vp]
    lib.h3attn_audio_euler_pack.restype = ctypes.c_int
    lib.h3attn_av_euler_pack.argtypes = [vp, i32, i32, i32, i32, vp, i64, vp, i64, vp, i32, i32, i32, vp, i64, vp, i64,
                                         ctypes.c_float, vp]
    lib.h3attn_av_euler_pack.restype = ctypes.c_int
    lib.h3attn_linear.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i32, i32, vp, i32, vp]
    lib.h3attn_rope_table.argtypes = [ctypes.POINTER(RopeCfg), vp, i64, vp, vp]
    lib.h3attn_rope_table.restype = ctypes.c_int
    lib.h3attn_linear.restype = ctypes.c_int
    lib.h3attn_forward_ws.argtypes = [ctypes.POINTER(RopeCfg), vp, i32, vp, vp, vp, vp, vp, i64, i32, i64, i64,
                                      ctypes.c_float, vp, i64, vp]
    lib.h3attn_forward_ws.restype = ctypes.c_int
    lib.h3attn_forward_noalloc.argtypes = [ctypes.POINTER(RopeCfg), vp, i32, vp, vp, vp, vp, vp, i64, i32, i64, i64,
                                           ctypes.c_float, vp]
    lib.h3attn_forward_noalloc.restype = ctypes.c_int
    lib.h3attn_forward_workspace_bytes.argtypes = [i64, i32]
    lib.h3attn_forward_workspace_bytes.restype = i64
    lib.h3attn_strerror.argtypes = [ctypes.c_int]
    lib.h3attn_strerror.restype = ctypes.c_char_p
    lib.h3attn_version.argtypes = []
    lib.h3attn_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _L():
    return _lib if _lib is not None else load_library()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def strerror(code):
    return _L().h3attn_strerror(int(code)).decode()


def version():
    return _L().h3attn_version().decode()


def _segments(segments):
    arr = (Segment * max(1, len(segments)))()
    for i, s in enumerate(segments):
        arr[i] = Segment(*[int(v) for v in tuple(s)[:6]])
    return arr


def build_coords(segments):
    """Coordinates (t, h, w) of every packed row, float32 [N, 3] (host)."""
    lib = _L()
    arr = _segments(segments)
    n = ctypes.c_int64(0)
    rc = lib.h3attn_build_coords(arr, len(segments), None, 0, ctypes.byref(n))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_build_coords", rc)
    out = np.zeros((n.value, 3), np.float32)
    if n.value:
        rc = lib.h3attn_build_coords(arr, len(segments), out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                     n.value, ctypes.byref(n))
        if rc != H3ATTN_OK:
            raise H3AttnError("h3attn_build_coords", rc)
    return out


def rope_qk(cfg, coords_dev, q_in, q_out, k_in, k_out, n_tokens, n_heads, row_stride, stream=None):
    rc = _L().h3attn_rope_qk(ctypes.byref(cfg), _ptr(coords_dev), _ptr(q_in), _ptr(q_out), _ptr(k_in),
                             _ptr(k_out), int(n_tokens), int(n_heads), int(row_stride), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_rope_qk", rc)


def forward(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
            scale=0.0, stream=None):
    rc = _L().h3attn_forward(ctypes.byref(cfg), _ptr(coords_dev), int(rope_q), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(o), _ptr(lse), int(n_tokens), int(n_heads), int(row_stride_qkv),
                             int(row_stride_o), float(scale), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_forward", rc)


def adaln_modulate(x, x_stride, t_idx, tags, shift, scale, entry_stride, n_entries, h, h_stride, n_rows,
                   hidden, norm_kind=LAYER_NORM, eps=1e-6, stream=None):
    rc = _L().h3attn_adaln_modulate(_ptr(x), int(x_stride), _ptr(t_idx), _ptr(tags), _ptr(shift), _ptr(scale),
                                    int(entry_stride), int(n_entries), _ptr(h), int(h_stride), int(n_rows),
                                    int(hidden), int(norm_kind), float(eps), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_adaln_modulate", rc)


def adaln_residual(x, y, xy_stride, t_idx, tags, gate, shift, scale, entry_stride, n_entries, x_out, h,
                   out_stride, n_rows, hidden, norm_kind=LAYER_NORM, eps=1e-6, stream=None):
    rc = _L().h3attn_adaln_residual(_ptr(x), _ptr(y), int(xy_stride), _ptr(t_idx), _ptr(tags), _ptr(gate),
                                    _ptr(shift), _ptr(scale), int(entry_stride), int(n_entries), _ptr(x_out),
                                    _ptr(h), int(out_stride), int(n_rows), int(hidden), int(norm_kind),
                                    float(eps), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_adaln_residual", rc)


def video_euler_pack(latent, channels, frames, lat_h, lat_w, v_tokens, v_stride, dt, tokens, tokens_stride,
                     stream=None):
    rc = _L().h3attn_video_euler_pack(_ptr(latent), int(channels), int(frames), int(lat_h), int(lat_w),
                                      _ptr(v_tokens), int(v_stride), float(dt), _ptr(tokens), int(tokens_stride),
                                      _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_video_euler_pack", rc)


def audio_euler_pack(latent, n_ch, steps, width, v_tokens, v_stride, dt, tokens, tokens_stride, stream=None):
    rc = _L().h3attn_audio_euler_pack(_ptr(latent), int(n_ch), int(steps), int(width), _ptr(v_tokens),
                                      int(v_stride), float(dt), _ptr(tokens), int(tokens_stride), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_audio_euler_pack", rc)


def av_euler_pack(video_latent, channels, frames, lat_h, lat_w, video_v, video_v_stride, video_tokens,
                  video_tokens_stride, audio_latent, n_ch, steps, width, audio_v, audio_v_stride, audio_tokens,
                  audio_tokens_stride, dt, stream=None):
    rc = _L().h3attn_av_euler_pack(_ptr(video_latent), int(channels), int(frames), int(lat_h), int(lat_w),
                                   _ptr(video_v), int(video_v_stride), _ptr(video_tokens), int(video_tokens_stride),
                                   _ptr(audio_latent), int(n_ch), int(steps), int(width), _ptr(audio_v),
                                   int(audio_v_stride), _ptr(audio_tokens), int(audio_tokens_stride), float(dt),
                                   _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_av_euler_pack", rc)


def linear(x, x_stride, w, w_stride, bias, y, y_stride, m, n_out, k, rope_table=None, rope_cols=0, stream=None):
    rc = _L().h3attn_linear(_ptr(x), int(x_stride), _ptr(w), int(w_stride), _ptr(bias), _ptr(y), int(y_stride),
                            int(m), int(n_out), int(k), _ptr(rope_table), int(rope_cols), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_linear", rc)


def rope_table(cfg, coords_dev, n_tokens, table, stream=None):
    rc = _L().h3attn_rope_table(ctypes.byref(cfg), _ptr(coords_dev), int(n_tokens), _ptr(table), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_rope_table", rc)


def make_rope_table(coords_dev, cfg=None):
    """Convenience: the rotation table of a sequence, float32 [N, 64, 2], allocated with torch."""
    import torch
    n = coords_dev.shape[0]
    table = torch.empty((n, 64, 2), dtype=torch.float32, device=coords_dev.device)
    rope_table(cfg or rope_cfg(), coords_dev, n, table)
    return table


def forward_ws(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o, scale,
               workspace, workspace_bytes, stream=None):
    rc = _L().h3attn_forward_ws(ctypes.byref(cfg), _ptr(coords_dev), int(rope_q), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(o), _ptr(lse), int(n_tokens), int(n_heads), int(row_stride_qkv),
                                int(row_stride_o), float(scale), _ptr(workspace), int(workspace_bytes),
                                _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_forward_ws", rc)


def forward_noalloc(cfg, coords_dev, rope_q, q, k, v, o, lse, n_tokens, n_heads, row_stride_qkv, row_stride_o,
                    scale=0.0, stream=None):
    rc = _L().h3attn_forward_noalloc(ctypes.byref(cfg), _ptr(coords_dev), int(rope_q), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(lse), int(n_tokens), int(n_heads), int(row_stride_qkv),
                                     int(row_stride_o), float(scale), _stream(stream))
    if rc != H3ATTN_OK:
        raise H3AttnError("h3attn_forward_noalloc", rc)


def forward_workspace_bytes(n_tokens, n_heads):
    return int(_L().h3attn_forward_workspace_bytes(int(n_tokens), int(n_heads)))


def mmrope_attention(q, k, v, coords_dev, cfg=None, scale=0.0, want_lse=True, fuse_q=True, k_rot=None,
                     out=None, lse=None, split=True):
    """Convenience: rotate K (and Q unless fused), then attend.  q, k, v: bf16 [N, H, 128] CUDA tensors.

    Allocates K~ (and Q~ when not fused), O, LSE and, with split=True, the workspace that lets the
    last, partly filled wave of workgroups run split along the keys (h3attn_forward_ws) with torch
    unless given.  Returns (O, LSE or None).
    """
    import torch
    cfg = cfg or rope_cfg()
    n, h, d = q.shape
    stride = q.stride(0)
    assert k.stride(0) == stride and v.stride(0) == stride
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    if fuse_q:
        rope_qk(cfg, coords_dev, None, None, k, k_rot, n, h, stride)
        q_use = q
    else:
        q_use = torch.empty_like(q)
        rope_qk(cfg, coords_dev, q, q_use, k, k_rot, n, h, stride)
    o = torch.empty((n, h, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((h, n), dtype=torch.float32, device=q.device)
    ws_bytes = forward_workspace_bytes(n, h) if split and n > 0 else 0
    if ws_bytes > 0:
        ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.float32, device=q.device)
        forward_ws(cfg, coords_dev, 1 if fuse_q else 0, q_use, k_rot, v, o, lse if want_lse else None, n, h,
                   stride, o.stride(0), scale, ws, ws_bytes)
    else:
        forward(cfg, coords_dev, 1 if fuse_q else 0, q_use, k_rot, v, o, lse if want_lse else None, n, h,
                stride, o.stride(0), scale)
    return o, (lse if want_lse else None)
