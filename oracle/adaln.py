"""Indexed AdaLN modulation around attention (oracle; test infrastructure only).

What the pages fix:
* "MiniMax H3 - one transformer that denoises video and audio together",
  AdaLN paragraphs: a sublayer input is normalised and then modulated,
  y = norm(x) * (1 + scale) + shift; H3 keeps a table indexed by
  (noise level, modality) and every row looks up its own entry with
  index = timestep_index * 3 + token_tag.
* "Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio",
  section 5: every block produces shift, scale and gate for both the attention
  and the MLP path, selected by the diffusion timestep and by whether the row
  is text, video or audio; the values are gathered per row.

Readings where the pages are silent (each one also stated with the library):
* norm is a layer norm without learned affine (the modulation replaces it):
  (x - mean) / sqrt(var + eps), biased variance over the hidden dim; a
  root-mean-square norm x / sqrt(mean(x^2) + eps) is offered as the other kind;
* a gate multiplies the sublayer output before it joins the residual stream:
  x_new = x + gate * y;
* the residual stream and the modulated output are bfloat16, the residual is
  rounded once (nearest even) and the norm that follows reads the rounded row.

All arithmetic is float64.
"""
import numpy as np

LAYER_NORM, RMS_NORM = 0, 1
N_TAGS = 3   # text, video, audio


def bf16_bits_to_f64(bits):
    """Exact widening of raw bfloat16 bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(v):
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits with the float32 exponent range; below
    2^-126 the quantum stays 2^-133.  Magnitudes that round to 2^128 or more
    overflow to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    fin = np.isfinite(v) & (v != 0)
    m, e = np.frexp(v[fin])                     # v = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))  # quantum of the result
    r = np.round(v[fin] / q) * q                # numpy rounds halves to even
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    out[~fin] = v[~fin]
    return out


def bits_of_bf16(v):
    """Raw bits of values that are already exact bfloat16 numbers (float64 input)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def adaln_index(t_idx, tags):
    """Table entry of every row: timestep_index * 3 + token_tag."""
    return np.asarray(t_idx, np.int64) * N_TAGS + np.asarray(tags, np.int64)


def norm_rows(x, kind, eps):
    """Normalise every row of x [N, C] (float64) without affine."""
    x = np.asarray(x, dtype=np.float64)
    if kind == LAYER_NORM:
        mu = x.mean(axis=1, keepdims=True)
        d = x - mu
        var = (d * d).mean(axis=1, keepdims=True)
        return d / np.sqrt(var + eps)
    if kind == RMS_NORM:
        ms = (x * x).mean(axis=1, keepdims=True)
        return x / np.sqrt(ms + eps)
    raise ValueError("unknown norm kind")


def modulate(x, idx, shift_tab, scale_tab, kind, eps):
    """norm(x) * (1 + scale[idx]) + shift[idx] per row; tables [E, C]; returns float64 [N, C]."""
    idx = np.asarray(idx, np.int64)
    shift = np.asarray(shift_tab, np.float64)[idx]
    scale = np.asarray(scale_tab, np.float64)[idx]
    return norm_rows(x, kind, eps) * (1.0 + scale) + shift


def residual_modulate(x, y, idx, gate_tab, shift_tab, scale_tab, kind, eps):
    """Gated residual then the next sublayer's modulated norm.

    x_new = RN_bf16(x + gate[idx] * y);  h = norm(x_new) * (1 + scale[idx]) + shift[idx].
    Returns (x_new as exact bf16 values in float64, h in float64).
    """
    idx = np.asarray(idx, np.int64)
    gate = np.asarray(gate_tab, np.float64)[idx]
    x_new = round_bf16(np.asarray(x, np.float64) + gate * np.asarray(y, np.float64))
    return x_new, modulate(x_new, idx, shift_tab, scale_tab, kind, eps)
