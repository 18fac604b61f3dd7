"""Seeded synthetic workloads for the packed text/video/stereo-audio attention path.

This module is shared by the oracle side and the HIP side and holds none of the
method's arithmetic: it only names the segment tables (which segments, in which
row order, with their sizes and time origins) and draws the seeded Q, K, V
inputs.  Everything that turns a segment table into coordinates, rotates, or
attends lives elsewhere, twice, independently.

Segment tables follow the packed-sequence description of the pages:
"Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio" (section 2:
every modality enters one packed sequence; section 4: the shared physical
timeline) and "MiniMax H3 - one transformer that denoises video and audio
together" (latent-frame paragraph: a 44x80 latent sheet patchified 1x2x2 is
22x40 = 880 tokens; 31 latent frames give 27,280 video tokens).

Times are integers in thirds of one audio latent (1/120 s), so that the video
advance of 20/3 clock units per latent frame is exact.
"""
from collections import namedtuple

import numpy as np

TEXT, VIDEO, AUDIO = 0, 1, 2

# kind   : TEXT / VIDEO / AUDIO
# frames : TEXT: tokens | VIDEO: latent frames (1 = a still / reference image) | AUDIO: 40 Hz steps
# grid_h : VIDEO: patch rows | TEXT, AUDIO: 1
# grid_w : VIDEO: patch columns | AUDIO: channels (2 = stereo) | TEXT: 1
# t0_thirds, dt_thirds : time of the first frame and advance per frame, in thirds of a clock unit
Segment = namedtuple("Segment", "kind frames grid_h grid_w t0_thirds dt_thirds")


def text(n, t0):
    """n text tokens at integer clock positions t0, t0+1, ..."""
    return Segment(TEXT, n, 1, 1, 3 * t0, 3)


def video(frames, gh, gw, t0_thirds=0):
    """Latent frames of gh x gw patches, 20/3 clock units apart (4 source frames at 24 fps on a 40 Hz clock)."""
    return Segment(VIDEO, frames, gh, gw, t0_thirds, 20)


def audio(steps, t0, channels=2):
    """40 Hz audio latents, one token per channel per step, one clock unit apart."""
    return Segment(AUDIO, steps, 1, channels, 3 * t0, 3)


def _ref2va():
    segs = [text(1024, -1684)]
    # nine reference images, one latent slot each, back to back, the last ending at -20/3
    segs += [video(1, 22, 40, t0_thirds=-180 + 20 * m) for m in range(9)]
    # three reference audio clips of 200 steps x 2 channels, back to back before the images
    segs += [audio(200, -660 + 200 * a) for a in range(3)]
    segs += [video(31, 22, 40), audio(200, 0)]
    return segs


# name -> (n_heads, segment table); row order is the table order
CONFIGS = {
    "tiny": (2, [text(16, -16), video(1, 4, 8), audio(8, 0)]),
    "4s": (42, [text(256, -256), video(25, 22, 40), audio(160, 0)]),
    "5s": (42, [text(512, -512), video(31, 22, 40), audio(200, 0)]),
    "ref2va": (42, _ref2va()),
    "15s": (42, [text(512, -512), video(91, 22, 40), audio(600, 0)]),
}

# expected packed lengths stated with each workload
CONFIG_TOKENS = {"tiny": 64, "4s": 22576, "5s": 28192, "ref2va": 37824, "15s": 81792}

HEAD_DIM = 128
ROPE_SECTIONS = (32, 48, 48)
ROPE_THETAS = (10000.0, 10000.0, 10000.0)
DEFAULT_SEED = 20260731


def n_tokens(segments):
    """Row count of a segment table (sizes only, no coordinates)."""
    n = 0
    for s in segments:
        n += s.frames * s.grid_h * s.grid_w
    return n


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even) and return the raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, seed, scale=1.0):
    """Seeded N(0, scale^2) draws rounded to bfloat16; returns uint16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def qkv(n, h, seed=DEFAULT_SEED, d=HEAD_DIM, q_scale=1.0):
    """Q, K, V as bf16 bit arrays [n, h, d]; seeds seed, seed+1, seed+2."""
    q = normal_bf16((n, h, d), seed, q_scale)
    k = normal_bf16((n, h, d), seed + 1)
    v = normal_bf16((n, h, d), seed + 2)
    return q, k, v


# ---- AdaLN modulation inputs (hidden size and per-row table selectors)
ADALN_HIDDEN = 5376   # 42 heads x 128
ADALN_PARAMS = 6      # per table entry: shift, scale, gate of the attention path, then of the MLP path


def adaln_rows(segments):
    """Per-row (timestep index, token tag) of a packed sequence, in row order.

    tag: the segment kind (0 text, 1 video, 2 audio).  Timestep index 0 is the
    denoising step of the target rows; text rows take the same index (text
    inherits the video timestep).  Media segments that start before t = 0 are
    references (clean context) and take index 1.
    """
    t_idx, tags = [], []
    for s in segments:
        rows = s.frames * s.grid_h * s.grid_w
        ref = s.kind != TEXT and s.t0_thirds < 0
        t_idx.append(np.full(rows, 1 if ref else 0, np.int32))
        tags.append(np.full(rows, s.kind, np.int32))
    if not t_idx:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    return np.concatenate(t_idx), np.concatenate(tags)


def adaln_inputs(n, c=ADALN_HIDDEN, n_timesteps=2, seed=DEFAULT_SEED, table_scale=0.5):
    """Residual stream x, sublayer output y (bf16 bits [n, c]) and the modulation
    table (bf16 bits [n_timesteps * 3, 6, c]); seeds seed+10, +11, +12."""
    x = normal_bf16((n, c), seed + 10)
    y = normal_bf16((n, c), seed + 11)
    table = normal_bf16((n_timesteps * 3, ADALN_PARAMS, c), seed + 12, table_scale)
    return x, y, table


# ---- latent packing inputs (sampler state and velocity tokens)
VIDEO_LATENT_CHANNELS = 24    # channels per latent cell
AUDIO_LATENT_WIDTH = 32       # values per audio latent frame and channel


def latent_inputs(frames, lat_h, lat_w, audio_steps, n_ch=2, seed=DEFAULT_SEED):
    """Sampler state and velocities of one target clip: video latent float32 [24][frames][lat_h][lat_w],
    its velocity tokens bf16 bits [frames * lat_h/2 * lat_w/2][96], audio latent float32
    [n_ch][audio_steps][32] and its velocity tokens bf16 bits [audio_steps * n_ch][32]; seeds +20..+23."""
    c = VIDEO_LATENT_CHANNELS
    video = np.random.default_rng(seed + 20).standard_normal((c, frames, lat_h, lat_w), dtype=np.float32)
    v_video = normal_bf16((frames * (lat_h // 2) * (lat_w // 2), 4 * c), seed + 21)
    audio = np.random.default_rng(seed + 22).standard_normal((n_ch, audio_steps, AUDIO_LATENT_WIDTH),
                                                             dtype=np.float32)
    v_audio = normal_bf16((audio_steps * n_ch, AUDIO_LATENT_WIDTH), seed + 23)
    return video, v_video, audio, v_audio


# ---- projection inputs
def projection_inputs(m, k, n, seed=DEFAULT_SEED, with_bias=True):
    """Activations x ~ N(0, 1) bf16 bits [m, k], weight ~ N(0, 1/k) bf16 bits [n, k] (so outputs are
    ~ unit variance), bias ~ N(0, 0.1^2) bf16 bits [n] or None; seeds +30, +31, +32."""
    x = normal_bf16((m, k), seed + 30)
    w = normal_bf16((n, k), seed + 31, 1.0 / np.sqrt(k))
    b = normal_bf16((n,), seed + 32, 0.1) if with_bias else None
    return x, w, b
