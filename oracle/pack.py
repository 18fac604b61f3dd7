"""Patchify / packing of latents into tokens and the Euler step of the sampler
(oracle; test infrastructure only).

What the pages fix ("MiniMax H3 - one transformer that denoises video and audio
together"):
* patchify paragraph: every non-overlapping 1 x 2 x 2 block of the video latent
  (1 time step x 2 latent rows x 2 latent columns) becomes one token holding the
  block's 24 x 1 x 2 x 2 = 96 channel values;
* latent-frame paragraph: a 44 x 80 latent sheet becomes 22 x 40 = 880 tokens
  that share one time coordinate; one audio latent frame is a single 32-value
  vector, i.e. one token per stereo channel;
* flow-matching paragraphs: x_t = t * x0 + (1 - t) * noise, t = 1 clean and
  t = 0 pure noise; the model predicts a velocity and a non-learned scheduler
  takes one step along it; only the target rows are updated (thread section 2).

Readings where the pages are silent:
* the video latent is channels-first [C][T][H][W]; token rows run frame-major,
  then patch row, then patch column (the coordinate builder's row order); inside
  a token the 4C values run channel-major: index (c * 2 + iy) * 2 + ix;
* the audio latent is per channel, [n_ch][steps][width]; token rows run
  step-major, channel-minor: row s * n_ch + ch holds latent[ch][s][:];
* one Euler step from t to t' = t + dt along the velocity v: x <- x + dt * v;
  the sampler state is float32, tokens are bfloat16 (nearest even).

All arithmetic is float64 unless stated.
"""
import numpy as np


def patchify_video(latent):
    """[C][T][H][W] -> tokens [T * H/2 * W/2][4C] (same dtype, a pure rearrangement)."""
    c, t, h, w = latent.shape
    if h % 2 or w % 2:
        raise ValueError("latent height and width must be even")
    x = latent.reshape(c, t, h // 2, 2, w // 2, 2)          # c, t, py, iy, px, ix
    x = x.transpose(1, 2, 4, 0, 3, 5)                       # t, py, px, c, iy, ix
    return x.reshape(t * (h // 2) * (w // 2), 4 * c)


def unpatchify_video(tokens, c, t, h, w):
    """Inverse of patchify_video."""
    x = np.asarray(tokens).reshape(t, h // 2, w // 2, c, 2, 2)   # t, py, px, c, iy, ix
    x = x.transpose(3, 0, 1, 4, 2, 5)                            # c, t, py, iy, px, ix
    return x.reshape(c, t, h, w)


def pack_audio(latent):
    """[n_ch][steps][width] -> tokens [steps * n_ch][width], row s * n_ch + ch = latent[ch][s]."""
    n_ch, steps, width = latent.shape
    return np.asarray(latent).transpose(1, 0, 2).reshape(steps * n_ch, width)


def unpack_audio(tokens, n_ch, steps, width):
    return np.asarray(tokens).reshape(steps, n_ch, width).transpose(1, 0, 2)


def flow_point(x0, noise, t):
    """The straight path of the pages: x_t = t * x0 + (1 - t) * noise."""
    return t * np.asarray(x0, np.float64) + (1.0 - t) * np.asarray(noise, np.float64)


def euler_step(x, v, dt):
    """x + dt * v for float32 x, float32 dt and bfloat16 v, formed in float64 (dt * v is exact there,
    the sum within 2^-53 relative) and rounded to float32."""
    return (np.asarray(x, np.float64) + np.float64(np.float32(dt)) * np.asarray(v, np.float64)).astype(np.float32)


def video_euler_pack(latent, v_tokens, dt):
    """One sampler step on a video latent (float32) from velocity tokens, then its tokens.

    Returns (new latent float32 [C][T][H][W], tokens as float32 values [rows][4C]
    before their bfloat16 rounding).  v_tokens None: no update, tokens only.
    """
    c, t, h, w = latent.shape
    new = latent.astype(np.float32)
    if v_tokens is not None:
        new = euler_step(latent, unpatchify_video(np.asarray(v_tokens, np.float64), c, t, h, w), dt)
    return new, patchify_video(new)


def audio_euler_pack(latent, v_tokens, dt):
    n_ch, steps, width = latent.shape
    new = latent.astype(np.float32)
    if v_tokens is not None:
        new = euler_step(latent, unpack_audio(np.asarray(v_tokens, np.float64), n_ch, steps, width), dt)
    return new, pack_audio(new)
