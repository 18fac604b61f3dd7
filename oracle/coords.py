"""Coordinate table of the packed sequence (oracle; test infrastructure only).

Each packed row gets a position triple (t, h, w).  The rules, from the pages:

* Clock: one unit is one audio latent, 1/40 s.  A 24 fps source frame lasts
  40/24 = 5/3 units ("MiniMax H3 - one transformer that denoises video and audio
  together", clock-unit paragraph; "Inside MiniMax H3 ...", section 4).  A video
  latent frame k stands for source frame 4k (temporal stride 4, causal
  downsampler paragraph), so it sits at t = 4k * 5/3 = 20k/3.
* Audio step j sits at t = j.  Left and right channels share t and differ on
  another axis, here w = channel, h = 0 ("Inside MiniMax H3 ...", section 4).
* Text token i has t = t0 + i and h = w = 0: plain 1-D RoPE on the time axis
  (explainer, text-position paragraph).  The origin t0 is an input.
* Video h, w: the patch grid normalised by sqrt(rows * cols) and centred on the
  [0, 32) canvas with the aspect ratio kept (explainer, spatial-grid paragraph).
  Read here as: spacing 32 / sqrt(H W), cell centres, mean 16.

Rows are emitted in segment order; VIDEO frame-major then row-major (r, c);
AUDIO step-major, channel-minor; TEXT in order.

Precision: t is the exact rational t3 / 3 rounded once to binary32 (ties to
even); h and w are evaluated as separate IEEE binary64 operations and rounded
once to binary32.
"""
import math
from fractions import Fraction

import numpy as np

TEXT, VIDEO, AUDIO = 0, 1, 2


def f32_round(fr):
    """Round an exact rational to the nearest binary32 value, ties to even.

    Written with integer arithmetic only (no floating-point division), so that it
    can serve as an independent definition of the rounded coordinate.
    """
    fr = Fraction(fr)
    if fr == 0:
        return np.float32(0.0)
    neg = fr < 0
    a = -fr if neg else fr
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if not Fraction(2) ** e <= a < Fraction(2) ** (e + 1):
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    if e > 127:
        raise OverflowError("value exceeds binary32 range")
    q = max(e - 23, -149)                  # weight of the last mantissa bit
    scaled = a / (Fraction(2) ** q)        # exact
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(n) * 2.0 ** q              # exact in binary64: n <= 2^24
    if val >= 2.0 ** 128:
        raise OverflowError("value exceeds binary32 range")
    return np.float32(-val if neg else val)


def video_hw_f64(grid_h, grid_w):
    """Cell-centre coordinates of a grid_h x grid_w patch grid, before rounding.

    spacing s2 = 32 / sqrt(H W); centre r -> 16 + (r + 1/2 - H/2) * s2, evaluated
    as 16 + (2r + 1 - H) * (16 / sqrt(H W)) in separate binary64 operations.
    Returns (h[grid_h], w[grid_w]) as Python-float lists.
    """
    s = 16.0 / math.sqrt(float(grid_h * grid_w))
    hs = [16.0 + float(2 * r + 1 - grid_h) * s for r in range(grid_h)]
    ws = [16.0 + float(2 * c + 1 - grid_w) * s for c in range(grid_w)]
    return hs, ws


def _seg_fields(s):
    return (int(s[0]), int(s[1]), int(s[2]), int(s[3]), int(s[4]), int(s[5]))


def build_coords(segments):
    """Segment table -> float32 array [N, 3] of (t, h, w), in packed row order."""
    parts = []
    for s in segments:
        kind, frames, gh, gw, t0, dt = _seg_fields(s)
        if frames < 0 or gh < 1 or gw < 1:
            raise ValueError("bad segment sizes")
        if frames == 0:
            continue
        t_frame = np.array([f32_round(Fraction(t0 + f * dt, 3)) for f in range(frames)],
                           dtype=np.float32)
        if kind == TEXT:
            if gh != 1 or gw != 1:
                raise ValueError("text segment must have grid 1x1")
            rows = np.zeros((frames, 3), np.float32)
            rows[:, 0] = t_frame
        elif kind == AUDIO:
            if gh != 1:
                raise ValueError("audio segment must have grid_h 1")
            rows = np.zeros((frames, gw, 3), np.float32)
            rows[:, :, 0] = t_frame[:, None]
            rows[:, :, 2] = np.arange(gw, dtype=np.float32)[None, :]
            rows = rows.reshape(frames * gw, 3)
        elif kind == VIDEO:
            hs, ws = video_hw_f64(gh, gw)
            h32 = np.array([np.float32(x) for x in hs], np.float32)
            w32 = np.array([np.float32(x) for x in ws], np.float32)
            rows = np.zeros((frames, gh, gw, 3), np.float32)
            rows[..., 0] = t_frame[:, None, None]
            rows[..., 1] = h32[None, :, None]
            rows[..., 2] = w32[None, None, :]
            rows = rows.reshape(frames * gh * gw, 3)
        else:
            raise ValueError("unknown segment kind %d" % kind)
        parts.append(rows)
    if not parts:
        return np.zeros((0, 3), np.float32)
    return np.ascontiguousarray(np.concatenate(parts, axis=0))
