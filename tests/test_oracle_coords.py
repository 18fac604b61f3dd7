"""Pins of the oracle's coordinate builder against what the pages fix.

Sources: "MiniMax H3 - one transformer that denoises video and audio together"
(latent-frame worked example, clock-rate mismatch, causal downsampler count,
clock unit and 5/3 rescale, text as 1-D RoPE, normalised spatial grid) and
"Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio", section 4
(L/R audio share t and differ on another axis).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _rows_of(segments, kind):
    """Row ranges of each segment of a kind (sizes only)."""
    out, r = [], 0
    for s in segments:
        n = s.frames * s.grid_h * s.grid_w
        if s.kind == kind:
            out.append((r, r + n, s))
        r += n
    return out


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_config_token_totals(name):
    h, segs = W.CONFIGS[name]
    c = oracle.build_coords(segs)
    assert c.shape == (W.CONFIG_TOKENS[name], 3)
    assert c.dtype == np.float32


def test_worked_example_counts():
    g = GOLD
    gh, gw = (g["latent_sheet_hw"][0] // g["patch_hw"][0], g["latent_sheet_hw"][1] // g["patch_hw"][1])
    assert gh * gw == g["tokens_per_latent_frame"]
    assert g["patch_channels"] * 1 * g["patch_hw"][0] * g["patch_hw"][1] == g["token_dim"]
    # causal temporal downsampler: T source frames -> (T - 1)/r + 1 latents; 5 s at 24 fps
    T = 5 * g["fps"] + 1
    assert (T - 1) // g["temporal_stride"] + 1 == g["latent_frames_5s"]
    assert g["latent_frames_5s"] * g["tokens_per_latent_frame"] == g["video_tokens_5s"]
    _, segs = W.CONFIGS["5s"]
    c = oracle.build_coords(segs)
    (v0, v1, seg), = _rows_of(segs, W.VIDEO)
    assert v1 - v0 == g["video_tokens_5s"]
    # every one of the 880 tokens of a latent frame carries the same t and differs in h, w
    vt = c[v0:v1].reshape(g["latent_frames_5s"], g["tokens_per_latent_frame"], 3)
    assert np.all(vt[:, :, 0] == vt[:, :1, 0])
    hw = {(float(a), float(b)) for a, b in vt[0, :, 1:]}
    assert len(hw) == g["tokens_per_latent_frame"]


def test_rate_mismatch_and_alignment():
    """Index 3 is 0.5 s of video but 0.075 s of audio; on the shared clock they line up by time."""
    g = GOLD
    clock = Fraction(1, g["audio_latents_per_s"])
    assert Fraction(3, g["video_latent_frames_per_s"]) == Fraction(g["index3_video_seconds"]).limit_denominator(1000)
    assert 3 * clock == Fraction(g["index3_audio_seconds"]).limit_denominator(10000)
    # clock units per 24 fps frame
    assert Fraction(1, g["fps"]) / clock == Fraction(*g["frame_rescale_clock_units"])
    _, segs = W.CONFIGS["5s"]
    c = oracle.build_coords(segs)
    (v0, v1, _), = _rows_of(segs, W.VIDEO)
    (a0, a1, _), = _rows_of(segs, W.AUDIO)
    vt = c[v0:v1:880, 0]
    at = c[a0:a1:2, 0]
    for k, t in enumerate(vt):
        # latent k stands for source frame 4k at 24 fps, i.e. 4k/24 s, in 1/40 s clock units
        secs = Fraction(g["temporal_stride"] * k, g["fps"])
        assert t == oracle.f32_round(secs / clock)
    # latent frame 3 = 0.5 s = audio step 20
    assert vt[3] == at[20] == np.float32(20.0)
    # exactly the frames k = 0, 3, ..., 27 share a time with an audio step of the 5 s clip
    shared = [k for k, t in enumerate(vt) if t in set(at.tolist())]
    assert shared == list(range(0, 28, 3))


def test_stereo_pairs_share_t_and_split_on_w():
    for name in ("tiny", "5s", "ref2va"):
        _, segs = W.CONFIGS[name]
        c = oracle.build_coords(segs)
        for a0, a1, s in _rows_of(segs, W.AUDIO):
            blk = c[a0:a1].reshape(s.frames, 2, 3)
            assert np.array_equal(blk[:, 0, 0].view(np.uint32), blk[:, 1, 0].view(np.uint32))
            assert np.all(blk[:, :, 1] == 0)
            assert np.all(blk[:, 0, 2] == 0) and np.all(blk[:, 1, 2] == 1)
            assert np.array_equal(blk[:, 0, 0], (np.arange(s.frames) + s.t0_thirds // 3).astype(np.float32))


def test_text_rows_are_1d():
    for name in W.CONFIGS:
        _, segs = W.CONFIGS[name]
        c = oracle.build_coords(segs)
        for r0, r1, s in _rows_of(segs, W.TEXT):
            assert np.all(c[r0:r1, 1:] == 0)
            t = c[r0:r1, 0]
            assert np.array_equal(np.diff(t), np.ones(r1 - r0 - 1, np.float32))
        # text occupies the integer slots right before the earliest media time
        media_t = min(float(c[r0:r1, 0].min()) for kind in (W.VIDEO, W.AUDIO)
                      for r0, r1, _ in _rows_of(segs, kind))
        (r0, r1, _), = _rows_of(segs, W.TEXT)
        assert float(c[r1 - 1, 0]) == math.ceil(media_t) - 1


def test_tiny_matches_its_statement():
    """Tiny: text t = i - 16, h = w = 0; one 4x8 latent frame at t = 0; audio t = j, h = 0, w = ch."""
    _, segs = W.CONFIGS["tiny"]
    c = oracle.build_coords(segs)
    assert np.array_equal(c[:16, 0], np.arange(16, dtype=np.float32) - 16)
    assert np.all(c[16:48, 0] == 0)
    j = np.repeat(np.arange(8), 2)
    ch = np.tile(np.arange(2), 8)
    assert np.array_equal(c[48:, 0], j.astype(np.float32))
    assert np.array_equal(c[48:, 2], ch.astype(np.float32))
    assert np.all(c[48:, 1] == 0)


def test_f32_round_agrees_with_ieee_division():
    rng = np.random.default_rng(7)
    vals = list(range(-3000, 3001)) + rng.integers(-(2 ** 24) + 1, 2 ** 24, 3000).tolist()
    for t3 in vals:
        a = oracle.f32_round(Fraction(t3, 3))
        b = np.float32(t3) / np.float32(3)
        assert a.view(np.uint32) == b.view(np.uint32), t3


def test_f32_round_ties_and_edges():
    # halfway between 1 and the next binary32 (1 + 2^-23) rounds to even (1.0)
    assert oracle.f32_round(1 + Fraction(1, 2 ** 24)) == np.float32(1.0)
    # just above halfway rounds up
    assert oracle.f32_round(1 + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 60)) == np.nextafter(np.float32(1), np.float32(2))
    # 3 * 2^-24 sits halfway between 1 + 2^-23 and 1 + 2^-22: rounds to the even one (1 + 2^-22)
    assert oracle.f32_round(1 + Fraction(3, 2 ** 24)) == np.float32(1 + 2.0 ** -22)
    assert oracle.f32_round(Fraction(-20, 3)) == -oracle.f32_round(Fraction(20, 3))
    assert oracle.f32_round(Fraction(2 ** 24 + 1)) == np.float32(2 ** 24)     # tie -> even
    assert oracle.f32_round(Fraction(2 ** 24 + 3)) == np.float32(2 ** 24 + 4)  # tie -> even


@pytest.mark.parametrize("gh,gw", [(22, 40), (4, 8), (44, 80), (9, 16), (1, 1), (3, 5)])
def test_spatial_grid_invariants(gh, gw):
    hs, ws = oracle.video_hw_f64(gh, gw)
    hs, ws = np.array(hs), np.array(ws)
    sp = 32.0 / math.sqrt(gh * gw)
    # centred on the middle of the [0, 32) canvas
    assert abs(hs.mean() - 16.0) < 1e-12 and abs(ws.mean() - 16.0) < 1e-12
    # uniform spacing 32 / sqrt(H W) in both axes (resolution-free, aspect kept)
    if gh > 1:
        assert np.allclose(np.diff(hs), sp, rtol=0, atol=1e-12)
    if gw > 1:
        assert np.allclose(np.diff(ws), sp, rtol=0, atol=1e-12)
    # cell-edge extents 32 sqrt(H/W) x 32 sqrt(W/H): the wider axis spans wider
    ext_h = hs[-1] - hs[0] + sp
    ext_w = ws[-1] - ws[0] + sp
    assert abs(ext_h - 32.0 * math.sqrt(gh / gw)) < 1e-12
    assert abs(ext_w - 32.0 * math.sqrt(gw / gh)) < 1e-12
    assert abs(ext_h * ext_w - 1024.0) < 1e-9


def test_same_aspect_same_range():
    """A 768p-like and a 2x denser grid of one aspect ratio cover the same coordinate range."""
    h1, w1 = oracle.video_hw_f64(22, 40)
    h2, w2 = oracle.video_hw_f64(44, 80)
    s1, s2 = 32 / math.sqrt(880), 32 / math.sqrt(3520)
    assert abs((h1[0] - s1 / 2) - (h2[0] - s2 / 2)) < 1e-12
    assert abs((w1[-1] + s1 / 2) - (w2[-1] + s2 / 2)) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 8, 32])
def test_square_grid_is_cell_centres(n):
    hs, ws = oracle.video_hw_f64(n, n)
    cells = [(r + 0.5) * 32.0 / n for r in range(n)]
    assert np.allclose(hs, cells, rtol=0, atol=1e-12)
    assert np.allclose(ws, cells, rtol=0, atol=1e-12)


def test_video_rows_round_once_from_f64():
    _, segs = W.CONFIGS["tiny"]
    c = oracle.build_coords(segs)
    hs, ws = oracle.video_hw_f64(4, 8)
    blk = c[16:48].reshape(4, 8, 3)
    assert np.array_equal(blk[:, 0, 1], np.array(hs, np.float64).astype(np.float32))
    assert np.array_equal(blk[0, :, 2], np.array(ws, np.float64).astype(np.float32))


def test_empty_and_zero_frame_segments():
    assert oracle.build_coords([]).shape == (0, 3)
    c = oracle.build_coords([W.text(0, 0), W.audio(0, 0), W.text(3, 5)])
    assert np.array_equal(c[:, 0], np.array([5, 6, 7], np.float32))
