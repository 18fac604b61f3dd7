"""Pins of the packing / Euler oracle (oracle/pack.py): brute-force index loops,
round trips, the pages' worked-example counts, the straight flow path.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import pack as P
from oracle.coords import f32_round


def test_patchify_matches_element_loop():
    # the definition written out: token (t, py, px), value (c, iy, ix) = latent[c][t][2py+iy][2px+ix]
    c, t, h, w = 3, 2, 4, 6
    lat = np.arange(c * t * h * w, dtype=np.float64).reshape(c, t, h, w)
    tok = P.patchify_video(lat)
    assert tok.shape == (t * (h // 2) * (w // 2), 4 * c)
    for tt in range(t):
        for py in range(h // 2):
            for px in range(w // 2):
                row = (tt * (h // 2) + py) * (w // 2) + px
                for cc in range(c):
                    for iy in range(2):
                        for ix in range(2):
                            assert tok[row, (cc * 2 + iy) * 2 + ix] == lat[cc, tt, 2 * py + iy, 2 * px + ix]
    # one element by hand: row (1, 1, 2) = 1*2*3 + 1*3 + 2 = 11, value (c=1, iy=0, ix=1) -> latent[1][1][2][5]
    assert tok[11, 5] == lat[1, 1, 2, 5]


def test_patchify_round_trip_and_worked_example():
    rng = np.random.default_rng(0)
    lat = rng.standard_normal((24, 3, 44, 80))
    tok = P.patchify_video(lat)
    assert tok.shape == (3 * 880, 96)             # 44 x 80 sheet -> 22 x 40 = 880 tokens of 24 x 2 x 2 = 96
    assert np.array_equal(P.unpatchify_video(tok, 24, 3, 44, 80), lat)
    # 31 latent frames of the 5 s example -> 27,280 video tokens
    assert P.patchify_video(np.zeros((24, 31, 44, 80), np.float32)).shape == (27280, 96)
    with pytest.raises(ValueError):
        P.patchify_video(np.zeros((24, 1, 43, 80)))


def test_audio_packing_order():
    n_ch, steps, width = 2, 5, 32
    lat = np.arange(n_ch * steps * width, dtype=np.float64).reshape(n_ch, steps, width)
    tok = P.pack_audio(lat)
    assert tok.shape == (steps * n_ch, width)     # one 32-value token per step and stereo channel
    for s in range(steps):
        for ch in range(n_ch):
            assert np.array_equal(tok[s * n_ch + ch], lat[ch, s])
    assert np.array_equal(P.unpack_audio(tok, n_ch, steps, width), lat)


def test_flow_path_endpoints_and_straight_euler():
    rng = np.random.default_rng(1)
    x0 = rng.standard_normal(1000)
    noise = rng.standard_normal(1000)
    assert np.array_equal(P.flow_point(x0, noise, 1.0), x0)        # t = 1 is the clean sample
    assert np.array_equal(P.flow_point(x0, noise, 0.0), noise)     # t = 0 is pure noise
    # the path is straight, so one Euler step along the exact velocity x0 - noise lands on the path
    v = x0 - noise
    x = P.flow_point(x0, noise, 0.3)
    assert np.max(np.abs(x + 0.25 * v - P.flow_point(x0, noise, 0.55))) < 1e-14
    # and a whole sampler run from t = 0 to t = 1 in 49 uneven steps reaches x0
    ts = np.concatenate([[0.0], np.sort(rng.uniform(0, 1, 48)), [1.0]])
    x = noise.copy()
    for a, b in zip(ts[:-1], ts[1:]):
        x = x + (b - a) * v
    assert np.max(np.abs(x - x0)) < 1e-13


def test_euler_step_rounds_the_exact_sum():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(400) * np.exp(rng.uniform(-8, 8, 400))).astype(np.float32)
    v = np.array([float(np.float32(z)) for z in rng.standard_normal(400)], np.float64)
    v = (np.floor(v * 128) / 128).astype(np.float64)        # short significands, like bfloat16
    dt = np.float32(-0.0417)
    got = P.euler_step(x, v, dt)
    want = np.array([f32_round(Fraction(float(a)) + Fraction(float(dt)) * Fraction(float(b))) for a, b in zip(x, v)],
                    np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_video_and_audio_steps():
    rng = np.random.default_rng(3)
    lat = rng.standard_normal((4, 2, 6, 8)).astype(np.float32)
    vt = rng.standard_normal((2 * 3 * 4, 16))
    new, tok = P.video_euler_pack(lat, vt, 0.5)
    assert np.array_equal(new, P.euler_step(lat, P.unpatchify_video(vt, 4, 2, 6, 8), 0.5))
    assert np.array_equal(tok, P.patchify_video(new))
    same, tok0 = P.video_euler_pack(lat, None, 0.5)
    assert np.array_equal(same, lat) and np.array_equal(tok0, P.patchify_video(lat))
    alat = rng.standard_normal((2, 7, 32)).astype(np.float32)
    av = rng.standard_normal((14, 32))
    anew, atok = P.audio_euler_pack(alat, av, -0.25)
    assert np.array_equal(anew, P.euler_step(alat, P.unpack_audio(av, 2, 7, 32), -0.25))
    assert np.array_equal(atok, P.pack_audio(anew))
