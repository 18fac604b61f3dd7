"""Pins of the projection oracle (oracle/linear.py): a plain loop, a library
linear layer, and the rotation applied only where the pages put it.  CPU only."""
import numpy as np
import torch

import oracle
import workloads as W
from oracle.linear import linear, qkv_rope


def test_linear_matches_loop_and_library():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    b = rng.standard_normal(3)
    y = linear(x, w, b)
    for i in range(5):
        for j in range(3):
            assert abs(y[i, j] - (sum(x[i, k] * w[j, k] for k in range(7)) + b[j])) < 1e-12
    xt, wt, bt = (torch.from_numpy(a) for a in (x, w, b))
    assert np.max(np.abs(y - torch.nn.functional.linear(xt, wt, bt).numpy())) < 1e-12
    assert np.max(np.abs(linear(x, w) - x @ w.T)) < 1e-12


def test_qkv_rope_rotates_q_and_k_only():
    rng = np.random.default_rng(1)
    heads, m, kdim = 2, 9, 32
    segs = [W.text(3, -3), W.video(1, 2, 3)]
    coords = oracle.build_coords(segs)
    x = rng.standard_normal((m, kdim))
    w = rng.standard_normal((3 * heads * 128, kdim))
    y = linear(x, w)
    out = qkv_rope(x, w, None, coords, heads, W.ROPE_SECTIONS, W.ROPE_THETAS)
    hd = heads * 128
    # V untouched, Q and K rotated per head by the row's coordinates
    assert np.array_equal(out[:, 2 * hd:], y[:, 2 * hd:])
    for part in (0, 1):
        blk = y[:, part * hd:(part + 1) * hd].reshape(m, heads, 128)
        want = oracle.rope(blk, coords, W.ROPE_SECTIONS, W.ROPE_THETAS).reshape(m, hd)
        assert np.max(np.abs(out[:, part * hd:(part + 1) * hd] - want)) < 1e-12
    # rotation preserves each pair's norm, and text rows' h/w sections are untouched (h = w = 0)
    q = out[:, :hd].reshape(m, heads, 128)
    q0 = y[:, :hd].reshape(m, heads, 128)
    assert np.max(np.abs(np.hypot(q[..., 0::2], q[..., 1::2]) - np.hypot(q0[..., 0::2], q0[..., 1::2]))) < 1e-9
    assert np.array_equal(q[:3, :, 32:], q0[:3, :, 32:])
    # scores between rotated Q and K depend only on coordinate differences (shift every row's coords;
    # coordinates on a 1/8 grid so that the shifted values stay exact in float32)
    grid = (rng.integers(-256, 256, (m, 3)) / 8).astype(np.float32)
    out = qkv_rope(x, w, None, grid, heads, W.ROPE_SECTIONS, W.ROPE_THETAS)
    out2 = qkv_rope(x, w, None, grid + np.float32(8.0), heads, W.ROPE_SECTIONS, W.ROPE_THETAS)
    s1 = np.einsum("ihd,jhd->hij", out[:, :hd].reshape(m, heads, 128), out[:, hd:2 * hd].reshape(m, heads, 128))
    s2 = np.einsum("ihd,jhd->hij", out2[:, :hd].reshape(m, heads, 128), out2[:, hd:2 * hd].reshape(m, heads, 128))
    assert np.max(np.abs(s1 - s2)) < 1e-8 * np.max(np.abs(s1))
