"""Pins of the oracle's three-axis RoPE.

Pinned against: a textbook 1-D RoPE library routine (GPT-J's adjacent-pair
rotary embedding in ``transformers``), the complex-number definition of the
rotation, group properties of rotations, and the relative-position property
that makes scores depend only on coordinate differences.  Text rows reduce to
plain 1-D RoPE on the time section ("MiniMax H3 - one transformer that denoises
video and audio together", text-position paragraph).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

SEC = W.ROPE_SECTIONS
TH = W.ROPE_THETAS


def _x(n, h, seed=0, d=128):
    return np.random.default_rng(seed).standard_normal((n, h, d))


def _gptj_rope(x, positions, dim):
    """transformers' GPT-J rotary embedding on the first `dim` dims of x [N, H, dim] at integer positions."""
    from transformers.models.gptj import modeling_gptj as g
    table = g.create_sinusoidal_positions(int(max(positions)) + 1, dim)      # [P, dim] = sin | cos
    sc = table[torch.as_tensor(positions, dtype=torch.long)][None]          # [1, N, dim]
    sin, cos = torch.split(sc, dim // 2, dim=-1)
    t = torch.as_tensor(x, dtype=torch.float32)[None]                       # [1, N, H, dim]
    return g.apply_rotary_pos_emb(t, sin, cos)[0].double().numpy()


def test_text_only_is_library_1d_rope():
    n = 300
    x = _x(n, 3, 1)
    coords = np.zeros((n, 3), np.float32)
    coords[:, 0] = np.arange(n)
    y = oracle.rope(x, coords, SEC, TH)
    ref = _gptj_rope(x[:, :, :32], np.arange(n), 32)
    assert np.max(np.abs(y[:, :, :32] - ref)) < 2e-4        # library runs in float32
    assert np.array_equal(y[:, :, 32:], x[:, :, 32:])       # h = w = 0 leave the spatial dims alone


@pytest.mark.parametrize("axis,off,d", [(1, 32, 48), (2, 80, 48)])
def test_spatial_sections_are_library_1d_rope(axis, off, d):
    n = 64
    x = _x(n, 2, 2)
    coords = np.zeros((n, 3), np.float32)
    coords[:, axis] = np.arange(n)
    y = oracle.rope(x, coords, SEC, TH)
    ref = _gptj_rope(x[:, :, off:off + d], np.arange(n), d)
    assert np.max(np.abs(y[:, :, off:off + d] - ref)) < 1e-4
    mask = np.ones(128, bool)
    mask[off:off + d] = False
    assert np.array_equal(y[:, :, mask], x[:, :, mask])


def test_complex_multiply_form():
    """Each adjacent pair is the complex number x + iy multiplied by exp(i pos theta)."""
    n = 40
    x = _x(n, 2, 3)
    coords = np.random.default_rng(4).uniform(-700, 700, (n, 3)).astype(np.float32)
    y = oracle.rope(x, coords, SEC, TH)
    zx = x[..., 0::2] + 1j * x[..., 1::2]
    pos = np.concatenate([np.repeat(coords[:, a:a + 1].astype(np.float64), SEC[a] // 2, 1) for a in range(3)], 1)
    freq = np.concatenate([TH[a] ** (-np.arange(0, SEC[a], 2) / SEC[a]) for a in range(3)])
    zy = zx * np.exp(1j * pos * freq)[:, None, :]
    assert np.max(np.abs(y[..., 0::2] - zy.real)) < 1e-12
    assert np.max(np.abs(y[..., 1::2] - zy.imag)) < 1e-12


def test_basis_vector_rotates_forward():
    """e_0 at t = 1 turns by +1 radian into dim 1; e_32 at h = 2 turns by +2 rad into dim 33."""
    x = np.zeros((2, 1, 128))
    x[0, 0, 0] = 1.0
    x[1, 0, 32] = 1.0
    c = np.array([[1, 0, 0], [0, 2, 0]], np.float32)
    y = oracle.rope(x, c, SEC, TH)
    assert np.allclose(y[0, 0, :2], [np.cos(1.0), np.sin(1.0)], atol=1e-15)
    assert np.allclose(y[1, 0, 32:34], [np.cos(2.0), np.sin(2.0)], atol=1e-15)


def test_identity_at_origin_and_norm():
    x = _x(20, 2, 5)
    assert np.array_equal(oracle.rope(x, np.zeros((20, 3), np.float32), SEC, TH), x)
    c = np.random.default_rng(6).uniform(-2000, 2000, (20, 3)).astype(np.float32)
    y = oracle.rope(x, c, SEC, TH)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(nx - ny)) < 1e-12


def test_composition():
    x = _x(16, 1, 7)
    rng = np.random.default_rng(8)
    c1 = rng.integers(-300, 300, (16, 3)).astype(np.float32)
    c2 = rng.integers(-300, 300, (16, 3)).astype(np.float32)
    y = oracle.rope(oracle.rope(x, c1, SEC, TH), c2, SEC, TH)
    z = oracle.rope(x, c1 + c2, SEC, TH)
    assert np.max(np.abs(y - z)) < 1e-11


def test_scores_depend_only_on_coordinate_differences():
    n = 48
    q, k = _x(n, 2, 9), _x(n, 2, 10)
    # coordinates on a 1/8 grid, so that the translation below is exact in float32
    c = (np.random.default_rng(11).integers(-800, 800, (n, 3)) / 8.0).astype(np.float32)
    s0 = np.einsum("ihd,jhd->hij", oracle.rope(q, c, SEC, TH), oracle.rope(k, c, SEC, TH))
    c2 = c + np.array([37.0, -5.0, 11.0], np.float32)
    s1 = np.einsum("ihd,jhd->hij", oracle.rope(q, c2, SEC, TH), oracle.rope(k, c2, SEC, TH))
    assert np.max(np.abs(s0 - s1)) < 1e-10
