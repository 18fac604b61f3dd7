"""Pins of the AdaLN oracle (oracle/adaln.py) against what the pages and the
mathematics fix: the index formula, library norms, closed forms, exact
bfloat16 rounding.  CPU only."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import adaln as A

EPS = 1e-6


def test_round_bf16_matches_integer_rounding_of_float32():
    # An independent route: float32 inputs rounded by the integer bit trick (no
    # double rounding is possible because the inputs are already float32).
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32)])
    want = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)).astype(np.float64)
    got = A.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_ties_overflow_subnormal():
    r = A.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.4e38, -3.4e38,
                               2.0 ** -134, 3 * 2.0 ** -134, 0.0]))
    assert r[0] == 1.0                      # tie to even (down)
    assert r[1] == 1 + 2.0 ** -6            # tie to even (up)
    assert r[2] == -1.0
    assert np.isinf(r[3]) and r[3] > 0 and np.isinf(r[4]) and r[4] < 0
    assert r[5] == 0.0                      # half the smallest subnormal: tie to even zero
    assert r[6] == 2.0 ** -132              # 1.5 quanta: tie to even (2 quanta)
    assert r[7] == 0.0


def test_index_formula_from_the_pages():
    # index = timestep_index * 3 + token_tag; a table whose entry e holds e shows the gather
    t_idx = np.array([0, 1, 2, 0, 3], np.int32)
    tags = np.array([2, 0, 1, 1, 2], np.int32)
    idx = A.adaln_index(t_idx, tags)
    assert idx.tolist() == [2, 3, 7, 1, 11]
    c = 8
    tab = np.repeat(np.arange(12, dtype=np.float64)[:, None], c, axis=1)
    zero = np.zeros((12, c))
    x = np.zeros((5, c))
    h = A.modulate(x, idx, tab, zero, A.LAYER_NORM, EPS)     # zero row: norm is 0, so h = shift
    assert np.array_equal(h[:, 0], np.array([2, 3, 7, 1, 11], np.float64))


@pytest.mark.parametrize("kind", [A.LAYER_NORM, A.RMS_NORM])
def test_norm_matches_torch(kind):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((17, 5376)) * 3 + 0.5
    xt = torch.from_numpy(x)
    if kind == A.LAYER_NORM:
        want = torch.nn.functional.layer_norm(xt, (5376,), eps=EPS).numpy()
    else:
        want = torch.nn.functional.rms_norm(xt, (5376,), eps=EPS).numpy()
    got = A.norm_rows(x, kind, EPS)
    assert np.max(np.abs(got - want)) < 1e-12


def test_modulate_is_affine_layer_norm_for_one_entry():
    rng = np.random.default_rng(3)
    c = 640
    x = rng.standard_normal((9, c))
    shift = rng.standard_normal((4, c)) * 0.5
    scale = rng.standard_normal((4, c)) * 0.5
    idx = np.full(9, 2)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (c,), weight=torch.from_numpy(1 + scale[2]),
                                          bias=torch.from_numpy(shift[2]), eps=EPS).numpy()
    got = A.modulate(x, idx, shift, scale, A.LAYER_NORM, EPS)
    assert np.max(np.abs(got - want)) < 1e-12


def test_layer_norm_moments_closed_form():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 1000)) * np.array([[0.01], [1.0], [7.0], [100.0], [1e-3]]) + 2.0
    n = A.norm_rows(x, A.LAYER_NORM, EPS)
    var = x.var(axis=1)
    assert np.max(np.abs(n.mean(axis=1))) < 1e-12
    assert np.max(np.abs((n * n).mean(axis=1) - var / (var + EPS))) < 1e-12
    r = A.norm_rows(x, A.RMS_NORM, EPS)
    ms = (x * x).mean(axis=1)
    assert np.max(np.abs((r * r).mean(axis=1) - ms / (ms + EPS))) < 1e-12


def test_residual_hand_example():
    # x = [1,2,3,4], y = [4,3,2,1], gate 0.5 -> x_new = [3, 3.5, 4, 4.5] (exact in bfloat16)
    x = np.array([[1.0, 2, 3, 4]])
    y = np.array([[4.0, 3, 2, 1]])
    gate = np.full((1, 4), 0.5)
    shift = np.array([[0.0, 1, 0, -1]])
    scale = np.array([[0.0, 0, 1, 0]])
    x_new, h = A.residual_modulate(x, y, [0], gate, shift, scale, A.LAYER_NORM, EPS)
    assert x_new.tolist() == [[3.0, 3.5, 4.0, 4.5]]
    # mean 3.75, deviations (-0.75, -0.25, 0.25, 0.75), biased variance 0.3125
    s = np.sqrt(0.3125 + EPS)
    want = np.array([-0.75 / s, -0.25 / s + 1, 2 * 0.25 / s, 0.75 / s - 1])
    assert np.max(np.abs(h[0] - want)) < 1e-15


def test_residual_special_cases():
    rng = np.random.default_rng(5)
    c = 256
    x = W.bf16_bits_to_f32(W.normal_bf16((6, c), 7)).astype(np.float64)
    y = rng.standard_normal((6, c))
    tab = rng.standard_normal((3, c))
    zero = np.zeros((3, c))
    idx = np.array([0, 1, 2, 0, 1, 2])
    # gate 0: the residual is untouched and h is the plain modulation of x
    x_new, h = A.residual_modulate(x, y, idx, zero, tab, tab, A.LAYER_NORM, EPS)
    assert np.array_equal(x_new, x)
    assert np.max(np.abs(h - A.modulate(x, idx, tab, tab, A.LAYER_NORM, EPS))) < 1e-15
    # gate 1 and y = -x: the residual cancels to zero and h = shift
    one = np.ones((3, c))
    x_new, h = A.residual_modulate(x, -x, idx, one, tab, zero, A.LAYER_NORM, EPS)
    assert np.array_equal(x_new, np.zeros_like(x))
    assert np.array_equal(h, tab[idx])
    # the residual is rounded once from the exact sum
    g = rng.standard_normal((3, c))
    x_new, h = A.residual_modulate(x, y, idx, g, tab, tab, A.LAYER_NORM, EPS)
    assert np.array_equal(x_new, A.round_bf16(x + g[idx] * y))
    # the next norm reads the stored (rounded) residual row, not the exact sum
    assert np.array_equal(h, A.modulate(x_new, idx, tab, tab, A.LAYER_NORM, EPS))
    assert np.max(np.abs(h - A.modulate(x + g[idx] * y, idx, tab, tab, A.LAYER_NORM, EPS))) > 1e-4


def test_workload_rows():
    t_idx, tags = W.adaln_rows(W.CONFIGS["ref2va"][1])
    assert len(t_idx) == W.CONFIG_TOKENS["ref2va"]
    assert np.bincount(tags).tolist() == [1024, 31 * 880 + 9 * 880, 400 + 3 * 400]
    assert int(t_idx.sum()) == 9 * 880 + 3 * 400   # reference rows take timestep index 1
    t_idx, tags = W.adaln_rows(W.CONFIGS["5s"][1])
    assert int(t_idx.max()) == 0 and np.bincount(tags).tolist() == [512, 27280, 400]
