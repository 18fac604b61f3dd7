"""GPU parity of the AdaLN entry points against the fp64 oracle (MI355X, gfx950).

Every call goes through the C ABI via the ctypes binding; expected values come
from oracle.adaln only.

Tolerances.
* Residual x_out = bf16(x + gate * y): the kernel forms x + gate * y with one
  float32 fused multiply-add and rounds that to bf16, the oracle rounds the
  exact sum once.  The two agree except where the float32 result lands exactly
  on a bf16 halfway point that the exact sum does not (about 2^-16 of the
  elements); there they may differ by one bf16 ulp.  Test: every element within
  one ulp, at most 1e-4 of them not bit-equal.
* h = norm(x_out) * (1 + scale) + shift: float32 statistics and arithmetic
  (relative error ~1e-6 of the terms) and one rounding to bf16.  Test:
  |h_gpu - h_ref| <= ulp_bf16(|h_ref|) + 1e-5 * (|n| * (1 + |scale|) + |shift|),
  with n the exact normalised value; elements whose x_out differed are skipped
  there (their normalised input moved by one ulp of x).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import adaln as A

pytestmark = pytest.mark.gpu

EPS = 1e-6


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return A.bf16_bits_to_f64(bits)


def ulp_bf16(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.frexp(np.maximum(a, 2.0 ** -126))[1]
    return np.ldexp(1.0, e - 8)


def tables(table_bits, c):
    """Planes of an [E][6][C] table as float64: shift/scale/gate for attention then MLP."""
    t = f64(table_bits)
    return {k: t[:, i, :] for i, k in enumerate(["shift_a", "scale_a", "gate_a", "shift_m", "scale_m", "gate_m"])}


def check_h(h_bits, h_ref, n_ref, scale_rows, shift_rows, skip=None, tag=""):
    hg = f64(h_bits)
    tol = ulp_bf16(h_ref) + 1e-5 * (np.abs(n_ref) * (1 + np.abs(scale_rows)) + np.abs(shift_rows))
    bad = np.abs(hg - h_ref) > tol
    if skip is not None:
        bad &= ~skip
    print("%s h: max|err| %.3e, max err/tol %.3f, %d over" % (
        tag, float(np.max(np.abs(hg - h_ref))), float(np.max(np.abs(hg - h_ref) / tol)), int(bad.sum())), flush=True)
    assert np.all(np.isfinite(hg))
    assert not bad.any(), np.argwhere(bad)[:5]


def check_xout(xo_bits, xo_ref, tag=""):
    xg = f64(xo_bits)
    diff = xg != xo_ref
    print("%s x_out: %d of %d not bit-equal" % (tag, int(diff.sum()), diff.size), flush=True)
    assert np.all(np.abs(xg - xo_ref) <= ulp_bf16(xo_ref))
    assert diff.sum() <= max(2, 1e-4 * diff.size)
    return diff


def case(n, c, seed, n_timesteps=2):
    x, y, table = W.adaln_inputs(n, c, n_timesteps, seed)
    rng = np.random.default_rng(seed)
    t_idx = rng.integers(0, n_timesteps, n).astype(np.int32)
    tags = rng.integers(0, 3, n).astype(np.int32)
    return x, y, table, t_idx, tags


def run_residual(h3, x, y, table, t_idx, tags, kind, eps=EPS, xy_stride=None, out_stride=None, in_place=False):
    n, c = x.shape
    xs = xy_stride or c
    os_ = xs if in_place else (out_stride or c)
    xd = torch.zeros((n, xs), dtype=torch.bfloat16, device="cuda")
    yd = torch.zeros((n, xs), dtype=torch.bfloat16, device="cuda")
    xd[:, :c] = dev_bf16(x)
    yd[:, :c] = dev_bf16(y)
    tab = dev_bf16(table)
    ti = torch.from_numpy(t_idx).cuda()
    tg = torch.from_numpy(tags).cuda()
    xo = xd if in_place else torch.full((n, os_), 7.0, dtype=torch.bfloat16, device="cuda")
    hd = torch.full((n, os_), 7.0, dtype=torch.bfloat16, device="cuda")
    base = tab.data_ptr()
    h3.adaln_residual(xd, yd, xs, ti, tg, base + 2 * 2 * c, base + 3 * 2 * c, base + 4 * 2 * c, 6 * c,
                      table.shape[0], xo, hd, os_, n, c, kind, eps)
    torch.cuda.synchronize()
    return host_bits(xo[:, :c]), host_bits(hd[:, :c]), host_bits(xo), host_bits(hd)


def reference_residual(x, y, table, t_idx, tags, kind, eps=EPS):
    c = x.shape[1]
    T = tables(table, c)
    idx = A.adaln_index(t_idx, tags)
    xo_ref, h_ref = A.residual_modulate(f64(x), f64(y), idx, T["gate_a"], T["shift_m"], T["scale_m"], kind, eps)
    n_ref = A.norm_rows(xo_ref, kind, eps)
    return xo_ref, h_ref, n_ref, T["scale_m"][idx], T["shift_m"][idx]


@pytest.mark.parametrize("kind", [A.LAYER_NORM, A.RMS_NORM])
def test_residual_parity(gpu_lib, kind):
    x, y, table, t_idx, tags = case(300, W.ADALN_HIDDEN, 101 + kind)
    xo, h, _, _ = run_residual(gpu_lib, x, y, table, t_idx, tags, kind)
    xo_ref, h_ref, n_ref, sc, sh = reference_residual(x, y, table, t_idx, tags, kind)
    diff = check_xout(xo, xo_ref, "residual kind %d" % kind)
    check_h(h, h_ref, n_ref, sc, sh, skip=diff, tag="residual kind %d" % kind)


@pytest.mark.parametrize("kind", [A.LAYER_NORM, A.RMS_NORM])
def test_modulate_parity(gpu_lib, kind):
    x, _, table, t_idx, tags = case(257, W.ADALN_HIDDEN, 201 + kind)
    c = x.shape[1]
    xd, tab = dev_bf16(x), dev_bf16(table)
    ti, tg = torch.from_numpy(t_idx).cuda(), torch.from_numpy(tags).cuda()
    hd = torch.empty_like(xd)
    base = tab.data_ptr()
    gpu_lib.adaln_modulate(xd, c, ti, tg, base, base + 2 * c, 6 * c, table.shape[0], hd, c, x.shape[0], c, kind,
                           EPS)
    torch.cuda.synchronize()
    T = tables(table, c)
    idx = A.adaln_index(t_idx, tags)
    h_ref = A.modulate(f64(x), idx, T["shift_a"], T["scale_a"], kind, EPS)
    check_h(host_bits(hd), h_ref, A.norm_rows(f64(x), kind, EPS), T["scale_a"][idx], T["shift_a"][idx],
            tag="modulate kind %d" % kind)
    # in place: h written over x gives the same bits
    gpu_lib.adaln_modulate(xd, c, ti, tg, base, base + 2 * c, 6 * c, table.shape[0], xd, c, x.shape[0], c, kind,
                           EPS)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(xd), host_bits(hd))


@pytest.mark.parametrize("c", [8, 24, 520, 1032, 4104, 5632, 5640, 8192])
def test_residual_hidden_sizes(gpu_lib, c):
    # every chunk count per lane the library instantiates, full and ragged last chunks
    x, y, table, t_idx, tags = case(37, c, 300 + c)
    xo, h, _, _ = run_residual(gpu_lib, x, y, table, t_idx, tags, A.LAYER_NORM)
    xo_ref, h_ref, n_ref, sc, sh = reference_residual(x, y, table, t_idx, tags, A.LAYER_NORM)
    diff = check_xout(xo, xo_ref, "c=%d" % c)
    check_h(h, h_ref, n_ref, sc, sh, skip=diff, tag="c=%d" % c)


def test_residual_strides_and_in_place(gpu_lib):
    x, y, table, t_idx, tags = case(65, 1032, 77)
    c = x.shape[1]
    xo_ref, h_ref, n_ref, sc, sh = reference_residual(x, y, table, t_idx, tags, A.LAYER_NORM)
    xo, h, xo_full, h_full = run_residual(gpu_lib, x, y, table, t_idx, tags, A.LAYER_NORM, xy_stride=c + 24,
                                          out_stride=c + 8)
    diff = check_xout(xo, xo_ref, "strided")
    check_h(h, h_ref, n_ref, sc, sh, skip=diff, tag="strided")
    assert np.all(xo_full[:, c:] == host_bits(torch.full((1,), 7.0, dtype=torch.bfloat16))[0])   # padding untouched
    assert np.all(h_full[:, c:] == host_bits(torch.full((1,), 7.0, dtype=torch.bfloat16))[0])
    xo2, h2, _, _ = run_residual(gpu_lib, x, y, table, t_idx, tags, A.LAYER_NORM, xy_stride=c + 24, in_place=True)
    assert np.array_equal(xo2, xo) and np.array_equal(h2, h)


def test_residual_closed_forms(gpu_lib):
    c = W.ADALN_HIDDEN
    x, y, table, t_idx, tags = case(64, c, 55)
    # gate 0: the residual is x bit for bit
    t = table.copy()
    t[:, 2, :] = 0
    xo, h, _, _ = run_residual(gpu_lib, x, y, t, t_idx, tags, A.LAYER_NORM)
    assert np.array_equal(xo, x)
    # gate 1, y = -x: the residual is zero and h is the shift entry, exactly
    t[:, 2, :] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    neg = x ^ np.uint16(0x8000)
    xo, h, _, _ = run_residual(gpu_lib, x, neg, t, t_idx, tags, A.LAYER_NORM)
    assert np.all(f64(xo) == 0.0)
    idx = A.adaln_index(t_idx, tags)
    assert np.array_equal(f64(h), f64(t[idx, 3, :]))


def test_invalid_index_rows_are_nan(gpu_lib):
    x, y, table, t_idx, tags = case(40, 520, 9)
    t_idx = t_idx.copy()
    tags = tags.copy()
    t_idx[3], tags[7], t_idx[11], tags[12] = -1, 3, 2, -2       # entry 6+ is outside a 6-entry table
    xo, h, _, _ = run_residual(gpu_lib, x, y, table, t_idx, tags, A.LAYER_NORM)
    bad = np.zeros(40, bool)
    bad[[3, 7, 11, 12]] = True
    assert np.all(np.isnan(f64(h[bad]))) and np.all(np.isnan(f64(xo[bad])))
    ok = ~bad
    xo_ref, h_ref, n_ref, sc, sh = reference_residual(x[ok], y[ok], table, t_idx[ok], tags[ok], A.LAYER_NORM)
    diff = check_xout(xo[ok], xo_ref)
    check_h(h[ok], h_ref, n_ref, sc, sh, skip=diff)


def test_empty_is_a_no_op(gpu_lib):
    z = torch.full((4, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    ti = torch.zeros(4, dtype=torch.int32, device="cuda")
    gpu_lib.adaln_residual(z, z[1:], 16, ti, ti, z, z, z, 0, 1, z[2:], z[3:], 16, 0, 16, 0, EPS)
    torch.cuda.synchronize()
    assert bool((z == 3.0).all())


@pytest.mark.parametrize("name", ["5s", "ref2va"])
def test_residual_full_size_all_rows(gpu_lib, name):
    """The full packed sequence in the launch shape the benchmark times; the oracle checks every row,
    in blocks of 4,096 rows (host memory)."""
    _, segs = W.CONFIGS[name]
    n = W.n_tokens(segs)
    x, y, table = W.adaln_inputs(n, W.ADALN_HIDDEN)
    t_idx, tags = W.adaln_rows(segs)
    xo, h, _, _ = run_residual(gpu_lib, x, y, table, t_idx, tags, A.LAYER_NORM)
    for r0 in range(0, n, 4096):
        rows = np.arange(r0, min(n, r0 + 4096))
        xo_ref, h_ref, n_ref, sc, sh = reference_residual(x[rows], y[rows], table, t_idx[rows], tags[rows],
                                                          A.LAYER_NORM)
        tag = "%s rows %d..%d" % (name, rows[0], rows[-1])
        diff = check_xout(xo[rows], xo_ref, tag)
        check_h(h[rows], h_ref, n_ref, sc, sh, skip=diff, tag=tag)
