"""GPU parity of h3attn_linear (projection GEMM with the RoPE epilogue) against
the fp64 oracle (MI355X, gfx950).

Tolerance.  The kernel sums exact bf16 products in float32 (error well below
2^-20 of sum |x||w| for these k), adds the bias, rotates in float32 (error
~1e-6 of the pair norm) and rounds once to bf16.  Test per element:
|y_gpu - y_ref| <= ulp_bf16(|y_ref|) + 1e-5 * (sum_k |x||w| + |b|) + 2e-6 * pair norm.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.linear import linear, qkv_rope

pytestmark = pytest.mark.gpu

SEC, TH = W.ROPE_SECTIONS, W.ROPE_THETAS
f64 = oracle.bf16_bits_to_f64


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_bf16(v):
    e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))[1]
    return np.ldexp(1.0, e - 8)


def pair_norm(y, rope_cols):
    p = np.sqrt(y[:, 0::2] ** 2 + y[:, 1::2] ** 2).repeat(2, axis=1)
    p[:, rope_cols:] = 0
    return p


def check(got_bits, ref, xs, ws, bs, rope_cols, tag=""):
    got = f64(got_bits)
    s = np.abs(xs) @ np.abs(ws).T + (np.abs(bs) if bs is not None else 0)
    tol = ulp_bf16(ref) + 1e-5 * s + 2e-6 * pair_norm(ref, rope_cols)
    err = np.abs(got - ref)
    print("%s max|err| %.3e  max err/tol %.3f" % (tag, float(err.max()), float((err / tol).max())), flush=True)
    assert np.all(np.isfinite(got))
    bad = err > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5])


def segs_of(m):
    # a packed sequence of exactly m rows: text, then stereo audio, then 4x8 video frames
    segs = [W.text(min(m, 20), -20)]
    r = m - min(m, 20)
    a = min(r // 2, 40)
    if a:
        segs.append(W.audio(a, 0))
    r -= 2 * a
    if r >= 32:
        segs.append(W.video(r // 32, 4, 8))
        r -= 32 * (r // 32)
    if r:
        segs.append(W.text(r, 100))
    assert W.n_tokens(segs) == m
    return segs


def run(h3, x, w, b, m, n, k, rope_cols=0, coords=None, x_stride=None, y_stride=None):
    xs, ys = x_stride or k, y_stride or n
    xd = torch.zeros((m, xs), dtype=torch.bfloat16, device="cuda")
    xd[:, :k] = dev_bf16(x)
    wd = dev_bf16(w)
    bd = dev_bf16(b) if b is not None else None
    yd = torch.full((m, ys), 3.0, dtype=torch.bfloat16, device="cuda")
    table = h3.make_rope_table(coords) if rope_cols else None
    h3.linear(xd, xs, wd, k, bd, yd, ys, m, n, k, table, rope_cols)
    torch.cuda.synchronize()
    return host_bits(yd)


@pytest.mark.parametrize("m", [300, 256, 1, 511])
def test_qkv_projection_with_rope(gpu_lib, m):
    heads, k = 2, 512
    n = 3 * heads * 128
    x, w, b = W.projection_inputs(m, k, n, seed=m)
    segs = segs_of(m)
    coords_h = gpu_lib.build_coords(segs)
    y = run(gpu_lib, x, w, b, m, n, k, 2 * heads * 128, torch.from_numpy(coords_h).cuda())
    ref = qkv_rope(f64(x), f64(w), f64(b), coords_h, heads, SEC, TH)
    check(y, ref, f64(x), f64(w), f64(b), 2 * heads * 128, "qkv m=%d" % m)


@pytest.mark.parametrize("k", [64, 128, 192, 320])
def test_short_reductions(gpu_lib, k):
    """One to five 64-deep k stages: the pipeline's first and last stages without a steady state."""
    m, heads = 287, 1
    n = 3 * heads * 128 + 128                     # Q, K, V of one head plus one more 128-wide block
    x, w, b = W.projection_inputs(m, k, n, seed=k)
    coords_h = gpu_lib.build_coords(segs_of(m))
    y = run(gpu_lib, x, w, b, m, n, k, 2 * heads * 128, torch.from_numpy(coords_h).cuda(), x_stride=k + 8)
    yr = linear(f64(x), f64(w), f64(b))
    yr[:, :256] = qkv_rope(f64(x), f64(w[:384]), f64(b[:384]), coords_h, heads, SEC, TH)[:, :256]
    check(y, yr, f64(x), f64(w), f64(b), 2 * heads * 128, "k=%d" % k)


def test_plain_projection_and_strides(gpu_lib):
    m, k, n = 257, 1024, 512
    x, w, _ = W.projection_inputs(m, k, n, seed=3, with_bias=False)
    y = run(gpu_lib, x, w, None, m, n, k, x_stride=k + 40, y_stride=n + 24)
    ref = linear(f64(x), f64(w))
    check(y[:, :n], ref, f64(x), f64(w), None, 0, "plain strided")
    assert np.all(y[:, n:] == host_bits(torch.full((1,), 3.0, dtype=torch.bfloat16))[0])   # padding untouched


@pytest.mark.parametrize("rope", [False, True])
def test_rows_past_m_untouched(gpu_lib, rope):
    """y rows past m (here guard rows of the same allocation) keep their contents: the last token
    tile is partly filled (m = 300: its second 128-row half holds no row at all)."""
    m, heads, k = 300, 1, 256
    n = 3 * heads * 128 + 128
    x, w, b = W.projection_inputs(m, k, n, seed=41)
    coords_h = gpu_lib.build_coords(segs_of(m))
    yd = torch.full((m + 300, n), 3.0, dtype=torch.bfloat16, device="cuda")
    table = gpu_lib.make_rope_table(torch.from_numpy(coords_h).cuda()) if rope else None
    gpu_lib.linear(dev_bf16(x), k, dev_bf16(w), k, dev_bf16(b), yd, n, m, n, k, table,
                   2 * heads * 128 if rope else 0)
    torch.cuda.synchronize()
    y = host_bits(yd)
    assert np.all(y[m:] == host_bits(torch.full((1,), 3.0, dtype=torch.bfloat16))[0])
    yr = linear(f64(x), f64(w), f64(b))
    if rope:
        yr[:, :256] = qkv_rope(f64(x), f64(w[:384]), f64(b[:384]), coords_h, heads, SEC, TH)[:, :256]
    check(y[:m], yr, f64(x), f64(w), f64(b), 2 * heads * 128 if rope else 0, "guard rows rope=%d" % rope)


def test_full_size_qkv_sampled(gpu_lib):
    """The 5 s fused QKV projection (28,192 x 5,376 -> 16,128) in the benchmark's launch shape:
    sampled rows over all 16,128 features, then every row of the Q, K and V slabs of heads 0 and
    41 (the first and last feature tiles of each part, and the last, 32-row token tile)."""
    _, segs = W.CONFIGS["5s"]
    m, k, heads = W.n_tokens(segs), W.ADALN_HIDDEN, 42
    n = 3 * heads * 128
    x, w, b = W.projection_inputs(m, k, n)
    coords_h = gpu_lib.build_coords(segs)
    y = run(gpu_lib, x, w, b, m, n, k, 2 * heads * 128, torch.from_numpy(coords_h).cuda())
    rows = np.unique(np.r_[0, 255, 256, m - 1, np.random.default_rng(8).integers(0, m, 20)])
    ref = qkv_rope(f64(x[rows]), f64(w), f64(b), coords_h[rows], heads, SEC, TH)
    check(y[rows], ref, f64(x[rows]), f64(w), f64(b), 2 * heads * 128, "5s qkv")
    assert not np.any((y & np.uint16(0x7F80)) == np.uint16(0x7F80))      # no bf16 inf / NaN anywhere
    xs = f64(x)
    for h in (0, heads - 1):
        # the one-head fused projection of head h: its Q, K and V weight rows, rotated as in the
        # full projection (the rotation acts on each head alone)
        cols = np.concatenate([np.arange(p * heads * 128 + h * 128, p * heads * 128 + (h + 1) * 128)
                               for p in range(3)])
        ws, bs = f64(w[cols]), f64(b[cols])
        ref = qkv_rope(xs, ws, bs, coords_h, 1, SEC, TH)
        check(y[:, cols], ref, xs, ws, bs, 256, "5s qkv head %d, all rows" % h)


def test_full_size_output_projection(gpu_lib):
    """The 5 s output projection (28,192 x 5,376 -> 5,376, no rotation) in the block's launch shape:
    every row of the first and last 256-feature tiles, and sampled rows over all features."""
    _, segs = W.CONFIGS["5s"]
    m, k = W.n_tokens(segs), W.ADALN_HIDDEN
    n = k
    x, w, b = W.projection_inputs(m, k, n, seed=W.DEFAULT_SEED + 40)
    y = run(gpu_lib, x, w, b, m, n, k)
    xs = f64(x)
    cols = np.r_[0:256, n - 256:n]
    check(y[:, cols], linear(xs, f64(w[cols]), f64(b[cols])), xs, f64(w[cols]), f64(b[cols]), 0,
          "5s out-proj, edge feature tiles, all rows")
    rows = np.unique(np.r_[0, m - 1, np.random.default_rng(9).integers(0, m, 16)])
    check(y[rows], linear(xs[rows], f64(w), f64(b)), xs[rows], f64(w), f64(b), 0, "5s out-proj, sampled rows")


def test_projection_feeds_attention(gpu_lib):
    """Fused QKV output -> h3attn_forward(rope_q = 0) through strided views, against the oracle chain."""
    h3 = gpu_lib
    m, k, heads = 300, 256, 2
    n = 3 * heads * 128
    x, w, b = W.projection_inputs(m, k, n, seed=21)
    segs = segs_of(m)
    coords_h = h3.build_coords(segs)
    coords = torch.from_numpy(coords_h).cuda()
    yd = torch.empty((m, 3, heads, 128), dtype=torch.bfloat16, device="cuda")
    h3.linear(dev_bf16(x), k, dev_bf16(w), k, dev_bf16(b), yd, n, m, n, k, h3.make_rope_table(coords),
              2 * heads * 128)
    o = torch.empty((m, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, m), dtype=torch.float32, device="cuda")
    h3.forward(h3.rope_cfg(), coords, 0, yd[:, 0], yd[:, 1], yd[:, 2], o, lse, m, heads, n, heads * 128)
    torch.cuda.synchronize()
    # the oracle chain from the same seeded inputs: exact projection and rotation, then exact attention
    # (the library rounds Q~, K~, V to bf16 in between; the attention bounds absorb that)
    yr = qkv_rope(f64(x), f64(w), f64(b), coords_h, heads, SEC, TH).reshape(m, 3, heads, 128)
    o_ref, lse_ref = oracle.attention(yr[:, 0], yr[:, 1], yr[:, 2], coords_h, SEC, TH, rope_q=False, rope_k=False)
    err = f64(host_bits(o)) - o_ref
    print("chain max|err| %.3e rms %.3e" % (np.abs(err).max(), np.sqrt((err ** 2).mean())), flush=True)
    assert np.abs(err).max() <= 2e-2 and np.sqrt((err ** 2).mean()) <= 2e-3
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-2


@pytest.mark.parametrize("cfg_name", ["5s", "tiny"])
def test_rope_table_matches_oracle(gpu_lib, cfg_name):
    """h3attn_rope_table: (cos, sin) of every row and pair.  The oracle rotates the unit vector (1, 0) of
    each pair, which gives (cos phi, sin phi) in float64; the kernel's float32 values are within
    6e-8 (angle reduced in float64, then a float32 polynomial) -- test 2.5e-7 absolute."""
    h3 = gpu_lib
    _, segs = W.CONFIGS[cfg_name]
    coords_h = h3.build_coords(segs)
    n = coords_h.shape[0]
    table = torch.full((n + 8, 64, 2), 7.0, dtype=torch.float32, device="cuda")
    h3.rope_table(h3.rope_cfg(), torch.from_numpy(coords_h).cuda(), n, table)
    torch.cuda.synchronize()
    got = table.cpu().numpy().astype(np.float64)
    assert np.all(got[n:] == 7.0)                                         # rows past n untouched
    unit = np.zeros((n, 1, 128))
    unit[:, :, 0::2] = 1.0
    ref = oracle.rope(unit, coords_h, SEC, TH)[:, 0].reshape(n, 64, 2)   # (cos, sin) per pair
    err = np.abs(got[:n] - ref)
    print("%s table max|err| %.3e" % (cfg_name, float(err.max())), flush=True)
    assert err.max() <= 2.5e-7


@pytest.mark.parametrize("sections,thetas", [((48, 40, 40), (5.0e5, 1.0e4, 2.0e3)), ((128, 0, 0), (1.0e4, 1.0e4, 1.0e4))])
def test_rope_table_other_configs(gpu_lib, sections, thetas):
    """The table and the projection that reads it follow the configuration passed to h3attn_rope_table
    (section split and per-axis bases), not the default one; same bounds as above."""
    h3 = gpu_lib
    m, heads, k = 300, 2, 256
    n = 3 * heads * 128
    x, w, b = W.projection_inputs(m, k, n, seed=77)
    coords_h = h3.build_coords(segs_of(m))
    coords = torch.from_numpy(coords_h).cuda()
    table = torch.empty((m, 64, 2), dtype=torch.float32, device="cuda")
    h3.rope_table(h3.rope_cfg(sections, thetas), coords, m, table)
    yd = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    h3.linear(dev_bf16(x), k, dev_bf16(w), k, dev_bf16(b), yd, n, m, n, k, table, 2 * heads * 128)
    torch.cuda.synchronize()
    unit = np.zeros((m, 1, 128))
    unit[:, :, 0::2] = 1.0
    ref_tab = oracle.rope(unit, coords_h, sections, thetas)[:, 0].reshape(m, 64, 2)
    terr = np.abs(table.cpu().numpy().astype(np.float64) - ref_tab).max()
    print("sections %s table max|err| %.3e" % (sections, terr), flush=True)
    assert terr <= 2.5e-7
    ref = qkv_rope(f64(x), f64(w), f64(b), coords_h, heads, sections, thetas)
    check(host_bits(yd), ref, f64(x), f64(w), f64(b), 2 * heads * 128, "qkv sections %s" % (sections,))
