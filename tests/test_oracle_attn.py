"""Pins of the oracle's attention.

Pinned against: 50-digit brute force (mpmath) on a small case, PyTorch's
scaled_dot_product_attention on the CPU in float64 (a library routine), closed
forms, permutation equivariance (shuffle the rows and the answer comes back
shuffled: "MiniMax H3 - one transformer that denoises video and audio
together", permutation paragraph) and bidirectionality (no mask; target rows
inform reference rows: same page, paragraph on the missing cross-step cache).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

SEC, TH = W.ROPE_SECTIONS, W.ROPE_THETAS


def _tiny(seed=W.DEFAULT_SEED, q_scale=1.0):
    h, segs = W.CONFIGS["tiny"]
    c = oracle.build_coords(segs)
    q, k, v = (oracle.bf16_bits_to_f64(a) for a in W.qkv(len(c), h, seed, q_scale=q_scale))
    return q, k, v, c


def test_matches_library_sdpa_fp64():
    q, k, v, c = _tiny()
    o, lse = oracle.attention(q, k, v, c, SEC, TH)
    qr = torch.from_numpy(oracle.rope(q, c, SEC, TH)).permute(1, 0, 2)
    kr = torch.from_numpy(oracle.rope(k, c, SEC, TH)).permute(1, 0, 2)
    vr = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vr).permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    s = torch.einsum("hid,hjd->hij", qr, kr) / np.sqrt(128)
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) < 1e-12


def test_brute_force_mpmath():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    q, k, v, c = _tiny()
    n = 12
    rows = np.arange(0, 64, 64 // n)[:n]
    o, lse = oracle.attention(q, k, v, c, SEC, TH, heads=[1], rows=rows)
    qr = oracle.rope(q[:, 1:2], c, SEC, TH)[:, 0]
    kr = oracle.rope(k[:, 1:2], c, SEC, TH)[:, 0]
    vv = v[:, 1]
    sc = mp.mpf(1) / mp.sqrt(128)
    for ri, i in enumerate(rows):
        s = [mp.fsum(mp.mpf(float(a)) * mp.mpf(float(b)) for a, b in zip(qr[i], kr[j])) * sc for j in range(64)]
        e = [mp.exp(x) for x in s]
        z = mp.fsum(e)
        for d in range(0, 128, 9):
            ref = mp.fsum(e[j] * mp.mpf(float(vv[j, d])) for j in range(64)) / z
            assert abs(float(ref) - o[ri, 0, d]) < 1e-13
        assert abs(float(mp.log(z)) - lse[0, ri]) < 1e-13


def test_permutation_equivariance():
    q, k, v, c = _tiny()
    perm = np.random.default_rng(3).permutation(64)
    o, lse = oracle.attention(q, k, v, c, SEC, TH)
    op, lsep = oracle.attention(q[perm], k[perm], v[perm], c[perm], SEC, TH)
    assert np.max(np.abs(op - o[perm])) < 1e-12
    assert np.max(np.abs(lsep - lse[:, perm])) < 1e-12


def test_closed_forms():
    q, k, v, c = _tiny()
    # all V rows equal -> O equals that row
    vc = np.broadcast_to(v[:1], v.shape).copy()
    o, _ = oracle.attention(q, k, vc, c, SEC, TH)
    assert np.max(np.abs(o - vc)) < 1e-13
    # Q = 0 -> uniform weights, O = mean of V, LSE = log N
    o, lse = oracle.attention(np.zeros_like(q), k, v, c, SEC, TH)
    assert np.max(np.abs(o - v.mean(0, keepdims=True))) < 1e-13
    assert np.max(np.abs(lse - np.log(64))) < 1e-13
    # one row -> O = V
    o, _ = oracle.attention(q[:1], k[:1], v[:1], c[:1], SEC, TH)
    assert np.max(np.abs(o - v[:1])) < 1e-15
    # identical keys at identical coordinates -> O = mean of V
    kc = np.broadcast_to(k[:1], k.shape).copy()
    cc = np.broadcast_to(c[:1], c.shape).copy()
    o, _ = oracle.attention(q, kc, v, cc, SEC, TH)
    assert np.max(np.abs(o - v.mean(0, keepdims=True))) < 1e-13


def test_bidirectional_no_mask():
    q, k, v, c = _tiny()
    o, _ = oracle.attention(q, k, v, c, SEC, TH)
    v2 = v.copy()
    v2[-1] += 1.0                       # last (audio) row
    o2, _ = oracle.attention(q, k, v2, c, SEC, TH)
    assert np.all(np.abs(o2[0] - o[0]) > 0)    # first (text) row sees it


def test_row_and_head_subsets_agree_with_full():
    q, k, v, c = _tiny(q_scale=8.0)
    o, lse = oracle.attention(q, k, v, c, SEC, TH, block=7)
    rows = np.array([63, 0, 17, 40])
    os_, lses = oracle.attention(q, k, v, c, SEC, TH, heads=[1], rows=rows)
    assert np.max(np.abs(os_[:, 0] - o[rows, 1])) < 1e-14
    assert np.max(np.abs(lses[0] - lse[1, rows])) < 1e-13


def test_prerotated_path_equals_fused():
    q, k, v, c = _tiny()
    o, _ = oracle.attention(q, k, v, c, SEC, TH)
    o2, _ = oracle.attention(oracle.rope(q, c, SEC, TH), oracle.rope(k, c, SEC, TH), v, c, SEC, TH,
                             rope_q=False, rope_k=False)
    assert np.max(np.abs(o - o2)) < 1e-14
