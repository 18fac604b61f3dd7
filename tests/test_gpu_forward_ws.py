"""GPU parity of h3attn_forward_ws (the key-split last wave) against the fp64 oracle and
against h3attn_forward (MI355X, gfx950).

Units that run over all keys are computed exactly as by h3attn_forward (bit-equal);
split units are merged from key-range partials, which changes only the rounding
order, so they are held to the attention tolerances of the other parity tests
(max |err| <= 2e-2, RMS <= 2e-3, |LSE err| <= tolerances.lse_bound(N), the bound
derived from the bf16 roundings of Q~, K~ and P).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tolerances import lse_bound

pytestmark = pytest.mark.gpu

SEC, TH = W.ROPE_SECTIONS, W.ROPE_THETAS
f64 = oracle.bf16_bits_to_f64


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run(h3, segs, q, k, v, ws_bytes=None):
    n, h, _ = q.shape
    coords = torch.from_numpy(h3.build_coords(segs)).cuda()
    cfg = h3.rope_cfg()
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    kr = torch.empty_like(kd)
    h3.rope_qk(cfg, coords, None, None, kd, kr, n, h, qd.stride(0))
    o = torch.empty_like(qd)
    lse = torch.empty((h, n), dtype=torch.float32, device="cuda")
    if ws_bytes is None:
        h3.forward(cfg, coords, 1, qd, kr, vd, o, lse, n, h, qd.stride(0), o.stride(0))
    else:
        ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda")
        h3.forward_ws(cfg, coords, 1, qd, kr, vd, o, lse, n, h, qd.stride(0), o.stride(0), 0.0, ws, ws_bytes)
    torch.cuda.synchronize()
    return host_bits(o), lse.cpu().numpy()


def check(o_bits, lse, q, k, v, segs, heads, rows, tag):
    c = oracle.build_coords(segs)
    o_ref, lse_ref = oracle.attention(f64(q[:, heads]), f64(k[:, heads]), f64(v[:, heads]), c, SEC, TH, rows=rows)
    err = f64(o_bits[rows][:, heads]) - o_ref
    le = np.abs(lse[heads][:, rows] - lse_ref).max()
    print("%s max|err| %.3e rms %.3e lse %.3e" % (tag, np.abs(err).max(), np.sqrt((err ** 2).mean()), le), flush=True)
    assert np.abs(err).max() <= 2e-2 and np.sqrt((err ** 2).mean()) <= 2e-3 and le <= lse_bound(q.shape[0])


def test_split_tail_small(gpu_lib):
    h3 = gpu_lib
    segs = [W.text(80, -80), W.video(3, 22, 24), W.audio(168, 0)]          # 2,000 rows
    n, heads = W.n_tokens(segs), 33                                         # 8 x 33 = 264 units
    q, k, v = W.qkv(n, heads, seed=5)
    need = h3.forward_workspace_bytes(n, heads)
    print("workspace bytes", need, flush=True)
    assert need > 0                                                         # a last wave of 8 units splits
    o_ws, lse_ws = run(h3, segs, q, k, v, need)
    o_ref, lse_ref = run(h3, segs, q, k, v)
    # the split units are the last ones in head-major order: head 32 here
    assert np.array_equal(o_ws[:, :32], o_ref[:, :32]) and np.array_equal(lse_ws[:32], lse_ref[:32])
    assert not np.array_equal(o_ws[:, 32], o_ref[:, 32])                  # the merged head really is split
    check(o_ws, lse_ws, q, k, v, segs, [32], np.arange(n), "split head")
    check(o_ws, lse_ws, q, k, v, segs, [0], np.arange(0, n, 7), "full head")
    # too small a workspace runs the unsplit schedule: bit-equal to h3attn_forward
    o_small, lse_small = run(h3, segs, q, k, v, need - 16)
    assert np.array_equal(o_small, o_ref) and np.array_equal(lse_small, lse_ref)


def test_workspace_overlapping_a_tensor_is_rejected(gpu_lib):
    h3 = gpu_lib
    segs = [W.text(80, -80), W.video(3, 22, 24), W.audio(168, 0)]
    n, heads = W.n_tokens(segs), 33
    need = h3.forward_workspace_bytes(n, heads)
    coords = torch.from_numpy(h3.build_coords(segs)).cuda()
    q = torch.zeros((n, heads, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(need // 2 + n * heads * 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(h3.H3AttnError) as e:
        h3.forward_ws(h3.rope_cfg(), coords, 1, q, q, q, o, None, n, heads, heads * 128, heads * 128, 0.0, o, need)
    assert e.value.code == h3.H3ATTN_EINVAL
    with pytest.raises(h3.H3AttnError):
        h3.forward_ws(h3.rope_cfg(), coords, 1, q, q, q, o, None, n, heads, heads * 128, heads * 128, 0.0,
                      o.data_ptr() + 8, need)                               # misaligned workspace


def test_split_tail_full_size(gpu_lib):
    """The 5 s workload in the benchmark's launch configuration (split last wave), sampled rows."""
    h3 = gpu_lib
    h, segs = W.CONFIGS["5s"]
    n = W.n_tokens(segs)
    q, k, v = W.qkv(n, h)
    need = h3.forward_workspace_bytes(n, h)
    print("5 s workspace bytes", need, flush=True)
    assert need > 0
    o_ws, lse_ws = run(h3, segs, q, k, v, need)
    rng = np.random.default_rng(2)
    # head 41's last query blocks are the split units; head 0 runs unsplit
    check(o_ws, lse_ws, q, k, v, segs, [41], np.unique(np.r_[n - 1, 20000, rng.integers(14592, n, 40)]), "5s split")
    check(o_ws, lse_ws, q, k, v, segs, [0], np.unique(np.r_[0, rng.integers(0, n, 30)]), "5s full")
    assert np.all(np.isfinite(lse_ws))


@pytest.mark.parametrize("heads", [10, 11])
def test_head_shard_full_length(gpu_lib, heads):
    """One GPU's share of the 42 heads under head sharding (11/11/10/10) at the 5 s length, through
    the benchmark's call; the cost model splits the last wave at both (8 and 5 key ranges)."""
    h3 = gpu_lib
    _, segs = W.CONFIGS["5s"]
    n = W.n_tokens(segs)
    q, k, v = W.qkv(n, heads, seed=40 + heads)
    need = h3.forward_workspace_bytes(n, heads)
    print("%d heads: workspace bytes %d" % (heads, need), flush=True)
    o_ws, lse_ws = run(h3, segs, q, k, v, need)
    rng = np.random.default_rng(heads)
    rows = np.unique(np.r_[0, n - 1, rng.integers(0, n, 24)])
    check(o_ws, lse_ws, q, k, v, segs, [heads - 1], rows, "%d heads, last" % heads)
    check(o_ws, lse_ws, q, k, v, segs, [0], rows, "%d heads, first" % heads)
    assert np.all(np.isfinite(lse_ws))
