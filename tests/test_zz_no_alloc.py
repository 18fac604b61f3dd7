"""GPU test of h3attn_forward_noalloc, the attention call that allocates nothing (MI355X, gfx950).

It runs the schedule and kernels of h3attn_forward_ws with the key-split partials in the
library's static device scratch instead of a caller workspace, so its output must equal
h3attn_forward_ws's bit for bit; the split rows are also held to the oracle tolerances.
Two calls in a row, the second on a smaller input whose partials cover less of the
scratch than the first call left there.
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


def both_calls(h3, segs, q, k, v):
    """(noalloc output, forward_ws output) for one problem, Q rotated in the kernel."""
    n, h, _ = q.shape
    coords = torch.from_numpy(h3.build_coords(segs)).cuda()
    cfg = h3.rope_cfg()
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    kr = torch.empty_like(kd)
    h3.rope_qk(cfg, coords, None, None, kd, kr, n, h, qd.stride(0))
    outs = []
    for use_ws in (False, True):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((h, n), float("nan"), dtype=torch.float32, device="cuda")
        if use_ws:
            need = h3.forward_workspace_bytes(n, h)
            ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
            h3.forward_ws(cfg, coords, 1, qd, kr, vd, o, lse, n, h, qd.stride(0), o.stride(0), 0.0, ws, need)
        else:
            h3.forward_noalloc(cfg, coords, 1, qd, kr, vd, o, lse, n, h, qd.stride(0), o.stride(0))
        torch.cuda.synchronize()
        outs.append((host_bits(o), lse.cpu().numpy()))
    return outs


def test_noalloc_two_calls_equal_forward_ws(gpu_lib):
    h3 = gpu_lib
    h5, segs5 = W.CONFIGS["5s"]
    small = [W.text(80, -80), W.video(3, 22, 24), W.audio(168, 0)]      # 2,000 rows; x 33 heads
    cases = [("5s", segs5, h5, W.DEFAULT_SEED, h5 - 1), ("2000x33", small, 33, 5, 32)]
    sizes = []
    for tag, segs, heads, seed, split_head in cases:
        n = W.n_tokens(segs)
        need = h3.forward_workspace_bytes(n, heads)
        print("%s: n=%d heads=%d partials %d bytes" % (tag, n, heads, need), flush=True)
        assert 0 < need <= h3.NOALLOC_SCRATCH_BYTES              # the call really uses the scratch
        sizes.append(need)
        q, k, v = W.qkv(n, heads, seed=seed)
        (o_na, l_na), (o_ws, l_ws) = both_calls(h3, segs, q, k, v)
        assert np.array_equal(o_na, o_ws) and np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32)), tag
        # the split head against the oracle (rows of its split query blocks, plus the first rows)
        rows = np.unique(np.r_[np.arange(0, n, max(1, n // 64)), np.arange(max(0, n - 512), n)])
        c = oracle.build_coords(segs)
        o_ref, lse_ref = oracle.attention(f64(q[:, [split_head]]), f64(k[:, [split_head]]),
                                          f64(v[:, [split_head]]), c, SEC, TH, rows=rows)
        err = f64(o_na[rows][:, [split_head]]) - o_ref
        le = float(np.abs(l_na[[split_head]][:, rows] - lse_ref).max())
        mx, rms = float(np.abs(err).max()), float(np.sqrt((err ** 2).mean()))
        print("%s head %d: max|err| %.3e rms %.3e lse %.3e" % (tag, split_head, mx, rms, le), flush=True)
        assert mx <= 2e-2 and rms <= 2e-3 and le <= lse_bound(n)
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_shapes_beyond_the_scratch(gpu_lib):
    """The 5 s rows with 11 heads need 125 MiB of partials: refused before anything runs."""
    h3 = gpu_lib
    _, segs = W.CONFIGS["5s"]
    n, heads = W.n_tokens(segs), 11
    assert h3.forward_workspace_bytes(n, heads) > h3.NOALLOC_SCRATCH_BYTES
    coords = torch.from_numpy(h3.build_coords(segs)).cuda()
    x = torch.zeros((n, heads, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(x, 3.0)
    with pytest.raises(h3.H3AttnError) as e:
        h3.forward_noalloc(h3.rope_cfg(), coords, 1, x, x, x, o, None, n, heads, heads * 128, heads * 128)
    assert e.value.code == h3.H3ATTN_ESCRATCH
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
