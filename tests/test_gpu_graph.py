"""HIP graph capture of the attention step (MI355X, gfx950).

h3attn_forward_noalloc exists for callers that cannot allocate device memory, code under HIP
graph capture among them.  The step (h3attn_rope_qk on K, then h3attn_forward_noalloc with Q
rotated in the kernel; the last head's query blocks split along the keys and merged, so the
partials go through the library's static scratch) is captured once into a graph and replayed.
Between replays the test runs other eager calls on the device, which reuse that scratch, and
synchronises, and it rewrites the buffers the graph reads; every replay must then reproduce bit
for bit the eager step on the inputs present at that moment.  Neither call records a memset, so
nothing in the graph depends on state the eager calls leave behind.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_graph_replays_match_eager_steps(gpu_lib):
    h3 = gpu_lib
    segs = [W.text(80, -80), W.video(3, 22, 24), W.audio(168, 0)]       # 2,000 rows
    n, heads = W.n_tokens(segs), 33
    need = h3.forward_workspace_bytes(n, heads)
    assert 0 < need <= h3.NOALLOC_SCRATCH_BYTES                         # the step uses the scratch
    cfg = h3.rope_cfg()
    coords = torch.from_numpy(h3.build_coords(segs)).cuda()
    inputs = {s: [dev_bf16(t) for t in W.qkv(n, heads, seed=s)] for s in (5, 6)}
    # the graph's buffers: inputs it reads, rotated K, outputs
    q, k, v = (torch.empty_like(inputs[5][0]) for _ in range(3))
    kr = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((heads, n), dtype=torch.float32, device="cuda")
    stride = q.stride(0)

    def step():
        h3.rope_qk(cfg, coords, None, None, k, kr, n, heads, stride)
        h3.forward_noalloc(cfg, coords, 1, q, kr, v, o, lse, n, heads, stride, o.stride(0))

    def load(seed):
        for dst, src in zip((q, k, v), inputs[seed]):
            dst.copy_(src)

    def clear():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        kr.fill_(float("nan"))

    # eager references (the first call also resolves the scratch address on this device)
    ref = {}
    for seed in (5, 6):
        load(seed)
        clear()
        step()
        torch.cuda.synchronize()
        ref[seed] = (o.clone(), lse.clone())
    assert not torch.equal(ref[5][0], ref[6][0])

    # other eager work on the same device that writes the scratch: a different problem
    other_segs = [W.text(500, -500), W.audio(750, 0)]
    on, oh = W.n_tokens(other_segs), 40
    assert h3.forward_workspace_bytes(on, oh) > 0
    ocoords = torch.from_numpy(h3.build_coords(other_segs)).cuda()
    oq, ok_, ov = (dev_bf16(t) for t in W.qkv(on, oh, seed=7))
    oo = torch.empty_like(oq)

    def other_work():
        h3.forward_noalloc(cfg, ocoords, 1, oq, ok_, ov, oo, None, on, oh, oq.stride(0), oo.stride(0))

    load(5)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i, seed in enumerate((5, 6, 5, 6)):
        load(seed)
        clear()
        other_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same_o = torch.equal(o.view(torch.int16), ref[seed][0].view(torch.int16))
        same_l = torch.equal(lse.view(torch.int32), ref[seed][1].view(torch.int32))
        print("replay %d (inputs %d): O bit-equal %s, LSE bit-equal %s" % (i, seed, same_o, same_l), flush=True)
        assert same_o and same_l
