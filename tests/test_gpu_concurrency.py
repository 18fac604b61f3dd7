"""Concurrent use of the C ABI from several host threads, each on its own stream (MI355X, gfx950).

The library keeps no state between calls apart from per-device attribute caches held in
atomics, so calls from different threads on different streams must give exactly the
results of the same calls made one after another.  Each thread runs the RoPE pass, the
attention call with its own workspace (two of the four problems split their last wave
into it) and a projection, three times, and every result is compared bit for bit with a
serial run.
"""
import threading

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def make_problem(h3, seed, n_text, frames, heads):
    segs = [W.text(n_text, -n_text), W.video(frames, 6, 8), W.audio(40, 0)]
    n = W.n_tokens(segs)
    q, k, v = W.qkv(n, heads, seed=seed)
    x, w, b = W.projection_inputs(n, 256, 512, seed=seed + 1)
    p = {"n": n, "heads": heads, "coords": torch.from_numpy(h3.build_coords(segs)).cuda(),
         "q": dev_bf16(q), "k": dev_bf16(k), "v": dev_bf16(v), "x": dev_bf16(x), "w": dev_bf16(w),
         "b": dev_bf16(b)}
    p["kr"] = torch.empty_like(p["k"])
    p["table"] = h3.make_rope_table(p["coords"])
    p["o"] = torch.empty_like(p["q"])
    p["lse"] = torch.empty((heads, n), dtype=torch.float32, device="cuda")
    p["y"] = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda")
    need = h3.forward_workspace_bytes(n, heads)
    p["ws_bytes"] = need
    p["ws"] = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
    return p


def run_problem(h3, p, stream):
    cfg = h3.rope_cfg()
    n, heads, stride = p["n"], p["heads"], p["q"].stride(0)
    h3.rope_qk(cfg, p["coords"], None, None, p["k"], p["kr"], n, heads, stride, stream=stream)
    h3.forward_ws(cfg, p["coords"], 1, p["q"], p["kr"], p["v"], p["o"], p["lse"], n, heads, stride, stride, 0.0,
                  p["ws"], p["ws_bytes"], stream=stream)
    h3.linear(p["x"], 256, p["w"], 256, p["b"], p["y"], 512, n, 512, 256, p["table"], 256, stream=stream)


def snapshot(p):
    return [p["o"].view(torch.int16).cpu(), p["lse"].view(torch.int32).cpu(), p["y"].view(torch.int16).cpu()]


def test_threads_on_separate_streams_match_serial(gpu_lib):
    h3 = gpu_lib
    # two problems of 33 heads x 8 query blocks (264 units: the last, partly filled wave is split
    # into the workspace) and two small ones
    problems = [make_problem(h3, 70, 20, 37, 33), make_problem(h3, 71, 33, 38, 33),
                make_problem(h3, 72, 46, 23, 5), make_problem(h3, 73, 59, 30, 5)]
    print("rows", [p["n"] for p in problems], "workspace bytes", [p["ws_bytes"] for p in problems], flush=True)
    assert problems[0]["ws_bytes"] > 0 and problems[1]["ws_bytes"] > 0
    for p in problems:
        run_problem(h3, p, None)
    torch.cuda.synchronize()
    ref = [snapshot(p) for p in problems]
    for p in problems:                      # clear the outputs so that stale values cannot pass
        p["o"].zero_()
        p["lse"].zero_()
        p["y"].zero_()
    torch.cuda.synchronize()

    errors = []
    streams = [torch.cuda.Stream() for _ in problems]

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    assert h3.forward_workspace_bytes(problems[i]["n"], problems[i]["heads"]) == \
                        problems[i]["ws_bytes"]
                    run_problem(h3, problems[i], streams[i])
            streams[i].synchronize()
        except Exception as e:   # reported in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(problems))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, p in enumerate(problems):
        got = snapshot(p)
        for name, a, b in zip(("O", "LSE", "y"), got, ref[i]):
            assert torch.equal(a, b), "problem %d: %s differs from the serial run" % (i, name)
