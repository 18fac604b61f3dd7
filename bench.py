"""Benchmark of the MM-RoPE + full-attention hot path on one MI355X.

One step = one pass of the whole path over the 5 s 704x1280 packed sequence
(512 text + 31 x 22 x 40 video + 200 x 2 audio = 28,192 rows, 42 heads x 128):
  h3attn_rope_qk   rotate K by its (t, h, w) coordinates (HBM-bound pass)
  h3attn_forward_ws  rotate Q in the tile load, then softmax(Q~ K~^T / sqrt(128)) V (the
                     last, partly filled wave of workgroups split along the keys, with a
                     caller-owned workspace allocated before the timed region)
Inputs are seeded synthetic bf16 N(0, 1) tensors, resident in HBM before the
timed region.  Prints one JSON line.

FLOP counted per step: 4 N^2 H D (the two products of full attention).

--path adaln times the AdaLN row instead: one h3attn_adaln_residual call (the
gated residual of a sublayer fused with the next modulated layer norm) over
the same 28,192 rows x 5,376 hidden, per-row table entries timestep * 3 + tag;
bytes counted per step: x, y read, x_out, h written (2 B each per element),
the int32 selectors and the three table planes once.

--path pack times one sampler step on the 5 s target clip in one launch
(h3attn_av_euler_pack): the Euler update of the float32 video latent
[24][31][44][80] from its 27,280 bf16 velocity tokens fused with re-packing it
into 1x2x2 tokens, and the same for the stereo audio latent [2][200][32]; bytes
counted per value: 4 + 4 (state) + 2 (velocity) + 2 (token).

--path qkv times the fused QKV projection of the 5 s rows with the rotary
embedding of Q and K in its epilogue (28,192 x 5,376 -> 3 x 42 x 128, bias,
synthetic weights), FLOP 2 M N K; the output projection (5,376 -> 5,376, no
rotation) is timed beside it.

--path block times the attention half of one DiT block over the 5 s rows, five
calls in a row with bf16 between them: AdaLN modulation, the fused QKV
projection with Q/K rotation, attention on the projection's strided Q/K/V
(rope_q = 0, split tail), the output projection, and the gated residual fused
with the next modulated norm.  FLOP counted: 4 N^2 H D + 2 N C 3C + 2 N C C; the
roofline object is the attention call's.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "stream_audio_video_amd", "csrc")
ATTN_SOURCE = os.path.join(CSRC, "attn_fwd.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_fwd_5s_hbm_traffic.json")
ADALN_SOURCE = os.path.join(CSRC, "adaln_kernel.hip")
ADALN_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "adaln_residual_5s_hbm_traffic.json")
GEMM_SOURCE = os.path.join(CSRC, "gemm_kernel.hip")
QKV_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "linear_qkv_5s_hbm_traffic.json")


def kernel_digest(source):
    """sha256 over a kernel's source and the headers it is compiled with, comments and whitespace
    removed (a comment edit does not change the kernel the counters describe)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in (source, os.path.join(CSRC, "launch.hpp"), os.path.join(CSRC, "rope_math.hpp")):
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(record=TRAFFIC_RECORD, source=ATTN_SOURCE, key="attn_fwd_sha256"):
    """HBM bytes per launch from a committed counter record, or None.

    The record holds FETCH_SIZE / WRITE_SIZE per dispatch already scaled by the
    copy-kernel calibration; it is used only while the kernel's sources (its file,
    launch.hpp and rope_math.hpp, comments aside) still have the digest the counters
    were taken with.
    """
    try:
        rec = json.load(open(record))
        digest = kernel_digest(source)
    except (OSError, ValueError):
        return None
    if rec.get(key) != digest:
        return None
    return rec.get("bytes_per_launch")


METRIC = "MM-RoPE+attention TFLOP/s & % bf16 MFMA peak, 28,192-token packed seq"
WORKLOAD = ("5 s 704x1280 packed sequence: 512 text + 31 latent frames x 22x40 video + "
            "200 steps x 2 audio = 28,192 tokens; 42 heads x 128; RoPE t/h/w 32/48/48, base 1e4")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def host_record():
    """The host the oracle ran on: logical CPUs, the ones this process may use, the CPU model and the
    BLAS thread count (numpy's matrix products use that many threads; its elementwise steps one)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "cpus_usable": usable, "cpu_model": model, "blas_threads": blas_threads()}


def cpu_baseline(name, q, k, v, segs, budget_s):
    """Time the fp64 oracle on a bounded sample: head 0, query rows in its default blocks of 1,024
    rows, for about budget_s seconds (the whole head at 5 s on a 16-CPU host)."""
    import oracle
    threads = blas_threads()
    n = q.shape[0]
    c = oracle.build_coords(segs)
    qh = oracle.bf16_bits_to_f64(q[:, :1])
    kh = oracle.bf16_bits_to_f64(k[:, :1])
    vh = oracle.bf16_bits_to_f64(v[:, :1])
    rows_done, t_used = 0, 0.0
    block = 1024
    while t_used < budget_s and rows_done < n:
        rows = np.arange(rows_done, min(n, rows_done + block))
        t0 = time.perf_counter()
        oracle.attention(qh, kh, vh, c, W.ROPE_SECTIONS, W.ROPE_THETAS, rows=rows, block=block)
        t_used += time.perf_counter() - t0
        rows_done += len(rows)
    flops = 4.0 * rows_done * n * W.HEAD_DIM
    rec = {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": "%s workload, head 0 of %d, query rows 0..%d against all %d keys (RoPE included), "
                     "%.1f s of fp64 numpy; FLOP 4*rows*N*D" % (name, q.shape[1], rows_done - 1, n, t_used)}
    rec.update(host_record())
    return rec


ADALN_METRIC = "AdaLN gated residual + modulated layer norm GB/s & % HBM peak, 28,192 rows x 5,376"


def adaln_bytes(n, c, n_entries):
    return 4 * n * c * 2 + 8 * n + 3 * n_entries * c * 2


def adaln_cpu_baseline(x, y, table, t_idx, tags, budget_s):
    """Time the fp64 oracle of the gated residual + modulated norm on rows in blocks of 256, ~budget_s."""
    from oracle import adaln as A
    n, c = x.shape
    tab = A.bf16_bits_to_f64(table)
    idx_all = A.adaln_index(t_idx, tags)
    rows_done, t_used = 0, 0.0
    while t_used < budget_s and rows_done < n:
        r = slice(rows_done, min(n, rows_done + 256))
        xb, yb = A.bf16_bits_to_f64(x[r]), A.bf16_bits_to_f64(y[r])
        t0 = time.perf_counter()
        A.residual_modulate(xb, yb, idx_all[r], tab[:, 2], tab[:, 3], tab[:, 4], A.LAYER_NORM, 1e-6)
        t_used += time.perf_counter() - t0
        rows_done = r.stop
    nbytes = 4 * rows_done * c * 2 + 8 * rows_done
    rec = {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "rows 0..%d of %d (blocks of 256), %.1f s of fp64 numpy; bytes 8*rows*C + 8*rows"
                     % (rows_done - 1, n, t_used)}
    rec.update(host_record())
    return rec


def bench_adaln(args):
    import torch
    import stream_audio_video_amd as h3
    h3.load_library()
    dev = torch.device("cuda:0")
    _, segs = W.CONFIGS[args.config]
    n, c = W.n_tokens(segs), W.ADALN_HIDDEN
    x, y, table = W.adaln_inputs(n, c)
    t_idx, tags = W.adaln_rows(segs)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    xd, yd, tab = to_dev(x), to_dev(y), to_dev(table)
    ti, tg = torch.from_numpy(t_idx).to(dev), torch.from_numpy(tags).to(dev)
    xo, hd = torch.empty_like(xd), torch.empty_like(xd)
    base, ne = tab.data_ptr(), table.shape[0]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        h3.adaln_residual(xd, yd, c, ti, tg, base + 2 * 2 * c, base + 3 * 2 * c, base + 4 * 2 * c, 6 * c, ne,
                          xo, hd, c, n, c, h3.LAYER_NORM, 1e-6)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    nbytes = adaln_bytes(n, c, ne)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    cpu = adaln_cpu_baseline(x, y, table, t_idx, tags, args.cpu_budget) if args.cpu_budget > 0 else None
    rec = {
        "metric": ADALN_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s packed sequence, %d rows x %d hidden, %d table entries (2 timesteps x 3 tags)"
                               % (args.config, n, c, ne),
                   "rows": n, "hidden": c, "norm": "layer", "kernel_ms": round(k_ms, 4),
                   "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(ADALN_TRAFFIC_RECORD, ADALN_SOURCE, "adaln_sha256")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


PACK_METRIC = "Euler step + 1x2x2 re-pack of the 5 s target latents GB/s & % HBM peak (27,280 video + 400 audio tokens)"
PACK_SOURCE = os.path.join(CSRC, "pack_kernel.hip")


def pack_cpu_baseline(video, v_video, audio, v_audio, dt, budget_s):
    """Time the fp64 oracle of the same step, repeated up to ~budget_s."""
    from oracle import pack as Pk
    from oracle import adaln as A
    vv, va = A.bf16_bits_to_f64(v_video), A.bf16_bits_to_f64(v_audio)
    reps, t_used = 0, 0.0
    while t_used < budget_s and reps < 50:
        t0 = time.perf_counter()
        Pk.video_euler_pack(video, vv, dt)
        Pk.audio_euler_pack(audio, va, dt)
        t_used += time.perf_counter() - t0
        reps += 1
    nbytes = 12 * (video.size + audio.size)
    rec = {"value": reps * nbytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "%d full steps of the 5 s clip, %.1f s of fp64 numpy" % (reps, t_used)}
    rec.update(host_record())
    return rec


def bench_pack(args):
    import torch
    import stream_audio_video_amd as h3
    h3.load_library()
    dev = torch.device("cuda:0")
    frames, lh, lw, steps = 31, 44, 80, 200
    c, aw = W.VIDEO_LATENT_CHANNELS, W.AUDIO_LATENT_WIDTH
    video, v_video, audio, v_audio = W.latent_inputs(frames, lh, lw, steps)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    vl, al = torch.from_numpy(video).to(dev), torch.from_numpy(audio).to(dev)
    vv, av = to_dev(v_video), to_dev(v_audio)
    vt = torch.empty((v_video.shape[0], 4 * c), dtype=torch.bfloat16, device=dev)
    at = torch.empty((v_audio.shape[0], aw), dtype=torch.bfloat16, device=dev)
    dt = 1.0 / 49

    def step(ev=None):
        # both target latents of the sampler step in one launch
        if ev is not None:
            ev[0].record()
        h3.av_euler_pack(vl, c, frames, lh, lw, vv, 4 * c, vt, 4 * c, al, 2, steps, aw, av, aw, at, aw, dt)
        if ev is not None:
            ev[1].record()

    def separate(ev):
        ev[0].record()
        h3.video_euler_pack(vl, c, frames, lh, lw, vv, 4 * c, dt, vt, 4 * c)
        ev[1].record()
        h3.audio_euler_pack(al, 2, steps, aw, av, aw, dt, at, aw)
        ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # for comparison, outside the timed steps: the two latents in two launches
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in sev:
        separate(e)
    torch.cuda.synchronize()
    v_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
    a_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
    nbytes = 12 * (video.size + audio.size)
    cpu = pack_cpu_baseline(video, v_video, audio, v_audio, dt, args.cpu_budget) if args.cpu_budget > 0 else None
    rec = {
        "metric": PACK_METRIC, "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "5 s target clip: video latent 24x31x44x80 (27,280 tokens of 96), audio latent "
                               "2x200x32 (400 tokens of 32), dt = 1/49",
                   "kernel_ms": round(k_ms, 4), "bytes_per_step": nbytes,
                   "separate_launches_ms": {"video": round(v_ms, 4), "audio": round(a_ms, 4)}},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (k_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(os.path.join(ROOT, "profiles", "pack_av_5s_hbm_traffic.json"),
                                                 PACK_SOURCE, "pack_sha256")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


QKV_METRIC = "Fused QKV projection + Q/K RoPE epilogue TFLOP/s & % bf16 MFMA peak, 28,192 x 5,376 -> 16,128"


def qkv_cpu_baseline(x, w, b, coords, budget_s):
    """Time the fp64 oracle of the fused projection on blocks of 64 rows, ~budget_s."""
    from oracle.linear import qkv_rope
    from oracle import bf16_bits_to_f64 as f64
    wf, bf = f64(w), f64(b)
    rows_done, t_used = 0, 0.0
    while t_used < budget_s and rows_done < x.shape[0]:
        r = slice(rows_done, min(x.shape[0], rows_done + 64))
        xb = f64(x[r])
        t0 = time.perf_counter()
        qkv_rope(xb, wf, bf, coords[r], 42, W.ROPE_SECTIONS, W.ROPE_THETAS)
        t_used += time.perf_counter() - t0
        rows_done = r.stop
    flop = 2.0 * rows_done * w.shape[0] * w.shape[1]
    rec = {"value": flop / t_used / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": "rows 0..%d of %d (blocks of 64), %.1f s of fp64 numpy; FLOP 2*rows*N*K"
                     % (rows_done - 1, x.shape[0], t_used)}
    rec.update(host_record())
    return rec


def rope_table_timed(h3, cfg, coords):
    """The sequence's rotation table, built once (the coordinates, and so the table, are fixed for all blocks
    and sampler steps of a sequence), with the time of that one launch in ms."""
    import torch
    n = coords.shape[0]
    table = torch.empty((n, 64, 2), dtype=torch.float32, device=coords.device)
    h3.rope_table(cfg, coords, n, table)                     # first launch: code object load
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    h3.rope_table(cfg, coords, n, table)
    ev[1].record()
    torch.cuda.synchronize()
    return table, float(ev[0].elapsed_time(ev[1]))


def bench_qkv(args):
    import torch
    import stream_audio_video_amd as h3
    h3.load_library()
    dev = torch.device("cuda:0")
    h, segs = W.CONFIGS[args.config]
    m, k = W.n_tokens(segs), W.ADALN_HIDDEN
    n = 3 * h * W.HEAD_DIM
    x, w, b = W.projection_inputs(m, k, n)
    _, wo, _ = W.projection_inputs(1, k, k, seed=W.DEFAULT_SEED + 1, with_bias=False)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    xd, wd, bd, wod = to_dev(x), to_dev(w), to_dev(b), to_dev(wo)
    coords_h = h3.build_coords(segs)
    coords = torch.from_numpy(coords_h).to(dev)
    yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    od = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    cfg = h3.rope_cfg(W.ROPE_SECTIONS, W.ROPE_THETAS)
    rope_tab, table_ms = rope_table_timed(h3, cfg, coords)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        h3.linear(xd, k, wd, k, bd, yd, n, m, n, k, rope_tab, 2 * h * W.HEAD_DIM)
        if ev is not None:
            ev[1].record()
        h3.linear(xd, k, wod, k, None, od, k, m, k, k)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    qkv_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    out_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    flop_qkv, flop_out = 2.0 * m * n * k, 2.0 * m * k * k
    achieved = flop_qkv / (qkv_ms * 1e-3) / 1e12
    cpu = qkv_cpu_baseline(x, w, b, coords_h, args.cpu_budget) if args.cpu_budget > 0 else None
    rec = {
        "metric": QKV_METRIC, "value": round((flop_qkv + flop_out) / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "%s rows %d, hidden %d, fused QKV %d outputs with bias and Q/K rotation; output "
                               "projection %d -> %d" % (args.config, m, k, n, k, k),
                   "qkv_ms": round(qkv_ms, 4), "qkv_TFLOPs": round(achieved, 2), "out_proj_ms": round(out_ms, 4),
                   "out_proj_TFLOPs": round(flop_out / (out_ms * 1e-3) / 1e12, 2),
                   "rope_table_ms_once_per_sequence": round(table_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (measured_traffic(QKV_TRAFFIC_RECORD, GEMM_SOURCE, "gemm_sha256")
                                 if args.config == "5s" else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


BLOCK_METRIC = ("Attention half of a DiT block (AdaLN, fused QKV + RoPE, attention, output projection, "
                "gated residual + AdaLN) TFLOP/s, 28,192-token packed seq")


def block_cpu_baseline(config, x, table, t_idx, tags, w_qkv, b_qkv, coords, segs, flops, adaln_b, budget_s):
    """Seconds of the fp64 oracle per block, composed from bounded samples of each stage kind."""
    heads = W.CONFIGS[config][0]
    n = x.shape[0]
    q, k, v = W.qkv(n, heads, W.DEFAULT_SEED)
    att = cpu_baseline(config, q, k, v, segs, budget_s / 3)
    gem = qkv_cpu_baseline(x, w_qkv, b_qkv, coords, budget_s / 3)
    ada = adaln_cpu_baseline(x, x, table, t_idx, tags, budget_s / 3)
    secs = (flops["attention"] / (att["value"] * 1e12) + (flops["qkv"] + flops["out_proj"]) / (gem["value"] * 1e12)
            + adaln_b / (ada["value"] * 1e9))
    rec = {"value": sum(flops.values()) / secs / 1e12, "unit": "TFLOP/s", "cores": max(att["cores"], gem["cores"]),
           "kind": "oracle",
           "sample": "per-stage oracle rates applied to the whole block's FLOP and bytes (AdaLN modulate "
                     "priced at the residual row's byte rate): attention %s; projections %s; AdaLN %s"
                     % (att["sample"], gem["sample"], ada["sample"])}
    rec.update(host_record())
    return rec


def bench_block(args):
    import torch
    import stream_audio_video_amd as h3
    h3.load_library()
    dev = torch.device("cuda:0")
    heads, segs = W.CONFIGS[args.config]
    n = W.n_tokens(segs)
    c = heads * W.HEAD_DIM
    x, _, table = W.adaln_inputs(n, c)
    t_idx, tags = W.adaln_rows(segs)
    _, w_qkv, b_qkv = W.projection_inputs(1, c, 3 * c)
    _, w_o, b_o = W.projection_inputs(1, c, c, W.DEFAULT_SEED + 1)
    coords_h = h3.build_coords(segs)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    xd, tab, wq, bq, wo, bo = to(x), to(table), to(w_qkv), to(b_qkv), to(w_o), to(b_o)
    ti, tg = torch.from_numpy(t_idx).to(dev), torch.from_numpy(tags).to(dev)
    coords = torch.from_numpy(coords_h).to(dev)
    cfg = h3.rope_cfg()
    rope_tab, table_ms = rope_table_timed(h3, cfg, coords)
    base = tab.data_ptr()                    # planes [E][6][C]: shift_a, scale_a, gate_a, shift_m, scale_m, gate_m
    n_e = table.shape[0]
    h1 = torch.empty_like(xd)
    qkv = torch.empty((n, 3, heads, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
    o = torch.empty((n, heads, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((heads, n), dtype=torch.float32, device=dev)
    ws_bytes = h3.forward_workspace_bytes(n, heads)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(xd)
    x_out, h2 = torch.empty_like(xd), torch.empty_like(xd)
    stages = ["adaln_modulate", "qkv_rope", "attention", "out_proj", "adaln_residual"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        h3.adaln_modulate(xd, c, ti, tg, base, base + 2 * c, 6 * c, n_e, h1, c, n, c, h3.LAYER_NORM, 1e-6)
        mark(1)
        h3.linear(h1, c, wq, c, bq, qkv, 3 * c, n, 3 * c, c, rope_tab, 2 * c)
        mark(2)
        h3.forward_ws(cfg, coords, 0, qkv[:, 0], qkv[:, 1], qkv[:, 2], o, lse, n, heads, 3 * c, c, 0.0, ws, ws_bytes)
        mark(3)
        h3.linear(o, c, wo, c, bo, y, c, n, c, c)
        mark(4)
        h3.adaln_residual(xd, y, c, ti, tg, base + 4 * c, base + 6 * c, base + 8 * c, 6 * c, n_e, x_out, h2, c, n,
                          c, h3.LAYER_NORM, 1e-6)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    stage_ms = {s: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, s in enumerate(stages)}
    flops = {"attention": 4.0 * n * n * heads * W.HEAD_DIM, "qkv": 2.0 * n * c * 3 * c, "out_proj": 2.0 * n * c * c}
    total = sum(flops.values())
    value = total / (ms_step * 1e-3) / 1e12
    achieved = flops["attention"] / (stage_ms["attention"] * 1e-3) / 1e12
    mod_b = 2 * n * c * 2 + 8 * n + 2 * n_e * c * 2          # modulate: x read, h written, selectors, 2 planes
    res_b = adaln_bytes(n, c, n_e)
    adaln_b = mod_b + res_b
    cpu = None
    if args.cpu_budget > 0:
        cpu = block_cpu_baseline(args.config, x, table, t_idx, tags, w_qkv, b_qkv, coords_h, segs, flops, adaln_b,
                                 args.cpu_budget)
    rec = {
        "metric": BLOCK_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD if args.config == "5s" else args.config, "n_tokens": n, "heads": heads,
                   "hidden": c, "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
                   "rope_table_ms_once_per_sequence": round(table_ms, 4),
                   "stage_TFLOPs": {"qkv_rope": round(flops["qkv"] / (stage_ms["qkv_rope"] * 1e-3) / 1e12, 2),
                                    "attention": round(achieved, 2),
                                    "out_proj": round(flops["out_proj"] / (stage_ms["out_proj"] * 1e-3) / 1e12, 2)},
                   "stage_GBps": {"adaln_modulate": round(mod_b / (stage_ms["adaln_modulate"] * 1e-3) / 1e9, 1),
                                  "adaln_residual": round(res_b / (stage_ms["adaln_residual"] * 1e-3) / 1e9, 1)},
                   "tokens_per_s": round(n / (ms_step * 1e-3), 1), "workspace_bytes": ws_bytes,
                   "flop_per_step": total},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},   # Q arrives rotated here (rope_q = 0): no counter record for this launch
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="5s", choices=list(W.CONFIGS))
    ap.add_argument("--mode", default="fused", choices=["fused", "prerotated"])
    ap.add_argument("--reuse-refs", action="store_true",
                    help="keep the reference rows' rotated K cached across steps; rotate only text and target rows")
    ap.add_argument("--heads", type=int, default=0,
                    help="attention path: number of heads instead of the workload's 42 (a head shard, e.g. 11)")
    ap.add_argument("--no-split", action="store_true",
                    help="attention without a workspace: the last, partly filled wave is not split along the keys")
    ap.add_argument("--path", default="attention", choices=["attention", "adaln", "pack", "qkv", "block"],
                    help="attention: MM-RoPE + attention (the headline); adaln: the AdaLN residual row")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB three times (scales HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": nbytes, "dispatches": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path is single-GPU (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.path == "adaln":
        bench_adaln(args)
        return
    if args.path == "pack":
        bench_pack(args)
        return
    if args.path == "qkv":
        bench_qkv(args)
        return
    if args.path == "block":
        bench_block(args)
        return

    import torch
    import stream_audio_video_amd as h3
    h3.load_library()
    dev = torch.device("cuda:0")
    h, segs = W.CONFIGS[args.config]
    if args.heads:
        h = args.heads          # one GPU's share of the heads under head (Ulysses) sharding
    n = W.n_tokens(segs)
    D = W.HEAD_DIM
    q, k, v = W.qkv(n, h, W.DEFAULT_SEED)
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    coords = torch.from_numpy(h3.build_coords(segs)).to(dev)
    cfg = h3.rope_cfg(W.ROPE_SECTIONS, W.ROPE_THETAS)
    stride = qd.stride(0)
    krot = torch.empty_like(kd)
    qrot = torch.empty_like(qd) if args.mode == "prerotated" else None
    o = torch.empty_like(qd)
    lse = torch.empty((h, n), dtype=torch.float32, device=dev)
    ws_bytes = 0 if args.no_split else h3.forward_workspace_bytes(n, h)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev)
    fused = args.mode == "fused"
    # row ranges rotated each step: all rows, or (reusing cached references) text and target rows only
    ranges = [(0, n)]
    if args.reuse_refs:
        ranges, r = [], 0
        for sg in segs:
            m = sg.frames * sg.grid_h * sg.grid_w
            if sg.kind == W.TEXT or sg.t0_thirds >= 0:
                if ranges and ranges[-1][1] == r:
                    ranges[-1] = (ranges[-1][0], r + m)
                else:
                    ranges.append((r, r + m))
            r += m
        h3.rope_qk(cfg, coords, None, None, kd, krot, n, h, stride)   # the cache: every row once, untimed
    esz = 2

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if fused:
            for a, b in ranges:
                h3.rope_qk(cfg, coords.data_ptr() + 12 * a, None, None, kd.data_ptr() + a * stride * esz,
                           krot.data_ptr() + a * stride * esz, b - a, h, stride)
        else:
            h3.rope_qk(cfg, coords, qd, qrot, kd, krot, n, h, stride)
        if ev is not None:
            ev[1].record()
        h3.forward_ws(cfg, coords, 1 if fused else 0, qd if fused else qrot, krot, vd, o, lse, n, h, stride,
                      stride, 0.0, ws, ws_bytes)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    rope_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    flop = 4.0 * n * n * h * D
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (attn_ms * 1e-3) / 1e12
    rope_rows = sum(b - a for a, b in ranges) if fused else n
    rope_bytes = (2 if fused else 4) * rope_rows * h * D * 2 + 12 * rope_rows

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(args.config, q, k, v, segs, args.cpu_budget)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (WORKLOAD if args.config == "5s" and not args.heads else
                                "%s, %d heads (one GPU's head share)" % (args.config, h) if args.heads else args.config),
                   "n_tokens": n, "heads": h,
                   "head_dim": D, "rope_sections": list(W.ROPE_SECTIONS), "mode": args.mode,
                   "frac_of_peak_step": round(value / PEAK_BF16_TFLOPS, 4),
                   "tokens_per_s": round(n / (ms_step * 1e-3), 1),
                   "rope_ms": round(rope_ms, 4), "rope_GBps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
                   "attn_ms": round(attn_ms, 4), "rope_rows": rope_rows,
                   "reuse_refs": bool(args.reuse_refs), "workspace_bytes": ws_bytes},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     # the counter record covers the default launch only: 5 s, 42 heads, Q rotated in the kernel
                     "traffic": (measured_traffic() if args.config == "5s" and not args.heads and not args.no_split
                                 and fused else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
