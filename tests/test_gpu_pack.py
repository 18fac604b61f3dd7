"""GPU parity of the packing / Euler entry points against the fp64 oracle (MI355X, gfx950).

Tolerances.  Packing without an update is a rearrangement plus one bf16 rounding
of float32 values: bit-exact.  With an update, the kernel forms x + dt * v with
one float32 fused multiply-add (correctly rounded); the oracle forms it in
float64 (within 2^-53 relative) and rounds to float32, so the two may differ by
one float32 ulp where the float64 value sits within 2^-53 of a float32 halfway
point.  Test: every element within one float32 ulp, at most 1e-5 of them not
bit-equal; tokens bit-equal wherever the state is.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import pack as P
from oracle import adaln as A

pytestmark = pytest.mark.gpu


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_of_f32(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def check_state(got, want, tag=""):
    diff = got.view(np.uint32) != want.view(np.uint32)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    print("%s state: %d of %d not bit-equal" % (tag, int(diff.sum()), diff.size), flush=True)
    assert np.all(np.abs(got.astype(np.float64) - want.astype(np.float64)) <= ulp)
    assert diff.sum() <= max(2, 1e-5 * diff.size)
    return diff


def run_video(h3, lat, v_bits, dt, want_tokens=True, v_stride=None, t_stride=None):
    c, f, hh, ww = lat.shape
    rows = f * (hh // 2) * (ww // 2)
    width = 4 * c
    ld = torch.from_numpy(lat.copy()).cuda()
    vs, ts = v_stride or width, t_stride or width
    vd = None
    if v_bits is not None:
        vd = torch.zeros((rows, vs), dtype=torch.bfloat16, device="cuda")
        vd[:, :width] = dev_bf16(v_bits)
    td = torch.full((rows, ts), 5.0, dtype=torch.bfloat16, device="cuda") if want_tokens else None
    h3.video_euler_pack(ld, c, f, hh, ww, vd, vs, dt, td, ts)
    torch.cuda.synchronize()
    return ld.cpu().numpy(), (host_bits(td) if want_tokens else None)


@pytest.mark.parametrize("shape", [(24, 31, 44, 80), (24, 1, 44, 80), (3, 2, 6, 10), (1, 1, 2, 2), (24, 3, 90, 160)])
def test_video_pack_only_is_exact(gpu_lib, shape):
    lat = np.random.default_rng(sum(shape)).standard_normal(shape).astype(np.float32)
    new, tok = run_video(gpu_lib, lat, None, 0.0)
    assert np.array_equal(new, lat)                          # no update without velocities
    want = bf16_of_f32(P.patchify_video(lat))
    assert np.array_equal(tok, want)


@pytest.mark.parametrize("dt", [0.0204, -0.5, 1.0])
def test_video_euler_step(gpu_lib, dt):
    lat, v, _, _ = W.latent_inputs(31, 44, 80, 200)
    new, tok = run_video(gpu_lib, lat, v, dt)
    want_state, want_tok = P.video_euler_pack(lat, A.bf16_bits_to_f64(v), dt)
    diff = check_state(new, want_state, "video dt=%g" % dt)
    same_tok = P.patchify_video(~diff)                       # token values whose state matched bit for bit
    assert np.array_equal(tok[same_tok], bf16_of_f32(want_tok)[same_tok])


def test_video_strides_and_update_without_tokens(gpu_lib):
    lat = np.random.default_rng(4).standard_normal((5, 3, 8, 12)).astype(np.float32)
    v = W.normal_bf16((3 * 4 * 6, 20), 5)
    new, tok = run_video(gpu_lib, lat, v, 0.25, v_stride=24, t_stride=28)
    want_state, want_tok = P.video_euler_pack(lat, A.bf16_bits_to_f64(v), 0.25)
    diff = check_state(new, want_state, "strided")
    assert not diff.any()
    assert np.array_equal(tok[:, :20], bf16_of_f32(want_tok))
    assert np.all(tok[:, 20:] == host_bits(torch.full((1,), 5.0, dtype=torch.bfloat16))[0])   # padding untouched
    new2, _ = run_video(gpu_lib, lat, v, 0.25, want_tokens=False, v_stride=24)
    assert np.array_equal(new2, new)


def test_video_exact_velocity_reaches_clean_latent(gpu_lib):
    # the straight path: from pure noise (t = 0) along v = x0 - noise, steps summing to 1 land on x0
    c, f, hh, ww = 24, 2, 44, 80
    rng = np.random.default_rng(6)
    x0 = A.bf16_bits_to_f64(W.normal_bf16((c, f, hh, ww), 7)).astype(np.float32)
    noise = np.zeros_like(x0)                                # noise 0 keeps x0 - noise exact in bf16
    v = bf16_of_f32(P.patchify_video(x0 - noise))
    ld = torch.from_numpy(noise.copy()).cuda()
    vd = dev_bf16(v)
    for dt in (0.25, 0.25, 0.5):                             # exact binary fractions: every sum is exact
        gpu_lib.video_euler_pack(ld, c, f, hh, ww, vd, 4 * c, dt, None, 4 * c)
    torch.cuda.synchronize()
    assert np.array_equal(ld.cpu().numpy(), x0)


@pytest.mark.parametrize("steps,dt", [(200, 0.0204), (600, -0.125), (1, 1.0), (7, 0.0)])
def test_audio_euler_pack(gpu_lib, steps, dt):
    _, _, lat, v = W.latent_inputs(1, 2, 2, steps)
    ld = torch.from_numpy(lat.copy()).cuda()
    vd = dev_bf16(v)
    td = torch.empty((steps * 2, 32), dtype=torch.bfloat16, device="cuda")
    gpu_lib.audio_euler_pack(ld, 2, steps, 32, vd, 32, dt, td, 32)
    torch.cuda.synchronize()
    want_state, want_tok = P.audio_euler_pack(lat, A.bf16_bits_to_f64(v), dt)
    diff = check_state(ld.cpu().numpy(), want_state, "audio")
    same = P.pack_audio(~diff)
    assert np.array_equal(host_bits(td)[same], bf16_of_f32(want_tok)[same])
    # packing alone is exact
    ld2 = torch.from_numpy(lat.copy()).cuda()
    gpu_lib.audio_euler_pack(ld2, 2, steps, 32, None, 32, 0.0, td, 32)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(td), bf16_of_f32(P.pack_audio(lat)))
    assert np.array_equal(ld2.cpu().numpy(), lat)


@pytest.mark.parametrize("with_v", [True, False])
def test_av_pack_equals_separate_calls(gpu_lib, with_v):
    """Video and audio latents of one sampler step in one launch: bit-equal to the two calls."""
    h3 = gpu_lib
    frames, lh, lw, steps = 31, 44, 80, 200
    c, aw = W.VIDEO_LATENT_CHANNELS, W.AUDIO_LATENT_WIDTH
    video, v_video, audio, v_audio = W.latent_inputs(frames, lh, lw, steps)
    dt = 1.0 / 49
    outs = []
    for combined in (True, False):
        vl, al = torch.from_numpy(video.copy()).cuda(), torch.from_numpy(audio.copy()).cuda()
        vv = dev_bf16(v_video) if with_v else None
        av = dev_bf16(v_audio) if with_v else None
        vt = torch.full((v_video.shape[0], 4 * c), 5.0, dtype=torch.bfloat16, device="cuda")
        at = torch.full((v_audio.shape[0], aw), 5.0, dtype=torch.bfloat16, device="cuda")
        if combined:
            h3.av_euler_pack(vl, c, frames, lh, lw, vv, 4 * c, vt, 4 * c, al, 2, steps, aw, av, aw, at, aw, dt)
        else:
            h3.video_euler_pack(vl, c, frames, lh, lw, vv, 4 * c, dt, vt, 4 * c)
            h3.audio_euler_pack(al, 2, steps, aw, av, aw, dt, at, aw)
        torch.cuda.synchronize()
        outs.append((vl.cpu().numpy(), al.cpu().numpy(), host_bits(vt), host_bits(at)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    # and against the oracle: the updated latents and their tokens
    if with_v:
        want_v, _ = P.video_euler_pack(video, A.bf16_bits_to_f64(v_video), dt)
        want_a, _ = P.audio_euler_pack(audio, A.bf16_bits_to_f64(v_audio), dt)
        check_state(outs[0][0], want_v, "av video")
        check_state(outs[0][1], want_a, "av audio")
    else:
        assert np.array_equal(outs[0][2], bf16_of_f32(P.patchify_video(video)))
        assert np.array_equal(outs[0][3], bf16_of_f32(P.pack_audio(audio)))


def test_av_pack_with_one_part_empty(gpu_lib):
    """Zero audio steps: the combined call does the video part alone."""
    h3 = gpu_lib
    video = np.random.default_rng(3).standard_normal((3, 2, 6, 10)).astype(np.float32)
    vl = torch.from_numpy(video.copy()).cuda()
    al = torch.zeros(16, dtype=torch.float32, device="cuda")
    vt = torch.zeros((2 * 3 * 5, 12), dtype=torch.bfloat16, device="cuda")
    at = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    h3.av_euler_pack(vl, 3, 2, 6, 10, None, 12, vt, 12, al, 2, 0, 32, None, 32, at, 32, 0.1)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(vt), bf16_of_f32(P.patchify_video(video)))
    assert torch.all(at == 0)
