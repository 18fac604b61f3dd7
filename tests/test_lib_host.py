"""Host-side checks of libh3attn: it loads, exports every declared symbol, its
coordinate builder is bit-exact against the oracle, and its argument checks
reject bad calls before touching a device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def h3():
    import stream_audio_video_amd as h3
    h3.load_library()
    return h3


def _declared():
    src = open(os.path.join(ROOT, "include", "h3attn.h")).read()
    return sorted(set(re.findall(r"\b(h3attn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(h3):
    decl = _declared()
    assert set(decl) == set(h3.EXPORTED)
    lib = h3.load_library()
    for name in decl:
        assert hasattr(lib, name)
    out = subprocess.run(["nm", "-D", "--defined-only", h3._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (h3attn_\w+)", out))
    assert set(decl) <= exported
    assert "gfx950" in h3.version()


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_coords_bit_exact_vs_oracle(h3, name):
    _, segs = W.CONFIGS[name]
    a = h3.build_coords(segs)
    b = oracle.build_coords(segs)
    assert a.shape == b.shape == (W.CONFIG_TOKENS[name], 3)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_coords_fuzz_bit_exact(h3):
    rng = np.random.default_rng(1234)
    for trial in range(1000):
        segs = []
        for _ in range(rng.integers(0, 6)):
            kind = int(rng.integers(0, 3))
            frames = int(rng.integers(0, 7))
            if kind == W.TEXT:
                gh, gw = 1, 1
            elif kind == W.AUDIO:
                gh, gw = 1, int(rng.integers(1, 4))
            else:
                gh, gw = int(rng.integers(1, 50)), int(rng.integers(1, 90))
            t0 = int(rng.integers(-(2 ** 22), 2 ** 22))
            dt = int(rng.integers(-40, 41))
            segs.append(W.Segment(kind, frames, gh, gw, t0, dt))
        a = h3.build_coords(segs)
        b = oracle.build_coords(segs)
        assert a.shape == b.shape
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (trial, segs)


def test_coords_count_only_and_capacity(h3):
    lib = h3.load_library()
    _, segs = W.CONFIGS["tiny"]
    arr = h3._segments(segs)
    n = ctypes.c_int64(-1)
    assert lib.h3attn_build_coords(arr, len(segs), None, 0, ctypes.byref(n)) == 0 and n.value == 64
    buf = np.full((63, 3), 7.0, np.float32)
    rc = lib.h3attn_build_coords(arr, len(segs), buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 63,
                                 ctypes.byref(n))
    assert rc == h3.H3ATTN_ERANGE and n.value == 64
    assert np.all(buf == 7.0)          # nothing written on error
    assert lib.h3attn_build_coords(arr, len(segs), None, 0, None) == h3.H3ATTN_EINVAL
    assert lib.h3attn_build_coords(None, 1, None, 0, ctypes.byref(n)) == h3.H3ATTN_EINVAL
    assert h3.build_coords([]).shape == (0, 3)


@pytest.mark.parametrize("seg,code", [
    (W.Segment(3, 1, 1, 1, 0, 3), -1),            # unknown kind
    (W.Segment(W.TEXT, 4, 2, 1, 0, 3), -1),       # text with a grid
    (W.Segment(W.AUDIO, 4, 2, 2, 0, 3), -1),      # audio with grid_h
    (W.Segment(W.VIDEO, -1, 2, 2, 0, 20), -1),    # negative frames
    (W.Segment(W.VIDEO, 1, 0, 2, 0, 20), -1),     # empty grid
    (W.Segment(W.TEXT, 2, 1, 1, 2 ** 24, 3), -2),            # t not exact in binary32
    (W.Segment(W.TEXT, 3, 1, 1, 2 ** 24 - 4, 3), -2),        # last t out of range
])
def test_coords_rejects(h3, seg, code):
    with pytest.raises(h3.H3AttnError) as e:
        h3.build_coords([seg])
    assert e.value.code == code


def _cfg(h3, **kw):
    c = h3.rope_cfg()
    for k, v in kw.items():
        if k == "sec":
            c.sec = (ctypes.c_int32 * 3)(*v)
        elif k == "theta":
            c.theta = (ctypes.c_double * 3)(*v)
        else:
            setattr(c, k, v)
    return c


BAD_CFGS = [dict(head_dim=64), dict(sec=(32, 48, 40)), dict(sec=(31, 49, 48)), dict(sec=(-2, 82, 48)),
            dict(theta=(1e4, 0.0, 1e4)), dict(theta=(1e4, float("nan"), 1e4))]


@pytest.mark.parametrize("kw", BAD_CFGS)
def test_abi_rejects_bad_cfg(h3, kw):
    lib = h3.load_library()
    cfg = _cfg(h3, **kw)
    p = 1 << 20
    assert lib.h3attn_rope_qk(ctypes.byref(cfg), p, p, p, None, None, 64, 2, 256, None) == h3.H3ATTN_EINVAL
    assert lib.h3attn_forward(ctypes.byref(cfg), p, 1, p, p, p, p * 4, None, 64, 2, 256, 256, 0.0,
                              None) == h3.H3ATTN_EINVAL


def test_abi_rejects_bad_geometry(h3):
    lib = h3.load_library()
    cfg = h3.rope_cfg()
    P = 1 << 20
    rq = lambda *a: lib.h3attn_rope_qk(ctypes.byref(cfg), *a)
    fw = lambda *a: lib.h3attn_forward(ctypes.byref(cfg), *a)
    E, R = h3.H3ATTN_EINVAL, h3.H3ATTN_ERANGE
    assert rq(P, None, None, None, None, 64, 2, 256, None) == E              # nothing to rotate
    assert rq(P, P, None, None, None, 64, 2, 256, None) == E                 # q_in without q_out
    assert rq(P, P + 2, P + 2, None, None, 64, 2, 256, None) == E            # misaligned
    assert rq(P, P, P, None, None, 64, 2, 200, None) == E                    # stride < H*D
    assert rq(P, P, P, None, None, 64, 2, 260, None) == E                    # stride not a multiple of 8
    assert rq(P, P, P, None, None, -1, 2, 256, None) == E                    # negative rows
    assert rq(P, P, P, None, None, 64, 0, 256, None) == E                    # no heads
    assert rq(None, P, P, None, None, 64, 2, 256, None) == E                 # coords missing
    assert rq(P, P, P, None, None, 2 ** 22, 42, 5376, None) == R             # offsets overflow 32 bits
    assert rq(P, P, P, None, None, 0, 2, 256, None) == 0                     # empty: no-op
    Q, K, V, O = P, 2 * P, 3 * P, 4 * P
    assert fw(P, 1, None, K, V, O, None, 64, 2, 256, 256, 0.0, None) == E    # null q
    assert fw(P, 1, Q, K, V, None, None, 64, 2, 256, 256, 0.0, None) == E    # null o
    assert fw(P, 1, Q, K, V, O + 8, None, 64, 2, 256, 256, 0.0, None) == E   # misaligned o
    assert fw(P, 1, Q, K, V, O, P + 2, 64, 2, 256, 256, 0.0, None) == E      # misaligned lse
    assert fw(P, 1, Q, K, V, Q, None, 64, 2, 256, 256, 0.0, None) == E       # o aliases q
    assert fw(P, 1, Q, K, V, V + 1024, None, 64, 2, 256, 256, 0.0, None) == E  # o overlaps v
    assert fw(None, 1, Q, K, V, O, None, 64, 2, 256, 256, 0.0, None) == E    # rope_q without coords
    assert fw(P, 1, Q, K, V, O, None, 64, 2, 256, 128, 0.0, None) == E       # o stride too small
    assert fw(P, 1, Q, K, V, O, None, 64, 2, 256, 256, float("inf"), None) == E
    assert fw(P, 1, Q, K, V, O, None, 2 ** 22, 42, 5376, 5376, 0.0, None) == R
    assert fw(P, 1, Q, K, V, O, None, 0, 2, 256, 256, 0.0, None) == 0        # empty: no-op


def test_rope_rejects_partial_aliasing(h3):
    """An output of h3attn_rope_qk may equal its own input (in place) and share no byte with any other
    tensor.  Every case below fails in the argument checks, before any device call."""
    lib = h3.load_library()
    cfg = h3.rope_cfg()
    P = 1 << 24
    QI, QO, KI, KO, C = P, 2 * P, 3 * P, 4 * P, 8 * P
    E = h3.H3ATTN_EINVAL
    rq = lambda qi, qo, ki, ko, stride=256, c=C: lib.h3attn_rope_qk(ctypes.byref(cfg), c, qi, qo, ki, ko, 64, 2,
                                                                      stride, None)
    assert rq(QI, QO, KI, QO) == E                   # both outputs in one place
    assert rq(QI, QO, KI, QO + 512) == E             # k_out one row behind q_out
    assert rq(QI, QO, KI, KI + 16) == E              # k_out overlaps its own input without being it
    assert rq(QI, KI, KI, KO) == E                   # q_out is the other input
    assert rq(QI, QI + 512, None, None) == E         # q_out shifted by a row from q_in
    assert rq(QI, QO, KI, QI) == E                   # k_out is q_in
    assert rq(QI, C, None, None) == E                # an output over the coordinates
    assert rq(QI, QO, None, None, c=QO + 1024) == E
    # [N][3][H][128] views (row pitch 1,536 B): Q slot at +0, K slot at +512 B; a K output half a slot
    # into the Q output's bytes overlaps it
    assert rq(QI, QO, QI + 512, QO + 256, stride=768) == E


def test_rope_accepts_interleaved_views(h3):
    """In place and interleaved slots of one fused buffer pass the checks; without a GPU the call then
    stops at the device check (these addresses are never dereferenced on the host)."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present: the accepted calls would launch (covered by the GPU tests)")
    lib = h3.load_library()
    cfg = h3.rope_cfg()
    P = 1 << 24
    rq = lambda qi, qo, ki, ko, stride: lib.h3attn_rope_qk(ctypes.byref(cfg), 8 * P, qi, qo, ki, ko, 64, 2, stride,
                                                           None)
    for rc in (rq(P, P, 3 * P, 3 * P, 256), rq(P, 2 * P, P + 512, 2 * P + 512, 768), rq(P, P, P + 512, P + 512, 768)):
        assert rc in (h3.H3ATTN_EUNSUPPORTED, h3.H3ATTN_EHIP)


def test_noalloc_rejects_bad_calls(h3):
    """h3attn_forward_noalloc runs the argument checks of h3attn_forward before anything else."""
    lib = h3.load_library()
    cfg = h3.rope_cfg()
    P = 1 << 20
    Q, K, V, O = P, 2 * P, 3 * P, 4 * P
    na = lambda *a: lib.h3attn_forward_noalloc(ctypes.byref(cfg), *a)
    E = h3.H3ATTN_EINVAL
    assert na(P, 1, None, K, V, O, None, 64, 2, 256, 256, 0.0, None) == E      # null q
    assert na(P, 1, Q, K, V, Q, None, 64, 2, 256, 256, 0.0, None) == E         # o aliases q
    assert na(None, 1, Q, K, V, O, None, 64, 2, 256, 256, 0.0, None) == E      # rope_q without coords
    assert na(P, 1, Q, K, V, O + 8, None, 64, 2, 256, 256, 0.0, None) == E     # misaligned o
    assert na(P, 1, Q, K, V, O, None, 2 ** 22, 42, 5376, 5376, 0.0, None) == h3.H3ATTN_ERANGE
    assert na(P, 1, Q, K, V, O, None, 0, 2, 256, 256, 0.0, None) == 0          # empty: no-op
    assert "scratch" in h3.strerror(h3.H3ATTN_ESCRATCH)


def test_strerror(h3):
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(h3.strerror(code), str) and h3.strerror(code)


def test_abi_rejects_bad_adaln_calls(h3):
    lib = h3.load_library()
    P = 1 << 24
    X, Y, XO, H, TI, TG, TAB = P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P
    C = 5376
    E, R = h3.H3ATTN_EINVAL, h3.H3ATTN_ERANGE

    def mod(x=X, xs=C, ti=TI, tg=TG, sh=TAB, sc=TAB + 2 * C, es=6 * C, ne=6, h=H, hs=C, n=64, c=C, kind=0,
            eps=1e-6):
        return lib.h3attn_adaln_modulate(x, xs, ti, tg, sh, sc, es, ne, h, hs, n, c, kind, eps, None)

    def res(x=X, y=Y, s=C, ti=TI, tg=TG, g=TAB + 4 * C, sh=TAB, sc=TAB + 2 * C, es=6 * C, ne=6, xo=XO, h=H,
            os_=C, n=64, c=C, kind=0, eps=1e-6):
        return lib.h3attn_adaln_residual(x, y, s, ti, tg, g, sh, sc, es, ne, xo, h, os_, n, c, kind, eps, None)

    assert mod(n=0) == 0 and res(n=0) == 0                 # empty: no-op
    assert mod(c=0) == E and mod(c=12) == E and mod(c=8200) == E
    assert mod(xs=C - 8) == E and mod(hs=C + 4) == E
    assert mod(kind=2) == E and mod(eps=-1.0) == E and mod(eps=float("nan")) == E
    assert mod(ne=0) == E and mod(es=-8) == E and mod(es=6 * C + 4) == E
    assert mod(x=None) == E and mod(ti=None) == E and mod(tg=None) == E and mod(sh=None) == E
    assert mod(x=X + 8) == E and mod(h=H + 2) == E and mod(ti=TI + 2) == E
    assert mod(n=-1) == E and mod(n=2 ** 31) == R
    assert mod(h=X + 1024) == E                            # h overlaps x without being x
    assert res(y=None) == E and res(g=None) == E and res(xo=None) == E
    assert res(y=Y + 8) == E and res(xo=XO + 8) == E
    assert res(h=X) == E and res(h=Y) == E and res(h=XO) == E     # h overlaps an input or x_out
    assert res(xo=Y) == E                                  # x_out overlaps y
    assert res(xo=X + 1024) == E                           # x_out overlaps x without being x
    assert res(xo=X, os_=2 * C) == E                       # in place needs one stride


def test_abi_rejects_bad_pack_calls(h3):
    lib = h3.load_library()
    P = 1 << 24
    L, V, T = P, 4 * P, 8 * P
    E, R = h3.H3ATTN_EINVAL, h3.H3ATTN_ERANGE

    def vid(lat=L, c=24, f=31, h=44, w=80, v=V, vs=96, dt=0.1, t=T, ts=96):
        return lib.h3attn_video_euler_pack(lat, c, f, h, w, v, vs, dt, t, ts, None)

    def aud(lat=L, ch=2, s=200, w=32, v=V, vs=32, dt=0.1, t=T, ts=32):
        return lib.h3attn_audio_euler_pack(lat, ch, s, w, v, vs, dt, t, ts, None)

    assert vid(f=0) == 0 and aud(s=0) == 0                  # empty: no-op
    assert vid(v=None, t=None) == E and aud(v=None, t=None) == E
    assert vid(lat=None) == E and vid(lat=L + 4) == E and vid(v=V + 2) == E and vid(t=T + 2) == E
    assert vid(c=0) == E and vid(f=-1) == E and vid(h=43) == E and vid(w=81) == E and vid(h=0) == E
    assert vid(vs=94) == E and vid(ts=97) == E and vid(dt=float("inf")) == E
    assert vid(c=24, w=344) == R                             # two latent rows of every channel exceed LDS
    assert vid(c=4, f=2 ** 20, h=32, w=32) == R              # more than 2^31 latent values
    assert vid(t=L + 4096) == E and vid(v=L) == E and vid(t=V + 64) == E   # overlaps
    assert aud(ch=0) == E and aud(s=-1) == E and aud(w=31) == E and aud(w=0) == E
    assert aud(vs=30) == E and aud(ts=33) == E and aud(v=L) == E and aud(t=L) == E


def test_abi_rejects_bad_av_pack_calls(h3):
    """h3attn_av_euler_pack checks each part as the single calls do, and the parts against each other."""
    lib = h3.load_library()
    P = 1 << 24
    VL, VV, VT, AL, AV, AT = P, 4 * P, 8 * P, 12 * P, 13 * P, 14 * P
    E = h3.H3ATTN_EINVAL

    def av(vl=VL, c=24, f=31, h=44, w=80, vv=VV, vs=96, vt=VT, ts=96, al=AL, ch=2, s=200, aw=32, a_v=AV, avs=32,
           at=AT, ats=32, dt=0.1):
        return lib.h3attn_av_euler_pack(vl, c, f, h, w, vv, vs, vt, ts, al, ch, s, aw, a_v, avs, at, ats, dt, None)

    assert av(f=0, s=0) == 0                                 # both parts empty: no-op
    assert av(h=43) == E and av(aw=31) == E and av(vv=None, vt=None) == E and av(a_v=None, at=None) == E
    assert av(dt=float("inf")) == E
    assert av(at=VL + 4096) == E                             # audio tokens inside the video latent
    assert av(vt=AL) == E                                    # video tokens over the audio latent
    assert av(al=VV + 64) == E                               # audio latent updated over the video velocities
    assert av(a_v=VL + 64) == E                              # audio velocities inside the updated video latent


def test_abi_rejects_bad_rope_table_calls(h3):
    lib = h3.load_library()
    cfg = h3.rope_cfg()
    P = 1 << 26
    C, T = P, 4 * P
    E, R = h3.H3ATTN_EINVAL, h3.H3ATTN_ERANGE

    def tab(cf=cfg, c=C, n=28192, t=T):
        return lib.h3attn_rope_table(ctypes.byref(cf) if cf is not None else None, c, n, t, None)

    assert tab(n=0) == 0                                     # empty: no-op
    assert tab(cf=None) == E and tab(cf=_cfg(h3, head_dim=64)) == E
    assert tab(c=None) == E and tab(t=None) == E and tab(t=T + 8) == E and tab(c=C + 2) == E and tab(n=-1) == E
    assert tab(t=C + 4096) == E                              # table over the coordinates
    assert tab(n=2 ** 25) == R                               # n * 64 pairs reach 2^31
    assert tab() not in (E, R)                               # valid: fails only for want of a GPU


def test_abi_rejects_bad_linear_calls(h3):
    lib = h3.load_library()
    P = 1 << 26
    X, Wt, B, Y, T = P, 4 * P, 8 * P, 12 * P, 16 * P
    E, R = h3.H3ATTN_EINVAL, h3.H3ATTN_ERANGE

    def lin(x=X, xs=5376, w=Wt, ws=5376, b=B, y=Y, ys=16128, m=28192, n=16128, k=5376, t=T, rc=10752):
        return lib.h3attn_linear(x, xs, w, ws, b, y, ys, m, n, k, t, rc, None)

    assert lin(m=0) == 0                                     # empty: no-op
    assert lin(x=None) == E and lin(w=None) == E and lin(y=None) == E
    assert lin(x=X + 8) == E and lin(y=Y + 2) == E and lin(b=B + 4) == E
    assert lin(n=16000) == E and lin(k=5370) == E and lin(k=0) == E and lin(n=0) == E and lin(m=-1) == E
    assert lin(xs=5368) == E and lin(ws=5380) == E and lin(ys=16120) == E
    assert lin(rc=100) == E and lin(rc=16384) == E and lin(rc=-128) == E
    assert lin(t=None) == E and lin(t=T + 8) == E           # rotation without its table, misaligned table
    assert lin(t=None, rc=0) not in (E, R)                   # no rotation: no table needed (fails later: no GPU)
    assert lin(t=Y + 16128 * 2 * 100) == E                   # y overlaps the table
    assert lin(y=X + 4096) == E and lin(y=Wt) == E and lin(b=Y + 64) == E   # y overlaps an input
    assert lin(xs=2 ** 22 + 8) == R                          # a 256-row tile of x spans 2^31 bytes
    assert lin(ys=2 ** 22) == R and lin(ws=2 ** 22) == R      # ... of y, of w
    assert lin(m=2 ** 19, xs=5376) == R                      # x spans 2^32 bytes
