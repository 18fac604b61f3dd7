"""GPU parity of the attention half of one DiT block, chained through the C ABI, against
the oracle's composition of the same steps (MI355X, gfx950).

The five calls: AdaLN modulation of the residual stream (h3attn_adaln_modulate), the
fused QKV projection with Q and K rotated in its epilogue (h3attn_linear), attention over
the projection's strided Q/K/V views with the split-tail workspace the library asks for
(h3attn_forward_ws, rope_q = 0), the output projection (h3attn_linear) and the gated
residual with the next sublayer's modulation (h3attn_adaln_residual).  Between the
calls both sides store bfloat16, as the C ABI does: the oracle rounds every stage's exact
result once (oracle.adaln.round_bf16) before the next stage.

Tolerances.  Each stage is first held to its own bound (the projection's per-element
bound, the attention bounds max |err| <= 2e-2 and RMS <= 2e-3).  A stage's inputs may
then differ from the oracle's by the last stage's error, which the contractions that
follow average down; the end results are held to |err| <= 2 ulp_bf16(|ref|) + 2e-2 per
element and relative RMS <= 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import adaln as A
from oracle.linear import linear, qkv_rope

pytestmark = pytest.mark.gpu

SEC, TH = W.ROPE_SECTIONS, W.ROPE_THETAS
EPS = 1e-6
f64 = A.bf16_bits_to_f64


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_bf16(v):
    e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))[1]
    return np.ldexp(1.0, e - 8)


def close(got_bits, ref, tag, abs_tol=2e-2, rel_rms=1e-2, ulps=2):
    got = f64(got_bits)
    err = np.abs(got - ref)
    rr = float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(ref ** 2)))
    tol = ulps * ulp_bf16(ref) + abs_tol
    print("%s max|err| %.3e  max err/tol %.3f  rel-rms %.3e" % (tag, float(err.max()), float((err / tol).max()), rr),
          flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= tol) and rr <= rel_rms


@pytest.mark.parametrize("kind", [A.LAYER_NORM, A.RMS_NORM])
def test_attention_half_block(gpu_lib, kind):
    h3 = gpu_lib
    heads = 2
    c = heads * 128
    segs = [W.text(40, -40), W.video(3, 6, 8), W.audio(70, 0)]          # 324 rows
    n = W.n_tokens(segs)
    x, _, table = W.adaln_inputs(n, c, 2, seed=61)
    t_idx, tags = W.adaln_rows(segs)
    _, w_qkv, b_qkv = W.projection_inputs(n, c, 3 * c, seed=62)
    _, w_o, b_o = W.projection_inputs(n, c, c, seed=63)
    coords_h = h3.build_coords(segs)

    # ---- GPU: five calls through the C ABI
    coords = torch.from_numpy(coords_h).cuda()
    xd, tab = dev_bf16(x), dev_bf16(table)
    ti, tg = torch.from_numpy(t_idx).cuda(), torch.from_numpy(tags).cuda()
    base = tab.data_ptr()                      # planes [E][6][C]: shift_a, scale_a, gate_a, shift_m, scale_m, gate_m
    h1 = torch.empty_like(xd)
    h3.adaln_modulate(xd, c, ti, tg, base, base + 2 * c, 6 * c, table.shape[0], h1, c, n, c, kind, EPS)
    qkv = torch.empty((n, 3, heads, 128), dtype=torch.bfloat16, device="cuda")
    h3.linear(h1, c, dev_bf16(w_qkv), c, dev_bf16(b_qkv), qkv, 3 * c, n, 3 * c, c, h3.make_rope_table(coords), 2 * c)
    o = torch.empty((n, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, n), dtype=torch.float32, device="cuda")
    need = h3.forward_workspace_bytes(n, heads)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
    h3.forward_ws(h3.rope_cfg(), coords, 0, qkv[:, 0], qkv[:, 1], qkv[:, 2], o, lse, n, heads, 3 * c, c, 0.0,
                  ws, need)
    y = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    h3.linear(o, c, dev_bf16(w_o), c, dev_bf16(b_o), y, c, n, c, c)
    x_out = torch.empty_like(xd)
    h2 = torch.empty_like(xd)
    h3.adaln_residual(xd, y, c, ti, tg, base + 2 * 2 * c, base + 3 * 2 * c, base + 4 * 2 * c, 6 * c, table.shape[0],
                      x_out, h2, c, n, c, kind, EPS)
    torch.cuda.synchronize()

    # ---- oracle: the same steps, bf16 between them
    planes = f64(table)
    idx = A.adaln_index(t_idx, tags)
    h1_ref = A.round_bf16(A.modulate(f64(x), idx, planes[:, 0], planes[:, 1], kind, EPS))
    qkv_ref = A.round_bf16(qkv_rope(h1_ref, f64(w_qkv), f64(b_qkv), coords_h, heads, SEC, TH)).reshape(
        n, 3, heads, 128)
    o_ref, lse_ref = oracle.attention(qkv_ref[:, 0], qkv_ref[:, 1], qkv_ref[:, 2], coords_h, SEC, TH,
                                      rope_q=False, rope_k=False)
    o_ref = A.round_bf16(o_ref)
    y_ref = A.round_bf16(linear(o_ref.reshape(n, c), f64(w_o), f64(b_o)))
    x_out_ref, h2_ref = A.residual_modulate(f64(x), y_ref, idx, planes[:, 2], planes[:, 3], planes[:, 4], kind, EPS)

    tag = "kind %d" % kind
    close(host_bits(h1), h1_ref, tag + " h1", abs_tol=1e-3, ulps=1)
    close(host_bits(qkv).reshape(n, 3, heads, 128), qkv_ref, tag + " qkv", abs_tol=5e-3)
    og = f64(host_bits(o))
    err = og - o_ref
    print("%s attention max|err| %.3e rms %.3e lse %.3e" % (tag, float(np.abs(err).max()),
                                                           float(np.sqrt(np.mean(err ** 2))),
                                                           float(np.abs(lse.cpu().numpy() - lse_ref).max())), flush=True)
    assert np.abs(err).max() <= 2e-2 and np.sqrt(np.mean(err ** 2)) <= 2e-3
    close(host_bits(y), y_ref, tag + " out-proj")
    close(host_bits(x_out), x_out_ref, tag + " x_out")
    close(host_bits(h2), h2_ref, tag + " h2")
