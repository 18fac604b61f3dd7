"""Attention projections with the rotary embedding folded in (oracle; test
infrastructure only).

What the pages fix: text, reference media and noisy latents share one set of
attention projections ("Inside MiniMax H3: One DiT Stream for Text, Video, and
Stereo Audio", section 2); positions reach attention only through rope()
rotating Q and K, never V ("MiniMax H3 - one transformer that denoises video
and audio together", position-chain paragraph).

Readings where the pages are silent: a projection is y = x W^T (+ b), W stored
[out_features][in_features]; the fused QKV projection writes, per row, Q then K
then V, each [heads][head_dim]; the rotation of Q and K is the oracle.rope
rotation applied to the projection's exact output (the library rotates its
float32 accumulators before the single rounding to bfloat16).

All arithmetic is float64; the product is numpy's matmul, checked against a
plain loop and a library linear layer in the pins.
"""
import numpy as np

from .rope import rope


def linear(x, w, bias=None):
    """y = x W^T (+ bias): x [M, K], w [N, K], bias [N] -> [M, N], float64."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y


def qkv_rope(x, w, bias, coords, heads, sections, thetas, head_dim=128):
    """Fused QKV projection with Q and K rotated: returns y [M, 3 * heads * head_dim] float64."""
    y = linear(x, w, bias)
    m = y.shape[0]
    hd = heads * head_dim
    if y.shape[1] != 3 * hd:
        raise ValueError("weight rows must be 3 * heads * head_dim")
    out = y.copy()
    for part in (0, 1):   # Q, K
        blk = y[:, part * hd:(part + 1) * hd].reshape(m, heads, head_dim)
        out[:, part * hd:(part + 1) * hd] = rope(blk, coords, sections, thetas).reshape(m, hd)
    return out
