"""Full bidirectional softmax attention with MM-RoPE (oracle; test infrastructure only).

Every row attends to every row with no mask: the open release runs full
attention ("MiniMax Opens H3 Base Weights ..."; "Inside MiniMax H3 ...",
section 6), and attention is bidirectional so information flows from target
rows back into reference rows (explainer, paragraph on the missing cross-step
cache).  Per head:

    Q~ = rope(Q), K~ = rope(K)
    S  = Q~ K~^T * scale          (scale = 1/sqrt(D) unless given)
    O  = softmax_rows(S) V,       LSE = log sum_j exp(S_ij)

float64 throughout.  Query rows are processed in blocks so memory stays
O(block * N); a block changes nothing but memory use.
"""
import numpy as np

from .rope import rope


def bf16_bits_to_f64(bits):
    """Raw bfloat16 bits (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attention(q, k, v, coords, sections, thetas, scale=None, rope_q=True, rope_k=True,
              heads=None, rows=None, block=1024):
    """Attention of float arrays q, k, v [N, H, D] with coordinates [N, 3].

    heads : iterable of head indices to compute (default: all)
    rows  : array of query row indices to compute (default: all)
    Returns (O [len(rows), len(heads), D] float64, LSE [len(heads), len(rows)] float64).
    """
    n, nh, dim = q.shape
    heads = list(range(nh)) if heads is None else [int(h) for h in heads]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(dim)
    coords = np.asarray(coords, np.float32)
    out = np.zeros((len(rows), len(heads), dim), np.float64)
    lse = np.zeros((len(heads), len(rows)), np.float64)
    for hi, h in enumerate(heads):
        qh = np.asarray(q[rows, h:h + 1, :], np.float64)
        kh = np.asarray(k[:, h:h + 1, :], np.float64)
        vh = np.asarray(v[:, h, :], np.float64)
        if rope_q:
            qh = rope(qh, coords[rows], sections, thetas)
        if rope_k:
            kh = rope(kh, coords, sections, thetas)
        qh = qh[:, 0, :]
        kh = kh[:, 0, :]
        for b0 in range(0, len(rows), block):
            s = (qh[b0:b0 + block] @ kh.T) * scale
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[b0:b0 + block, hi, :] = (p @ vh) / l
            lse[hi, b0:b0 + block] = (m + np.log(l))[:, 0]
    return out, lse
