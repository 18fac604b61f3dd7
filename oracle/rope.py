"""Three-axis rotary position embedding (oracle; test infrastructure only).

The (t, h, w) coordinates of a row rotate its Q and K ("MiniMax H3 - one
transformer that denoises video and audio together", position-chain paragraph:
position_ids -> rope() -> rotate Q, K; V is not rotated).  The inverse
frequencies are computed from rope_theta and the per-axis dimension split, not
loaded (same page, inv_freq paragraph).

Layout read here: the head dimension is cut into three contiguous sections,
t first, then h, then w (sizes d_t, d_h, d_w).  Inside section a, pair p
rotates the adjacent dims (o_a + 2p, o_a + 2p + 1) by the angle
pos_a * base_a ** (-2p / d_a):
    (x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi).
All arithmetic is float64; coordinates enter as their float32 values.
"""
import numpy as np


def rope(x, coords, sections, thetas):
    """Rotate x [N, H, D] (any float dtype) by coords [N, 3]; returns float64 [N, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(coords, dtype=np.float32).astype(np.float64)
    n, _, dim = x.shape
    if sum(sections) != dim or any(s % 2 for s in sections):
        raise ValueError("sections must be even and sum to the head dim")
    out = x.copy()
    off = 0
    for a in range(3):
        d = int(sections[a])
        if d == 0:
            continue
        p = np.arange(d // 2, dtype=np.float64)
        freq = float(thetas[a]) ** (-(2.0 * p) / d)            # [d/2]
        ang = pos[:, a:a + 1] * freq[None, :]                   # [N, d/2]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        xe = x[:, :, off:off + d:2]
        xo = x[:, :, off + 1:off + d:2]
        out[:, :, off:off + d:2] = xe * c - xo * s
        out[:, :, off + 1:off + d:2] = xe * s + xo * c
        off += d
    return out
