"""fp64 CPU oracle for MM-RoPE + full bidirectional attention over one packed sequence.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the hot path computes, written from the pages:

* "Inside MiniMax H3: One DiT Stream for Text, Video, and Stereo Audio"
  (section 2: one packed sequence; section 4: RoPE creates a shared physical
  timeline; section 6: full attention is the cost),
* "MiniMax H3 - one transformer that denoises video and audio together"
  (paragraphs on latent frames, the 40 Hz clock and the 5/3 frame rescale,
  text as 1-D RoPE, the position chain into rope(), the normalised spatial grid),
* "MiniMax Opens H3 Base Weights ..." (full attention only in the open release),
* AdaLN: the AdaLN paragraphs of the explainer page (norm(x) * (1 + scale) +
  shift, index = timestep_index * 3 + token_tag) and section 5 of the thread
  (shift, scale and gate per block for the attention and MLP paths),
* packing: the explainer's patchify, latent-frame and flow-matching paragraphs.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and imports
nothing from it; the two meet only in the seeded inputs of ``workloads``.

Modules:
  coords     - segment table -> (t, h, w) per row, float32, exact rounding
  rope       - three-axis rotary embedding of Q / K, float64
  attention  - softmax(QK^T * scale) V per head, float64, plus log-sum-exp
  adaln      - per-row indexed modulation, the gated residual, float64
  pack       - 1x2x2 patchify of video latents, audio packing, the Euler step
  linear     - the attention projections, with Q and K rotated (fused QKV)
"""
from .coords import build_coords, f32_round, video_hw_f64
from .rope import rope
from .attention import attention, bf16_bits_to_f64
from . import adaln
from . import pack
from . import linear

__all__ = ["build_coords", "f32_round", "video_hw_f64", "rope",
           "attention", "bf16_bits_to_f64", "adaln", "pack", "linear"]
