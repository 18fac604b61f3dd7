"""Error bound on the attention LSE against the exact fp64 oracle, derived from the kernel's roundings.

The kernel multiplies Q~ * scale * log2(e) rounded once to bf16 and K~ rounded once to bf16, and it
rounds every weight P to bf16 before PV.  One bf16 rounding of a continuously distributed value leaves
a relative error delta with E[delta^2] = 2^-16 E[1/m^2] / 3 = 2.75e-6 (m the significand,
log-uniform in [1, 2)).  For the unit-variance workloads (Q, K ~ N(0, 1), scale 1/sqrt(D)):

  * the Q rounding is common to every key of a row: dLSE = scale sum_d q_d delta_d kbar_d with kbar
    the softmax-weighted mean of K~, q / sqrt(D) for Gaussian keys, so its variance is
    3 E[delta^2] / D (2.5e-4 squared at D = 128);
  * the K rounding (each score moves by ~1.66e-3) and the P rounding (each weight by ~1.66e-3) are
    independent per key and average over the keys that carry weight: their variance is
    2 E[delta^2] sum p^2 / (sum p)^2, and sum p^2 / (sum p)^2 = e / N for lognormal weights of unit
    log-variance.

The bound is 8 standard deviations of the sum: 4.4e-3 at N = 64, 2.3e-3 at N = 1,000 and 2.0e-3
from N = 28,192 up.  A float64 simulation with 28,192 keys gives a maximum of 4.9 standard
deviations over 12,288 rows (the Q term is weighted by q_d^2, whose tail is heavier than a normal
one), so a full head of up to 81,792 rows stays below about 6.5.  The survey's 1e-3 gate cannot hold
on whole heads: their expected maximum is 1.2-1.6e-3 from the Q rounding alone.
"""
import numpy as np

E_DELTA2 = 2.75e-6


def lse_bound(n_keys, head_dim=128):
    var = 3.0 * E_DELTA2 / head_dim + 2.0 * E_DELTA2 * np.e / max(int(n_keys), 1)
    return 8.0 * float(np.sqrt(var))
