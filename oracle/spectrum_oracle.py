"""Plain float64 CPU oracle for the singular-spectrum diagnostic (SVD entropy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library.

Source: [MS] "Muon is Scalable for LLM Training" (reading notes on the Moonlight
paper), Sec. 3.4 "Dynamics of Singular Spectrum": for a weight matrix with singular
values sigma_1..sigma_n the SVD entropy is the Shannon entropy of the normalised
squared singular values q_i = sigma_i^2 / sum_j sigma_j^2, divided by log n, so a
flat spectrum scores 1 and a rank-one matrix 0. The page uses it to compare the
spectra of Muon- and AdamW-trained weights (higher means the update directions were
more diverse).

Readings taken where the page is silent:
  R21 n is the number of singular values, min(A, B) for an [A, B] matrix (the page
      indexes sigma_1..sigma_n), so the normalisation is log(min(A, B)).
  R22 Zero singular values contribute 0 (the limit of q log q as q -> 0). A matrix
      with a single singular value (min(A, B) = 1) has entropy 0: its one q is 1 and
      the unnormalised entropy is exactly 0. An all-zero matrix has no spectrum to
      normalise and its entropy is NaN (0 / 0).
  R23 The log base cancels in the ratio; natural logs are used.

Parity pins (tests/test_oracle_spectrum_pins.py): flat spectra give 1, rank one gives
0, hand-derived values for two-level spectra, a 2x2 closed form from the quadratic
formula, eigenvalues of W W^T from a different library routine, and invariance under
scaling, transposition and orthogonal transforms.
"""
from __future__ import annotations

import math

import numpy as np


def singular_values_sq(w) -> np.ndarray:
    """sigma_i^2 of W in float64, descending (length min(A, B))."""
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2:
        raise ValueError("a weight matrix is 2-D")
    if min(w.shape) == 0:
        return np.zeros(0)
    s = np.linalg.svd(w, compute_uv=False)
    return s * s


def entropy_of_spectrum(sigma_sq) -> float:
    """[MS] Sec. 3.4: -(1 / log n) sum_i q_i log q_i, q_i = sigma_i^2 / sum_j sigma_j^2."""
    lam = np.asarray(sigma_sq, dtype=np.float64)
    n = lam.size
    if n == 0:
        raise ValueError("empty spectrum")
    total = float(np.sum(lam))
    if total == 0.0:
        return math.nan  # R22: nothing to normalise
    if n == 1:
        return 0.0  # R22
    h = 0.0
    for x in lam:
        q = float(x) / total
        if q > 0.0:  # R22: q log q -> 0
            h -= q * math.log(q)
    return h / math.log(n)  # R21


def svd_entropy(w) -> float:
    """SVD entropy of one weight matrix ([MS] Sec. 3.4)."""
    return entropy_of_spectrum(singular_values_sq(w))
