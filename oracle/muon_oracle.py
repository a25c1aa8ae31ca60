"""Plain, slow, float64 CPU oracle for the Muon step and its Periodic Row-wise variant.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

Sources (the pages this follows; sections named, no line numbers):
  [MS]  "Muon is Scalable for LLM Training" (reading notes on the Moonlight paper):
        Sec. 2.1 Eq. 1 (momentum, Newton-Schulz, plain update), the Newton-Schulz
        paragraph with Eq. 2 and the coefficients a, b, c; Sec. 2.2 Eq. 3 (weight
        decay), Lemma 1 (update RMS), Eq. 4 (0.2 * sqrt(max(A,B)) scale), and the
        "other hyper-parameters" paragraph (N = 5, mu = 0.95).
  [DiT] "Scaling Muon for Diffusion Transformers" (summary page): the Periodic
        Row-wise Muon paragraphs (NS5 once every K steps, RowNorm of the current
        momentum on the other steps, K = 3, gamma = 0.15, gamma = 1 means reusing
        the Muon learning rate) and the distributed-implementation paragraph
        (rows of flat matrices are shard-local; tall matrices reduce per-column norms).
  [ABS] The same paper's abstract page: "a full NS5 spectral update once every K
        steps and a row-wise constrained update based on the current momentum at
        the remaining steps".

Readings taken where the pages are silent (each is also listed in the design notes):
  R1  The Periodic non-refresh update is Eq. 4 with O replaced by gamma * RowNorm(M_t).
  R2  RowNorm scales each row of M to unit l2 norm when A <= B (flat or square) and
      each column when A > B (tall).
  R3  Normalisations divide by max(norm, eps), eps = 1e-7 (the pages divide exactly).
  R4  Step s (0-based count of completed steps) is a refresh step iff s % K == 0.
  R5  Momentum is plain heavy-ball (Eq. 1), accumulated on every step of either kind.
  R6  Weight decay applies on RowNorm steps as well (Eq. 4 is otherwise unchanged).
  R7  The update scale is 0.2 * sqrt(max(A,B)) (Eq. 4, whose square root is lost in
      the extracted plain text but is present in its LaTeX form and in Eq. 7).
  R8  Tall matrices (A > B) run Newton-Schulz on M^T so the Gram matrix is the
      smaller one; the result is transposed back. Identical in exact arithmetic.

Parity pins (tests/test_oracle_pins.py): every function here is pinned to a closed
form, an invariant or a brute-force computation that is not this code.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class OracleHParams:
    """Hyperparameters with the pages' defaults.

    mu = 0.95 and N = 5 ([MS] Sec. 2.2, other hyper-parameters); a, b, c ([MS]
    Sec. 2.1, Newton-Schulz paragraph); 0.2 ([MS] Eq. 4); K = 3, gamma = 0.15
    ([DiT] Periodic Row-wise paragraph). lr and weight decay are workload choices.
    """

    lr: float = 1e-3
    weight_decay: float = 0.1
    mu: float = 0.95
    ns_a: float = 3.4445
    ns_b: float = -4.7750
    ns_c: float = 2.0315
    ns_steps: int = 5
    rms_scale: float = 0.2
    period_k: int = 3
    gamma: float = 0.15
    eps: float = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def momentum(m_prev, grad, mu: float) -> np.ndarray:
    """M_t = mu * M_{t-1} + grad ([MS] Sec. 2.1 Eq. 1; M_0 = 0)."""
    return mu * _f64(m_prev) + _f64(grad)


def is_tall(shape) -> bool:
    """A matrix [A, B] is tall when A > B (reading R8); square counts as flat."""
    return shape[0] > shape[1]


def newton_schulz(m, a: float = 3.4445, b: float = -4.7750, c: float = 2.0315,
                  steps: int = 5, eps: float = 1e-7) -> np.ndarray:
    """O = Newton-Schulz(M) ([MS] Sec. 2.1, Eq. 2).

    X_0 = M / ||M||_F, then `steps` times
        X <- a X + b (X X^T) X + c (X X^T)^2 X,
    written term by term as Eq. 2 states it. Tall inputs are transposed first
    and the result transposed back (R8); the Frobenius norm divides by
    max(||M||_F, eps) (R3).
    """
    x = _f64(m)
    tall = is_tall(x.shape)
    if tall:
        x = x.T
    fro = math.sqrt(float(np.sum(x * x)))
    x = x / max(fro, eps)
    for _ in range(steps):
        gram = x @ x.T                          # X X^T
        x = a * x + b * (gram @ x) + c * (gram @ (gram @ x))
    return x.T if tall else x


def row_normalise(m, eps: float = 1e-7) -> np.ndarray:
    """RowNorm of the momentum (reading R2, [DiT] Periodic and distributed paragraphs).

    Flat or square [A, B] (A <= B): each row divided by max(its l2 norm, eps).
    Tall (A > B): each column divided by max(its l2 norm, eps).
    """
    x = _f64(m)
    if is_tall(x.shape):
        norms = np.sqrt(np.sum(x * x, axis=0, keepdims=True))
    else:
        norms = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    return x / np.maximum(norms, eps)


def scaled_update(w, u, lr: float, weight_decay: float, rms_scale: float = 0.2) -> np.ndarray:
    """W_t = W_{t-1} - lr * (0.2 * U * sqrt(max(A, B)) + lambda * W_{t-1}) ([MS] Eq. 4, R7)."""
    w = _f64(w)
    n = max(w.shape)
    return w - lr * (rms_scale * _f64(u) * math.sqrt(n) + weight_decay * w)


def is_refresh_step(step: int, period_k: int) -> bool:
    """Reading R4: NS5 refresh iff step % K == 0 ([ABS]: once every K steps)."""
    if period_k < 1:
        raise ValueError("period_k must be >= 1")
    return step % period_k == 0


def ns5_update_direction(m, hp: OracleHParams) -> np.ndarray:
    """The refresh-step direction O_t = NS5(M_t)."""
    return newton_schulz(m, hp.ns_a, hp.ns_b, hp.ns_c, hp.ns_steps, hp.eps)


def rownorm_update_direction(m, hp: OracleHParams) -> np.ndarray:
    """The non-refresh direction gamma * RowNorm(M_t) (readings R1, R2)."""
    return hp.gamma * row_normalise(m, hp.eps)


def muon_step(w, m_prev, grad, step: int, hp: OracleHParams = OracleHParams()):
    """One Periodic Row-wise Muon step for one [A, B] matrix; returns (W_t, M_t).

    Momentum every step (Eq. 1, R5); on refresh steps (R4) the direction is
    NS5(M_t), otherwise gamma * RowNorm(M_t) (R1, R2); the update is Eq. 4 with
    weight decay on both kinds of step (R6, R7). period_k = 1 is vanilla Muon.
    """
    m = momentum(m_prev, grad, hp.mu)
    if is_refresh_step(step, hp.period_k):
        u = ns5_update_direction(m, hp)
    else:
        u = rownorm_update_direction(m, hp)
    w_new = scaled_update(w, u, hp.lr, hp.weight_decay, hp.rms_scale)
    return w_new, m


def rownorm_step(w, m_prev, grad, hp: OracleHParams = OracleHParams()):
    """A non-refresh step regardless of the schedule; returns (W_t, M_t)."""
    m = momentum(m_prev, grad, hp.mu)
    u = rownorm_update_direction(m, hp)
    return scaled_update(w, u, hp.lr, hp.weight_decay, hp.rms_scale), m


def vanilla_step(w, m_prev, grad, hp: OracleHParams = OracleHParams()):
    """A refresh (vanilla Muon) step regardless of the schedule; returns (W_t, M_t)."""
    m = momentum(m_prev, grad, hp.mu)
    u = ns5_update_direction(m, hp)
    return scaled_update(w, u, hp.lr, hp.weight_decay, hp.rms_scale), m
