"""Plain, slow, float64 CPU oracle for the Muon step and its Periodic Row-wise variant.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

Sources (the pages this follows; sections named, no line numbers):
  [MS]  "Muon is Scalable for LLM Training" (reading notes on the Moonlight paper):
        Sec. 2.1 Eq. 1 (momentum, Newton-Schulz, plain update), the Newton-Schulz
        paragraph with Eq. 2 and the coefficients a, b, c; Sec. 2.2 Eq. 3 (weight
        decay), Lemma 1 (update RMS), Eq. 4 (0.2 * sqrt(max(A,B)) scale), and the
        paragraph on the remaining hyper-parameters (N = 5, mu = 0.95).
  [DiT] "Scaling Muon for Diffusion Transformers" (summary page): the Periodic
        Row-wise Muon paragraphs (NS5 once every K steps, RowNorm of the current
        momentum on the other steps, K = 3, gamma = 0.15, gamma = 1 means reusing
        the Muon learning rate) and the distributed-implementation paragraph
        (rows of flat matrices are shard-local; tall matrices reduce per-column norms).
  [ABS] The same paper's abstract page: the full NS5 update runs once in every K
        steps, and the steps in between take a row-wise constrained update of the
        momentum as it stands at that step.

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
  R14 The scale rules of [MS] Sec. 3.1 replace the factor 0.2 * sqrt(max(A, B)) of
      Eq. 4: Eq. 5 uses 0.2 * sqrt(H) with H the model's hidden size (a caller
      parameter), Eq. 6 uses 0.2 / RMS(O) with RMS(O) = sqrt(mean(O^2)), divided as
      max(RMS(O), eps) so that O = 0 gives a zero update (the page divides exactly).
      Eq. 7 is Eq. 4.
  R15 On RowNorm steps Eq. 6 takes RMS(R) = 1/sqrt(max(A, B)), the exact RMS of a
      RowNorm output whose lines all have norm >= eps, so the step is 0.2 * sqrt(max)
      * gamma * R as under Eq. 4. (Measuring RMS(gamma R) instead would cancel gamma,
      which [DiT] uses to set the RowNorm step size relative to NS5.)
  R16 The update-RMS monitor of a step is RMS(c U): the RMS of the term that Eq. 4
      (5, 6) multiplies by the learning rate, weight decay excluded; [MS] Lemma 1 and
      the consistent-update-RMS paragraph make it about 0.2 under Eq. 4.

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
    scale_mode: str = "max_dim"   # "max_dim" (Eq. 4 / Eq. 7), "hidden" (Eq. 5), "rms" (Eq. 6)
    hidden: int = 0               # H of Eq. 5


SCALE_MODES = ("max_dim", "hidden", "rms")


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


def rms(x) -> float:
    """RMS(X) = sqrt(mean of the squared entries) ([MS] Lemma 1, Sec. 3.1 Eq. 6)."""
    x = _f64(x)
    return math.sqrt(float(np.sum(x * x)) / x.size) if x.size else 0.0


def direction_scale(u, shape, kind: str, hp) -> float:
    """The factor c that multiplies the direction U in W - lr (c U + lambda W).

    kind is "ns5" (U = O on refresh steps) or "rownorm" (U = gamma R).
      max_dim: c = 0.2 sqrt(max(A, B))       ([MS] Eq. 4, the same as Eq. 7)
      hidden:  c = 0.2 sqrt(H)               ([MS] Eq. 5)
      rms:     c = 0.2 / max(RMS(O), eps)    ([MS] Eq. 6, R14) on refresh steps,
               c = 0.2 sqrt(max(A, B))       on RowNorm steps (R15)
    """
    mode = hp.scale_mode
    if mode not in SCALE_MODES:
        raise ValueError(f"unknown scale mode {mode!r}")
    if mode == "hidden":
        if hp.hidden < 1:
            raise ValueError("the hidden scale rule needs hidden >= 1")
        return hp.rms_scale * math.sqrt(hp.hidden)
    if mode == "rms" and kind == "ns5":
        return hp.rms_scale / max(rms(u), hp.eps)
    return hp.rms_scale * math.sqrt(max(shape))


def apply_update(w, u, coef: float, lr: float, weight_decay: float) -> np.ndarray:
    """W_t = W_{t-1} - lr * (coef * U + lambda * W_{t-1}) (the common form of Eq. 4-7)."""
    w = _f64(w)
    return w - lr * (coef * _f64(u) + weight_decay * w)


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


def _step(w, m_prev, grad, refresh: bool, hp: OracleHParams):
    m = momentum(m_prev, grad, hp.mu)
    if refresh:
        u, kind = ns5_update_direction(m, hp), "ns5"
    else:
        u, kind = rownorm_update_direction(m, hp), "rownorm"
    coef = direction_scale(u, m.shape, kind, hp)
    w_new = apply_update(w, u, coef, hp.lr, hp.weight_decay)
    return w_new, m, coef * rms(u)


def muon_step(w, m_prev, grad, step: int, hp: OracleHParams = OracleHParams()):
    """One Periodic Row-wise Muon step for one [A, B] matrix; returns (W_t, M_t).

    Momentum every step (Eq. 1, R5); on refresh steps (R4) the direction is
    NS5(M_t), otherwise gamma * RowNorm(M_t) (R1, R2); the update is Eq. 4 (or the
    scale rule hp.scale_mode selects, R14, R15) with weight decay on both kinds of
    step (R6, R7). period_k = 1 is vanilla Muon.
    """
    w_new, m, _ = _step(w, m_prev, grad, is_refresh_step(step, hp.period_k), hp)
    return w_new, m


def muon_step_monitored(w, m_prev, grad, step: int, hp: OracleHParams = OracleHParams()):
    """muon_step plus the step's update RMS (R16); returns (W_t, M_t, rms)."""
    return _step(w, m_prev, grad, is_refresh_step(step, hp.period_k), hp)


def rownorm_step(w, m_prev, grad, hp: OracleHParams = OracleHParams()):
    """A non-refresh step regardless of the schedule; returns (W_t, M_t)."""
    w_new, m, _ = _step(w, m_prev, grad, False, hp)
    return w_new, m


def vanilla_step(w, m_prev, grad, hp: OracleHParams = OracleHParams()):
    """A refresh (vanilla Muon) step regardless of the schedule; returns (W_t, M_t)."""
    w_new, m, _ = _step(w, m_prev, grad, True, hp)
    return w_new, m
