"""Plain float64 CPU oracle for the AdamW companion of the hybrid optimizer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

Sources (pages named by title; sections, no line numbers):
  [DiT] "Scaling Muon for Diffusion Transformers" (summary page), setup paragraph:
        Muon updates only the 2-D weights inside the transformer blocks (about 99%
        of the trainable parameters); biases, normalisation parameters and every
        parameter outside the blocks stay on AdamW, an auxiliary group at lr 1e-4.
  [MS]  "Muon is Scalable for LLM Training", Sec. 2.2, matching-update-RMS
        paragraph: AdamW handles the non-matrix parameters and shares the learning
        rate and weight decay with Muon; Eq. 3 gives the decoupled decay form.

Readings (the pages name AdamW but do not restate it):
  R17 AdamW is Adam with bias-corrected moments and decoupled weight decay in
      Eq. 3's form: m <- b1 m + (1 - b1) g, v <- b2 v + (1 - b2) g^2,
      W <- W - lr (m_hat / (sqrt(v_hat) + eps) + wd W), m_hat = m / (1 - b1^t),
      v_hat = v / (1 - b2^t), with t = s + 1 for the 0-based step s.
  R18 Defaults: b1 = 0.9, b2 = 0.999, eps = 1e-8 (PyTorch's AdamW defaults; the
      pages train with PyTorch and give no values), lr = 1e-4 ([DiT] auxiliary
      group), wd = 0.1 (shared with Muon per [MS]).
  R19 Parameter-group rule ([DiT] setup paragraph): a parameter goes to Muon iff it
      is 2-D and lives inside a transformer block; everything else goes to AdamW.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class AdamWHParams:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1


def adamw_step(w, g, m, v, step: int, hp: AdamWHParams = AdamWHParams()):
    """One AdamW step (R17) at 0-based step `step`; returns (W, m, v) in float64."""
    if step < 0:
        raise ValueError("step must be >= 0")
    w, g, m, v = (np.asarray(x, dtype=np.float64) for x in (w, g, m, v))
    t = step + 1
    m = hp.beta1 * m + (1.0 - hp.beta1) * g
    v = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    m_hat = m / (1.0 - hp.beta1 ** t)
    v_hat = v / (1.0 - hp.beta2 ** t)
    w = w - hp.lr * (m_hat / (np.sqrt(v_hat) + hp.eps) + hp.weight_decay * w)
    return w, m, v


def goes_to_muon(name: str, shape, block_prefix: str = "blocks.") -> bool:
    """R19: 2-D parameters inside a transformer block are Muon's; the rest AdamW's."""
    return len(shape) == 2 and name.startswith(block_prefix)


def update_rms(w_old, w_new, hp: AdamWHParams) -> float:
    """RMS of the AdamW direction m_hat / (sqrt(v_hat) + eps) recovered from W."""
    w_old = np.asarray(w_old, dtype=np.float64)
    d = ((1.0 - hp.lr * hp.weight_decay) * w_old - np.asarray(w_new, dtype=np.float64)) / hp.lr
    return math.sqrt(float(np.mean(d * d))) if d.size else 0.0
