"""CPU emulation of the bf16 Newton-Schulz recipe, for deriving parity tolerances.

Test infrastructure: it reproduces, in float32 torch CPU arithmetic, where the GPU's
Newton-Schulz ("Muon is Scalable for LLM Training", Sec. 2.1 Eq. 2) rounds to bf16.
Eq. 2's a X + b A X + c A^2 X is evaluated as P X with P = a I + b A + c A^2:

  X0 = bf16(M)                 unscaled; s = 1 / max(||M||_F, eps) in float32
  per iteration t (s_t = s on the first iteration, 1 afterwards):
    A  = bf16(s_t^2 * X X^T)             fp32 accumulation
    P  = bf16(a I + b A + c (A A))       A is the bf16 matrix
    X' = bf16(s_t * (P X))               iterations 1 .. N-1
    O  = fp32(s_t * (P X))               the last iteration

It shares no code with the HIP library and is not the oracle: the oracle is the exact
float64 iteration. The difference between the two is the rounding error a correct
bf16 implementation makes, which is what the tolerances have to cover. The float32
matmuls add in another order than the GPU's MFMA tiles; at these sizes that moves
the error by far less than the bf16 roundings do.
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).to(torch.float32)  # round to nearest even


def newton_schulz_bf16(m, a=3.4445, b=-4.7750, c=2.0315, steps=5, eps=1e-7) -> np.ndarray:
    """The bf16 recipe above on a float32 [A, B] matrix; tall inputs run transposed."""
    x = torch.from_numpy(np.ascontiguousarray(m, dtype=np.float32))
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T.contiguous()
    fro = float(np.sqrt(np.sum(x.double().numpy() ** 2)))
    s = float(np.float32(1.0) / np.float32(max(np.float32(fro), np.float32(eps))))
    xb = _bf16(x)
    eye = torch.eye(xb.shape[0])
    out = None
    for it in range(steps):
        st = s if it == 0 else 1.0
        gram = _bf16((st * st) * (xb @ xb.T))
        poly = _bf16(a * eye + b * gram + c * (gram @ gram))
        y = (poly @ xb) * st
        if it + 1 < steps:
            xb = _bf16(y)
        else:
            out = y
    o = out.T if tall else out
    return o.double().numpy()
