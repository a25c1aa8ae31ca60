"""Parity tolerances shared by the GPU tests.

Newton-Schulz in bf16 ("Muon is Scalable for LLM Training", Sec. 2.1 Eq. 2 with bf16
GEMM operands, unit roundoff 2^-9, fp32 accumulation) is held to the relative Frobenius
error 2e-2 that the method's bf16 recipe is stated to meet, on every matrix whose
working size m = min(A, B) is 64 or more. That covers every diffusion-transformer
shape of the workloads (m >= 2048 measured about 1%).

The tolerances below come from tests/ns_tol_sweep.py: seeded Gaussian and
Student-t(3) matrices of every working size m = 1..63 (400 draws per m and seed) and
of twelve sizes from 64 to 600 (40 draws each), the other side random up to 600 or a
small multiple of m, flat and tall. Each draw runs the float64 oracle and a CPU
emulation of the GPU's bf16 rounding recipe (tests/bf16_emulation.py: P = a I + b A +
c A^2 rounded to bf16, X' = P X) on the same input. Two seeds (2024/2025 and
7777/7778) gave these maxima per band of m:

    m          whole matrix        one line (row of a flat output, column of a tall one)
    1..12      0.106   0.439       0.165   0.820
    13..31     0.047   0.037       0.114   0.141
    32..63     0.030   0.029       0.083   0.123
    64..255    0.014   0.015       0.051   0.046
    256..600   0.012   0.012       0.048   0.053

and on 1024 x 4096, 2048 x 2048 and 2048 x 8192 (flat and tall, Gaussian and
Student-t(3)): at most 0.0081 whole and 0.032 per line. Each tolerance is the band's
maximum times a margin of 1.3 to 1.7, rounded up.

Why small m is worse: X0 = M / ||M||_F has normalised singular values x_i, and the five
iterations map them through f^5 with f(x) = a x + b x^3 + c x^5, whose slope at small x
is up to a^5 = 490. bf16 rounding perturbs every direction by about 2^-9 of the matrix;
directions with small x_i carry that perturbation amplified into outputs of order one.
With many directions (large m) that averages out in the Frobenius norm; with a handful
it does not. A nearly singular input (a normalised singular value near 1e-3, which
random square matrices of side 2 to 12 produce now and then) gave the 0.44 above, and
one of its lines was 82% off: the relative error of such inputs has no useful bound.
For m <= 12 the whole-matrix tolerance is an envelope of the draws, not a bound, and
no per-line bound is applied. These sizes are edge cases of the kernels' ragged
handling, not workload shapes.

The per-line bound catches what a whole-matrix error can hide: one wrong row of a
5120-row output adds only sqrt(1/5120) = 1.4% to the whole-matrix error, but 100% or
more to its own line's error.

fp32 element-wise maps with fp32 tree reductions (momentum, RowNorm, AdamW): 1e-5.
"""
import numpy as np

NS_TOL = 2e-2
FP32_TOL = 1e-5

# (largest m of the band, whole-matrix tolerance, per-line tolerance; None: no bound)
NS_BANDS = (
    (12, 0.6, None),
    (31, 0.065, 0.19),
    (63, 0.04, 0.17),
    (255, NS_TOL, 0.07),
    (None, NS_TOL, 0.07),
)


def _band(shape):
    m = min(shape)
    for hi, whole, line in NS_BANDS:
        if hi is None or m <= hi:
            return whole, line
    raise AssertionError("unreachable")


def ns_tol(shape):
    """The bf16 Newton-Schulz whole-matrix tolerance for a matrix of this shape."""
    return _band(shape)[0]


def ns_line_tol(shape):
    """The bf16 Newton-Schulz per-line tolerance for a matrix of this shape (inf where
    no per-line bound applies)."""
    line = _band(shape)[1]
    return float("inf") if line is None else line


def line_errors(x, ref):
    """Relative l2 error of every line of x against ref: rows of a flat or square
    matrix, columns of a tall one (the rows of the Newton-Schulz working matrix)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    axis = 0 if ref.shape[0] > ref.shape[1] else 1
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axis))
    den = np.sqrt(np.sum(ref ** 2, axis=axis))
    return num / np.where(den > 0, den, 1.0)


def ns_errors(x, ref):
    """(relative Frobenius error, largest relative line error) of x against ref."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    whole = float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))
    return whole, float(line_errors(x, ref).max()) if ref.size else 0.0


def assert_ns_close(x, ref, shape=None, tag="", scale=1.0):
    """Assert the bf16 Newton-Schulz bounds (whole matrix and every line) for x against
    the oracle's ref; `scale` widens both (more iterations than five). Returns
    (whole, worst line)."""
    shape = tuple(shape if shape is not None else np.shape(ref))
    whole, line = ns_errors(x, ref)
    assert whole < ns_tol(shape) * scale, (tag, shape, "whole", whole)
    assert line < ns_line_tol(shape) * scale, (tag, shape, "line", line)
    return whole, line
