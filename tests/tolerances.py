"""Parity tolerances shared by the GPU tests (relative Frobenius error).

Newton-Schulz in bf16 (Eq. 2 with bf16 GEMM operands, unit roundoff 2^-9, fp32
accumulation): five iterations of three products give about 1% on DiT-block shapes
(min(A, B) >= 2048 measured 1.1%), inside the 2e-2 the method's bf16 recipe is held to.

The error is larger when min(A, B) = m is small. X0 = M / ||M||_F has singular values
near 1 / sqrt(m), and each iteration multiplies small ones by about a = 3.4445, so they
reach the region near 1 after about log(0.5 sqrt(m)) / log(a) iterations. There
a + B = 3.4445 - 2.7435 = 0.70 cancels, and the bf16 rounding of B is amplified about
4x per iteration. For m >= 2048 that happens in the last two iterations only. For
m < 64 it happens in four or five of them: up to 5 * 4 * 2^-9 = 4e-2, which is the
tolerance there. Gaussian inputs with m between 3 and 48 measured up to 4.8e-2 at m = 3
(16 draws: mean 1.9e-2), 2.4e-2 at m = 22 and 1.95e-2 at m = 48, and at most 1.5e-2 for
m >= 64.

fp32 element-wise maps with fp32 tree reductions (momentum, RowNorm, AdamW): 1e-5.
"""
NS_TOL = 2e-2
NS_TOL_SMALL_M = 4e-2
SMALL_M = 64
FP32_TOL = 1e-5


def ns_tol(shape):
    """The bf16 Newton-Schulz tolerance for a matrix of this shape."""
    return NS_TOL_SMALL_M if min(shape) < SMALL_M else NS_TOL
