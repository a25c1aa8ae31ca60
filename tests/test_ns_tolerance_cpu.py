"""The bf16 Newton-Schulz tolerances against a fresh sweep (CPU).

tests/tolerances.py sets the whole-matrix and per-line tolerances from the maxima of
tests/ns_tol_sweep.py over two seeds. This runs a smaller sweep with a third seed, the
float64 oracle against the CPU emulation of the GPU's bf16 rounding recipe, and checks
that every draw lies inside its band's tolerances; and that the per-line bound rejects
one wrong line that the whole-matrix bound lets through.
"""
import numpy as np
import pytest
import torch

import ns_tol_sweep as S
from bf16_emulation import newton_schulz_bf16
from oracle import muon_oracle as O
from tolerances import NS_TOL, assert_ns_close, ns_errors, ns_line_tol, ns_tol


@pytest.fixture(autouse=True)
def one_thread():
    n = torch.get_num_threads()
    torch.set_num_threads(1)
    yield
    torch.set_num_threads(n)


def test_bands_cover_a_fresh_sweep():
    worst = {}
    for ms, draws, seed in ((range(1, 64), 16, 4242), (S.LARGE_M, 3, 4243)):
        for m in ms:
            rng = np.random.default_rng([seed, m])
            for d in range(draws):
                x = S.draw(rng, m, d)
                assert_ns_close(newton_schulz_bf16(x), O.newton_schulz(x), x.shape, f"m {m} draw {d}")
                whole, line = S.measure(x)
                w0, l0 = worst.get(m, (0.0, 0.0))
                worst[m] = (max(w0, whole / ns_tol(x.shape)), max(l0, line / ns_line_tol(x.shape)))
    # the workloads' sizes keep the stated 2e-2
    assert all(ns_tol((m, 600)) == NS_TOL for m in S.LARGE_M)
    assert max(v[0] for v in worst.values()) < 1.0


def test_per_line_bound_catches_one_wrong_row():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((512, 2048)).astype(np.float32)
    ref = O.newton_schulz(x)
    emu = newton_schulz_bf16(x)
    assert_ns_close(emu, ref, x.shape)
    bad = emu.copy()
    bad[100] *= 1.1  # one row 10% off
    whole, line = ns_errors(bad, ref)
    assert whole < ns_tol(x.shape), whole      # hidden in the whole-matrix error
    assert line > ns_line_tol(x.shape), line   # caught per line
    with pytest.raises(AssertionError):
        assert_ns_close(bad, ref, x.shape)
    bad_t = emu.T.copy()                       # the same on a tall output: columns
    bad_t[:, 7] = -bad_t[:, 7]
    with pytest.raises(AssertionError):
        assert_ns_close(bad_t, ref.T, bad_t.shape)
