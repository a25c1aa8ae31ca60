"""Seeded randomized parity of muon_step through the C ABI against the float64 oracle.

Each case draws a set of 1-12 matrices with independent random shapes (each side
1-600; two cases draw 1-4 matrices with sides up to 2000), flat, tall and square, every
residue modulo the 4-, 64- and 256-element blockings, a random step index and period K (so refresh and RowNorm steps both
occur), a random update-scale rule, and the monitor on or off. Refresh steps are
checked through the W = 0 probe (the update itself) at the bf16 Newton-Schulz
tolerance (2e-2, wider bands when min(A, B) < 64, from tolerances.py) and its per-line
bound; RowNorm steps
and the momentum at the
fp32 tolerance 1e-5; the monitor against the oracle at the same tolerances.
"""
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import FP32_TOL, assert_ns_close, ns_tol

pytestmark = pytest.mark.gpu

MODES = {B.SCALE_MAX_DIM: "max_dim", B.SCALE_HIDDEN: "hidden", B.SCALE_RMS: "rms"}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


def rel_fro(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


@pytest.mark.parametrize("seed,max_side,max_count", [(s, 600, 12) for s in range(10)] + [(10, 2000, 4), (11, 2000, 4)])
def test_random_sets_vs_oracle(torch_dev, seed, max_side, max_count):
    torch, dev = torch_dev
    rng = np.random.default_rng(900 + seed)
    count = int(rng.integers(1, max_count + 1))
    shapes = [(int(rng.integers(1, max_side + 1)), int(rng.integers(1, max_side + 1))) for _ in range(count)]
    k = int(rng.choice([1, 2, 3, 5]))
    step = int(rng.integers(0, 10))
    if max_side > 600:
        step = 0  # the large draws run the Newton-Schulz refresh
    mode = int(rng.choice(list(MODES)))
    hidden = int(rng.integers(64, 1025))
    monitor = bool(rng.integers(0, 2))
    refresh = step % k == 0
    hp = B.default_hparams(period_k=k, scale_mode=mode, hidden=hidden if mode == B.SCALE_HIDDEN else 0)
    ohp = O.OracleHParams(period_k=k, scale_mode=MODES[mode], hidden=hidden if mode == B.SCALE_HIDDEN else 0)
    log(f"seed {seed}: {count} matrices {shapes}, K {k}, step {step} ({'refresh' if refresh else 'RowNorm'}), "
        f"scale {MODES[mode]}, monitor {monitor}")
    key = 950 + seed
    w_h = [np.zeros(s, np.float32) for s in shapes]  # W = 0 probe: W' is the update
    m_h = [WL.host_normal(key, WL.ROLE_M, i, s, 0.02) for i, s in enumerate(shapes)]
    g_h = [WL.host_normal(key, WL.ROLE_G, i, s, 1e-3) for i, s in enumerate(shapes)]
    w = [torch.from_numpy(x).to(dev) for x in w_h]
    m = [torch.from_numpy(x).to(dev) for x in m_h]
    g = [torch.from_numpy(x).to(dev) for x in g_h]
    rms = torch.full((count,), -1.0, dtype=torch.float32, device=dev) if monitor else None
    B.muon_step(w, m, g, step, hp, update_rms=rms)
    torch.cuda.synchronize()
    rms_h = rms.cpu().numpy() if monitor else None
    worst, worst_shape = 0.0, None
    for i, s in enumerate(shapes):
        w_ref, m_ref, u_rms = O.muon_step_monitored(w_h[i], m_h[i], g_h[i], step, ohp)
        tol = ns_tol(s) if refresh else FP32_TOL
        em = rel_fro(m[i].cpu().numpy(), m_ref)
        ew = rel_fro(w[i].cpu().numpy(), w_ref)
        if ew > worst:
            worst, worst_shape = ew, s
        assert em < FP32_TOL, (seed, s, "momentum", em)
        if refresh:  # W = 0 probe: W' is the update, held per line as well
            assert_ns_close(w[i].cpu().numpy(), w_ref, s, (seed, "update"))
        else:
            assert ew < tol, (seed, s, "update", ew, tol)
        if monitor:
            assert abs(rms_h[i] - u_rms) <= tol * abs(u_rms) + 1e-12, (seed, s, "monitor", rms_h[i], u_rms)
    log(f"seed {seed}: worst update error {worst:.2e} at {worst_shape}")
