"""GPU parity of the AdamW companion and the hybrid optimizer (through the C ABI).

AdamW runs in fp32 on the device against the float64 oracle: the update
W' - (1 - lr wd) W is compared at 1e-5 relative Frobenius (fp32 elementwise work
with one square root and one division per element), and the moments at 1e-6.
Weights start at zero so that W stays the size of the updates and fp32 rounding of
W does not swamp the update's own error; weight decay on a non-zero W is checked
separately (zero gradient).
Sizes cover one element, ragged tails around the 4096-element block, more than the
48 tensors one launch carries, and a large step (bias corrections near 1).
The hybrid optimizer runs a small double-stream DiT (20 block matrices in two
groups, 42 AdamW tensors) through a K = 3 Periodic schedule, teacher-forced per step
against the Muon and AdamW oracles.
"""
import sys

import numpy as np
import pytest

from oracle import adamw_oracle as A
from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import hybrid as H
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import FP32_TOL, assert_ns_close

pytestmark = pytest.mark.gpu

UPD_TOL = 1e-5
MOM_TOL = 1e-6
# The device receives fp32 hyperparameters; the oracle gets the same values (1 - beta2
# would otherwise amplify the fp32 rounding of 0.999 a thousandfold, to 1.3e-5).
AHP = A.AdamWHParams(**{f: float(np.float32(getattr(A.AdamWHParams(), f)))
                        for f in ("lr", "beta1", "beta2", "eps", "weight_decay")})


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


def to_dev(torch, dev, x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def to_host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_fro(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def check_adamw(torch, dev, shapes, steps, key, start_step=0, g_std=1e-3):
    """Teacher-forced AdamW steps on the GPU against the oracle."""
    n = len(shapes)
    w_h = [np.zeros(s) for s in shapes]
    m_h = [np.zeros(s) for s in shapes]
    v_h = [np.zeros(s) for s in shapes]
    w = [to_dev(torch, dev, x) for x in w_h]
    m = [torch.zeros_like(x) for x in w]
    v = [torch.zeros_like(x) for x in w]
    decay = 1.0 - AHP.lr * AHP.weight_decay
    worst = 0.0
    for k in range(steps):
        step = start_step + k
        g_h = [WL.host_normal(key, WL.ROLE_G, i, s, g_std, step) for i, s in enumerate(shapes)]
        B.adamw_step(w, [to_dev(torch, dev, x) for x in g_h], m, v, step)
        torch.cuda.synchronize()
        for i in range(n):
            w_ref, m_ref, v_ref = A.adamw_step(w_h[i], g_h[i], m_h[i], v_h[i], step, AHP)
            w1, m1, v1 = to_host(w[i]), to_host(m[i]), to_host(v[i])
            err = rel_fro(w1 - decay * w_h[i], w_ref - decay * w_h[i])
            worst = max(worst, err)
            assert err < UPD_TOL, (shapes[i], step, err)
            assert rel_fro(m1, m_ref) < MOM_TOL and rel_fro(v1, v_ref) < MOM_TOL, (shapes[i], step)
            w_h[i], m_h[i], v_h[i] = w1, m1, v1  # teacher forcing
    return worst


def test_adamw_ragged_sizes_vs_oracle(torch_dev):
    torch, dev = torch_dev
    shapes = [(1,), (3,), (4095,), (4096,), (4097,), (10000,), (7, 33), (128, 256), (3, 5, 7)]
    worst = check_adamw(torch, dev, shapes, 4, 400)
    log(f"ragged sizes: worst update rel err {worst:.2e}")


def test_adamw_more_tensors_than_one_launch(torch_dev):
    torch, dev = torch_dev
    shapes = [(37 * (i % 7) + 5,) for i in range(100)]
    worst = check_adamw(torch, dev, shapes, 2, 401)
    log(f"100 tensors: worst update rel err {worst:.2e}")


def test_adamw_large_step_and_zero_gradient(torch_dev):
    torch, dev = torch_dev
    check_adamw(torch, dev, [(5000,), (64, 64)], 2, 402, start_step=100000)
    # zero gradient from zero state: W' = (1 - lr wd) W, moments stay zero
    w_h = WL.host_normal(403, WL.ROLE_W, 0, (4100,), 0.02)
    w = [to_dev(torch, dev, w_h)]
    m, v = [torch.zeros_like(w[0])], [torch.zeros_like(w[0])]
    B.adamw_step(w, [torch.zeros_like(w[0])], m, v, 0)
    torch.cuda.synchronize()
    assert float(m[0].abs().max()) == 0.0 and float(v[0].abs().max()) == 0.0
    assert rel_fro(to_host(w[0]), A.adamw_step(w_h, np.zeros(4100), np.zeros(4100), np.zeros(4100), 0, AHP)[0]) < 1e-7


def test_adamw_is_deterministic(torch_dev):
    torch, dev = torch_dev
    g = to_dev(torch, dev, WL.host_normal(404, WL.ROLE_G, 0, (50000,), 1e-3))
    outs = []
    for _ in range(2):
        w = [to_dev(torch, dev, WL.host_normal(404, WL.ROLE_W, 0, (50000,), 0.02))]
        m, v = [torch.zeros_like(w[0])], [torch.zeros_like(w[0])]
        for s in range(3):
            B.adamw_step(w, [g], m, v, s)
        torch.cuda.synchronize()
        outs.append((w[0].clone(), m[0].clone(), v[0].clone()))
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))


def test_hybrid_optimizer_small_dit_periodic_schedule(torch_dev):
    torch, dev = torch_dev
    pl = H.dit_parameter_list(256, 2, head_dim=64, text_dim=512, pooled_dim=256, freq_dim=64)
    muon_names, adamw_names = H.split_param_groups(pl)
    assert len(muon_names) == 20 and len(adamw_names) == 42
    shapes = dict(pl)
    names = [n for n, _ in pl]
    w_h = {n: np.zeros(shapes[n]) for n in names}  # W = 0: comparisons at the updates' scale
    params = {n: to_dev(torch, dev, w_h[n]) for n in names}
    opt = H.HybridOptimizer(params)
    mhp = O.OracleHParams()
    m_h = {n: np.zeros(shapes[n]) for n in muon_names}
    am_h = {n: np.zeros(shapes[n]) for n in adamw_names}
    av_h = {n: np.zeros(shapes[n]) for n in adamw_names}
    decay_m = 1.0 - mhp.lr * mhp.weight_decay
    decay_a = 1.0 - AHP.lr * AHP.weight_decay
    for step in range(4):
        g_h = {n: WL.host_normal(405, WL.ROLE_G, i, shapes[n], 1e-3, step) for i, n in enumerate(names)}
        opt.step({n: to_dev(torch, dev, g_h[n]) for n in names})
        torch.cuda.synchronize()
        refresh = step % 3 == 0
        worst_m = worst_a = 0.0
        for n in muon_names:
            w_ref, m_ref = O.muon_step(w_h[n], m_h[n], g_h[n], step, mhp)
            w1 = to_host(params[n])
            if refresh:
                err = assert_ns_close(w1 - decay_m * w_h[n], w_ref - decay_m * w_h[n], w1.shape, (n, step))[0]
            else:
                err = rel_fro(w1 - decay_m * w_h[n], w_ref - decay_m * w_h[n])
                assert err < FP32_TOL, (n, step, err)
            worst_m = max(worst_m, err)
            w_h[n], m_h[n] = w1, to_host(opt.momenta[n])
        for n in adamw_names:
            w_ref, m_ref, v_ref = A.adamw_step(w_h[n], g_h[n], am_h[n], av_h[n], step, AHP)
            w1 = to_host(params[n])
            err = rel_fro(w1 - decay_a * w_h[n], w_ref - decay_a * w_h[n])
            worst_a = max(worst_a, err)
            assert err < UPD_TOL, (n, step, err)
            w_h[n], am_h[n], av_h[n] = w1, to_host(opt.exp_avg[n]), to_host(opt.exp_avg_sq[n])
        log(f"step {step} ({'refresh' if refresh else 'rownorm'}): Muon worst {worst_m:.2e}, AdamW worst {worst_a:.2e}")
    assert opt.step_count == 4
