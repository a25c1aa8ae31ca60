"""GPU parity of the update-scale rules (Eq. 5, Eq. 6) and the update-RMS monitor.

"Muon is Scalable for LLM Training", Sec. 3.1: Eq. 5 scales O by 0.2 sqrt(H), Eq. 6
by 0.2 / RMS(O). The HIP path is called through the C ABI and compared with the
float64 oracle on the same seeded inputs:
  * the update of a refresh step (NS5 through bf16 MFMA) at 2e-2 relative Frobenius;
  * RowNorm steps and momentum at 1e-5 (fp32 elementwise maps, fp32 tree sums);
  * Eq. 6 makes the update RMS exactly 0.2: with W = 0 the RMS of W' / lr is checked
    at 1e-5, which tests the device's RMS(O) reduction independently of NS5's error;
  * the monitor against the oracle's value (2e-2 on refresh steps, 1e-5 on RowNorm
    steps) and against the RMS of the GPU's own update (W = 0 probe, 1e-5).
"""
import math
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import FP32_TOL, assert_ns_close, ns_tol

pytestmark = pytest.mark.gpu

MODES = {"max_dim": B.SCALE_MAX_DIM, "hidden": B.SCALE_HIDDEN, "rms": B.SCALE_RMS}
HIDDEN = 320
# flat, tall, square, ragged, several 256-tiles, a single row and column
SHAPES = [(128, 512), (384, 96), (256, 256), (300, 700), (700, 300), (1, 9), (9, 1), (640, 1152)]


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


def inputs(key, shapes, w_std=0.02, m_std=0.02, g_std=1e-3):
    ws = [WL.host_normal(key, WL.ROLE_W, i, s, w_std) for i, s in enumerate(shapes)]
    ms = [WL.host_normal(key, WL.ROLE_M, i, s, m_std) for i, s in enumerate(shapes)]
    gs = [WL.host_normal(key, WL.ROLE_G, i, s, g_std) for i, s in enumerate(shapes)]
    return ws, ms, gs


def oracle_hp(mode, **kw):
    return O.OracleHParams(scale_mode=mode, hidden=HIDDEN, **kw)


def run_gpu(torch, dev, ws, ms, gs, step, mode, period_k=3, monitor=True, w_zero=False):
    w = [to_dev(torch, dev, np.zeros_like(x) if w_zero else x) for x in ws]
    m = [to_dev(torch, dev, x) for x in ms]
    g = [to_dev(torch, dev, x) for x in gs]
    rms = torch.full((len(ws),), -1.0, dtype=torch.float32, device=dev) if monitor else None
    hp = B.default_hparams(scale_mode=MODES[mode], hidden=HIDDEN, period_k=period_k)
    B.muon_step(w, m, g, step, hp, update_rms=rms)
    torch.cuda.synchronize()
    return [to_host(x) for x in w], [to_host(x) for x in m], (to_host(rms) if monitor else None)


@pytest.mark.parametrize("mode", ["max_dim", "hidden", "rms"])
def test_refresh_step_each_scale_rule_vs_oracle(torch_dev, mode):
    torch, dev = torch_dev
    ws, ms, gs = inputs(300, SHAPES)
    log(f"refresh step, scale rule {mode}: {SHAPES}")
    w1, m1, mon = run_gpu(torch, dev, ws, ms, gs, 0, mode)
    hp = oracle_hp(mode)
    decay = 1.0 - HP_LR_WD(hp)
    for i, s in enumerate(SHAPES):
        w_ref, m_ref, mon_ref = O.muon_step_monitored(ws[i], ms[i], gs[i], 0, hp)
        assert rel_fro(m1[i], m_ref) < FP32_TOL
        # the update itself (W' - decay W), so that W's size does not hide its error
        merr = abs(mon[i] - mon_ref) / mon_ref
        err, line = assert_ns_close(w1[i] - decay * ws[i], w_ref - decay * ws[i], s)
        log(f"  {s}: update rel err {err:.3e}, worst line {line:.3e}, monitor {mon[i]:.5f} vs {mon_ref:.5f}")
        assert merr < ns_tol(s), (s, mon[i], mon_ref)


def HP_LR_WD(hp):
    return hp.lr * hp.weight_decay


@pytest.mark.parametrize("mode", ["max_dim", "hidden", "rms"])
def test_rownorm_step_each_scale_rule_vs_oracle(torch_dev, mode):
    torch, dev = torch_dev
    ws, ms, gs = inputs(301, SHAPES)
    log(f"RowNorm step, scale rule {mode}")
    w1, m1, mon = run_gpu(torch, dev, ws, ms, gs, 1, mode)
    hp = oracle_hp(mode)
    for i, s in enumerate(SHAPES):
        w_ref, m_ref, mon_ref = O.muon_step_monitored(ws[i], ms[i], gs[i], 1, hp)
        assert rel_fro(m1[i], m_ref) < FP32_TOL
        assert rel_fro(w1[i], w_ref) < FP32_TOL, s
        assert abs(mon[i] - mon_ref) / mon_ref < FP32_TOL, (s, mon[i], mon_ref)


def test_eq6_refresh_update_rms_is_point_two_exactly(torch_dev):
    """W = 0: the Eq. 6 update is -lr 0.2 O / RMS(O), whatever NS5's rounding did to O."""
    torch, dev = torch_dev
    ws, ms, gs = inputs(302, SHAPES, m_std=0.0, g_std=1.0)
    w1, _, mon = run_gpu(torch, dev, ws, ms, gs, 0, "rms", w_zero=True)
    lr = O.OracleHParams().lr
    for i, s in enumerate(SHAPES):
        r = math.sqrt(float(np.mean(w1[i] ** 2))) / lr
        log(f"  {s}: RMS(update) / lr = {r:.7f}, monitor {mon[i]:.7f}")
        assert abs(r - 0.2) < 0.2 * FP32_TOL, (s, r)
        assert abs(mon[i] - 0.2) < 0.2 * FP32_TOL, (s, mon[i])


@pytest.mark.parametrize("step", [0, 1])
def test_monitor_equals_rms_of_gpu_update(torch_dev, step):
    """W = 0 probe: the monitor equals the RMS of the GPU's own update to fp32 rounding."""
    torch, dev = torch_dev
    ws, ms, gs = inputs(303, SHAPES)
    lr = O.OracleHParams().lr
    for mode in ("max_dim", "hidden"):
        w1, _, mon = run_gpu(torch, dev, ws, ms, gs, step, mode, w_zero=True)
        for i, s in enumerate(SHAPES):
            r = math.sqrt(float(np.mean(w1[i] ** 2))) / lr
            assert abs(mon[i] - r) < r * FP32_TOL, (mode, step, s, mon[i], r)


def test_eq6_zero_direction_leaves_pure_decay(torch_dev):
    torch, dev = torch_dev
    shapes = [(64, 200), (200, 64)]
    ws, _, _ = inputs(304, shapes)
    zeros = [np.zeros(s) for s in shapes]
    w1, _, mon = run_gpu(torch, dev, ws, zeros, zeros, 0, "rms")
    hp = oracle_hp("rms")
    for i in range(len(shapes)):
        assert np.all(np.isfinite(w1[i]))
        w_ref, _ = O.vanilla_step(ws[i], zeros[i], zeros[i], hp)
        assert rel_fro(w1[i], w_ref) < 1e-6
        assert mon[i] == 0.0


def test_monitor_leaves_results_unchanged_and_skips_empty(torch_dev):
    """Asking for the monitor changes no bit of W or M; empty matrices keep their entry."""
    torch, dev = torch_dev
    shapes = [(128, 512), (0, 16), (384, 96)]
    ws, ms, gs = inputs(305, [(128, 512), (1, 16), (384, 96)])
    ws[1], ms[1], gs[1] = (np.zeros((0, 16)),) * 3
    for step in (0, 1):
        for mode in ("max_dim", "hidden"):
            a_w, a_m, mon = run_gpu(torch, dev, ws, ms, gs, step, mode, monitor=True)
            b_w, b_m, _ = run_gpu(torch, dev, ws, ms, gs, step, mode, monitor=False)
            for i in range(len(shapes)):
                assert np.array_equal(a_w[i], b_w[i]) and np.array_equal(a_m[i], b_m[i])
            assert mon[1] == -1.0 and mon[0] > 0 and mon[2] > 0


def test_eq6_and_monitor_over_two_groups(torch_dev):
    """More than 16 matrices: two groups reuse one workspace region."""
    torch, dev = torch_dev
    shapes = [(64 + 16 * (i % 5), 96 + 32 * (i % 3)) if i % 2 == 0 else (96 + 32 * (i % 3), 64 + 16 * (i % 5))
              for i in range(18)]
    ws, ms, gs = inputs(306, shapes)
    w1, _, mon = run_gpu(torch, dev, ws, ms, gs, 0, "rms")
    hp = oracle_hp("rms")
    decay = 1.0 - HP_LR_WD(hp)
    worst = 0.0
    for i, s in enumerate(shapes):
        w_ref, _, mon_ref = O.muon_step_monitored(ws[i], ms[i], gs[i], 0, hp)
        err = assert_ns_close(w1[i] - decay * ws[i], w_ref - decay * ws[i], s)[0]
        worst = max(worst, err)
        assert abs(mon[i] - 0.2) < 1e-5
    log(f"  18 matrices, worst update rel err {worst:.3e}")


def test_rownorm_update_entry_point_monitor(torch_dev):
    """rownorm_update (every step RowNorm: the pages' RowNorm-only ablation) with the monitor."""
    torch, dev = torch_dev
    ws, ms, gs = inputs(307, SHAPES)
    w = [to_dev(torch, dev, x) for x in ws]
    m = [to_dev(torch, dev, x) for x in ms]
    hp_o = oracle_hp("max_dim")
    w_h, m_h = [x.copy() for x in ws], [x.copy() for x in ms]
    for step in range(3):
        g = [WL.host_normal(307, WL.ROLE_G, i, s, 1e-3, step) for i, s in enumerate(SHAPES)]
        rms = torch.zeros(len(SHAPES), dtype=torch.float32, device=dev)
        B.rownorm_update(w, m, [to_dev(torch, dev, x) for x in g], B.default_hparams(), update_rms=rms)
        torch.cuda.synchronize()
        mon = to_host(rms)
        for i, s in enumerate(SHAPES):
            w_ref, m_ref, mon_ref = O.muon_step_monitored(w_h[i], m_h[i], g[i], 1, hp_o)  # 1 % 3: RowNorm
            assert rel_fro(to_host(w[i]), w_ref) < FP32_TOL
            assert abs(mon[i] - mon_ref) < mon_ref * FP32_TOL
            w_h[i], m_h[i] = to_host(w[i]), to_host(m[i])  # teacher forcing
