"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times: every matrix of a workload goes through one muon_step call per step.

The float64 oracle cannot redo a full workload in test time, so each step is
checked on outputs it can compute piece by piece:
  * momentum M' = mu M + G on every element (elementwise);
  * a RowNorm step on sampled rows of flat matrices and sampled columns of tall
    ones (each depends only on its own row or column), at 1e-5;
  * a refresh step (W = 0 probe) on whole sampled matrices, the smallest of the
    workload and one tall one, and for the 15B-scale set also its largest tall
    [30720, 5120] and flat [5120, 20480] matrices, against the oracle's NS5, at 2e-2
    for the whole matrix and 6e-2 for every row of a flat output (column of a tall
    one), so that one wrong line cannot hide in the whole-matrix error;
  * on every matrix of a refresh step, Lemma 1's band: for a non-square [A, B]
    matrix whose normalised singular values are all >= 2e-3 (true for these
    Gaussian / Student-t inputs), RMS(O) * sqrt(max(A, B)) lies in [0.68, 1.21].
Inputs are drawn on the device by the seeded generators (workloads.device_fill)
and copied to the host for the oracle; nothing the oracle receives comes from the
HIP path except, in the multi-step run, the previous step's state.
"""
import math
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import FP32_TOL, assert_ns_close

pytestmark = pytest.mark.gpu

HP = O.OracleHParams()


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
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0))


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def fill_state(torch, dev, wl, w_zero=False, m_std=0.0, step=0):
    ws, ms, gs = [], [], []
    for i, s in enumerate(wl.shapes):
        w = torch.empty(s, dtype=torch.float32, device=dev)
        if w_zero:
            w.zero_()
        else:
            WL.device_fill(w, wl.key, WL.ROLE_W, i, wl.w_std)
        m = torch.empty_like(w)
        WL.device_fill(m, wl.key, WL.ROLE_M, i, m_std)
        g = torch.empty_like(w)
        WL.device_fill(g, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist, step)
        ws.append(w), ms.append(m), gs.append(g)
    return ws, ms, gs


def sample_lines(shape, k=3):
    """Row indices of a flat matrix or column indices of a tall one."""
    n_lines = shape[1] if shape[0] > shape[1] else shape[0]
    return sorted({0, n_lines - 1, *np.random.default_rng(shape[0] * 7 + shape[1]).integers(0, n_lines, k).tolist()})


def take_lines(t, shape, idx):
    return host(t[:, idx]) if shape[0] > shape[1] else host(t[idx, :])


def check_rownorm_lines(w0, m0, g0, w1, m1, shape, tag):
    """Oracle RowNorm step on whole rows (flat) or whole columns (tall)."""
    n = max(shape)
    if shape[0] > shape[1]:
        mm = HP.mu * m0 + g0                                   # [rows, k] columns
        norms = np.sqrt(np.sum(mm * mm, axis=0, keepdims=True))
    else:
        mm = HP.mu * m0 + g0                                   # [k, cols] rows
        norms = np.sqrt(np.sum(mm * mm, axis=1, keepdims=True))
    r = mm / np.maximum(norms, HP.eps)
    w_ref = w0 - HP.lr * (HP.rms_scale * math.sqrt(n) * HP.gamma * r + HP.weight_decay * w0)
    em, ew = rel_fro(m1, mm), rel_fro(w1, w_ref)
    assert em < FP32_TOL, (tag, shape, em)
    assert ew < FP32_TOL, (tag, shape, ew)
    return max(em, ew)


FULL = [WL.DIT_BLOCK_H2048, WL.MIXED_BUCKET_H2048, WL.MMDIT_PAIR_H3072, WL.LAYER_SET_15B_H5120]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: f"key{w.key}")
def test_fullsize_refresh_step(torch_dev, wl):
    """One refresh step over the whole set with W = 0: the update is -lr 0.2 sqrt(n) O."""
    torch, dev = torch_dev
    log(f"refresh step, {wl.name}: {len(wl.shapes)} matrices")
    w, m, g = fill_state(torch, dev, wl, w_zero=True)
    ws = B.make_workspace(wl.shapes, dev)
    B.muon_step(w, m, g, 0, B.default_hparams(period_k=3), ws)
    torch.cuda.synchronize()
    for i in range(len(wl.shapes)):
        assert torch.equal(m[i], g[i])  # M' = 0.95 * 0 + G exactly
    scale = HP.lr * HP.rms_scale
    for i, s in enumerate(wl.shapes):
        if s[0] == s[1]:
            continue
        rms = float(torch.sqrt(torch.mean(w[i].double() ** 2)).item()) / scale  # RMS(O) * sqrt(n)
        assert 0.68 <= rms <= 1.21, (s, rms)
    smallest = min(range(len(wl.shapes)), key=lambda i: wl.shapes[i][0] * wl.shapes[i][1])
    talls = [i for i, s in enumerate(wl.shapes) if s[0] > s[1]]
    picks = [smallest] + ([min(talls, key=lambda i: wl.shapes[i][0])] if talls else [])
    for i in picks:
        s = wl.shapes[i]
        g64 = host(g[i])
        ref = -HP.lr * HP.rms_scale * math.sqrt(max(s)) * O.newton_schulz(g64)
        err, line = assert_ns_close(host(w[i]), ref, s, i)
        log(f"  matrix {i} {s}: update rel err {err:.3e}, worst line {line:.3e}")


@pytest.mark.timeout(900)
def test_fullsize_refresh_15b_largest_matrices(torch_dev):
    """The 15B-scale set's refresh step with W = 0, all ten matrices in one call; its
    largest tall matrix [30720, 5120] (the longest Gram, K = 30720) and its flat
    [5120, 20480] matrix against the oracle's NS5 (about 50 TFLOP of float64 work on
    the host, one matrix at a time)."""
    torch, dev = torch_dev
    wl = WL.LAYER_SET_15B_H5120
    w, m, g = fill_state(torch, dev, wl, w_zero=True)
    ws = B.make_workspace(wl.shapes, dev)
    log(f"refresh step, {wl.name}, W = 0")
    B.muon_step(w, m, g, 0, B.default_hparams(period_k=3), ws)
    torch.cuda.synchronize()
    del ws, m
    for want in ((30720, 5120), (5120, 20480)):
        i = wl.shapes.index(want)
        g64 = host(g[i])
        log(f"  matrix {i} {want}: oracle NS5 on the host")
        ref = -HP.lr * HP.rms_scale * math.sqrt(max(want)) * O.newton_schulz(g64)
        err, line = assert_ns_close(host(w[i]), ref, want, i)
        log(f"  matrix {i} {want}: update rel err {err:.3e}, worst line {line:.3e}")
        del g64, ref


@pytest.mark.parametrize("wl", FULL, ids=lambda w: f"key{w.key}")
def test_fullsize_rownorm_step(torch_dev, wl):
    torch, dev = torch_dev
    log(f"RowNorm step, {wl.name}")
    w, m, g = fill_state(torch, dev, wl, m_std=1e-3)
    lines = [sample_lines(s) for s in wl.shapes]
    before = [(take_lines(w[i], s, lines[i]), take_lines(m[i], s, lines[i]), take_lines(g[i], s, lines[i]))
              for i, s in enumerate(wl.shapes)]
    ws = B.make_workspace(wl.shapes, dev)
    B.muon_step(w, m, g, 1, B.default_hparams(period_k=3), ws)
    torch.cuda.synchronize()
    worst = 0.0
    for i, s in enumerate(wl.shapes):
        w0, m0, g0 = before[i]
        worst = max(worst, check_rownorm_lines(w0, m0, g0, take_lines(w[i], s, lines[i]),
                                               take_lines(m[i], s, lines[i]), s, "rownorm"))
    log(f"  worst sampled-line error {worst:.2e}")


def test_fullsize_periodic_schedule_mixed_bucket(torch_dev):
    """The 16-matrix [2048,8192]/[8192,2048] bucket over 12 steps with K = 3 at full size.

    Every step: M' elementwise on sampled lines. RowNorm steps: W' on sampled lines.
    Refresh steps: the Lemma 1 band on every matrix, and at steps 0 and 9 the oracle's
    NS5 on one flat and one tall matrix, from the state the GPU's earlier steps left
    (teacher forced: the oracle advances that state by one step).
    """
    torch, dev = torch_dev
    wl = WL.MIXED_BUCKET_H2048
    hp = B.default_hparams(period_k=3, gamma=0.15)
    w, m, _ = fill_state(torch, dev, wl)
    m = [torch.zeros_like(x) for x in w]
    ws = B.make_workspace(wl.shapes, dev)
    lines = [sample_lines(s, 2) for s in wl.shapes]
    decay = 1.0 - HP.lr * HP.weight_decay
    for step in range(12):
        g = []
        for i, s in enumerate(wl.shapes):
            t = torch.empty(s, dtype=torch.float32, device=dev)
            WL.device_fill(t, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist, step)
            g.append(t)
        refresh = step % 3 == 0
        before = [(take_lines(w[i], s, lines[i]), take_lines(m[i], s, lines[i]), take_lines(g[i], s, lines[i]))
                  for i, s in enumerate(wl.shapes)]
        full = None
        if step in (0, 9):
            full = {i: (host(w[i]), host(m[i]), host(g[i])) for i in (0, 1)}
        w_prev = [x.clone() for x in w] if refresh else None
        log(f"step {step} ({'refresh' if refresh else 'rownorm'})")
        B.muon_step(w, m, g, step, hp, ws)
        torch.cuda.synchronize()
        for i, s in enumerate(wl.shapes):
            w0, m0, g0 = before[i]
            m1 = take_lines(m[i], s, lines[i])
            assert rel_fro(m1, HP.mu * m0 + g0) < FP32_TOL
            if refresh:
                upd = w[i].double() - decay * w_prev[i].double()
                rms = float(torch.sqrt(torch.mean(upd * upd)).item()) / (HP.lr * HP.rms_scale)
                assert 0.68 <= rms <= 1.21, (step, s, rms)
            else:
                check_rownorm_lines(w0, m0, g0, take_lines(w[i], s, lines[i]), m1, s, f"step {step}")
        if full is not None:
            for i, (w0, m0, g0) in full.items():
                s = wl.shapes[i]
                o = O.newton_schulz(HP.mu * m0 + g0)
                upd_ref = -HP.lr * HP.rms_scale * math.sqrt(max(s)) * o
                err, line = assert_ns_close(host(w[i]) - decay * w0, upd_ref, s, (step, i))
                log(f"  matrix {i} {s}: update rel err {err:.3e}, worst line {line:.3e}")


@pytest.mark.parametrize("wl", [WL.MIXED_BUCKET_H2048, WL.LAYER_SET_15B_H5120], ids=lambda w: f"key{w.key}")
def test_fullsize_eq6_refresh_and_monitor(torch_dev, wl):
    """Eq. 6 refresh over the whole set with W = 0: every matrix's update has RMS exactly
    lr * 0.2, the monitor reads 0.2, and the smallest matrix matches the oracle."""
    torch, dev = torch_dev
    log(f"Eq. 6 refresh step, {wl.name}")
    w, m, g = fill_state(torch, dev, wl, w_zero=True)
    ws = B.make_workspace(wl.shapes, dev)
    rms = torch.zeros(len(wl.shapes), dtype=torch.float32, device=dev)
    B.muon_step(w, m, g, 0, B.default_hparams(period_k=3, scale_mode=B.SCALE_RMS), ws, update_rms=rms)
    torch.cuda.synchronize()
    mon = host(rms)
    for i, s in enumerate(wl.shapes):
        r = float(torch.sqrt(torch.mean(w[i].double() ** 2)).item()) / HP.lr
        assert abs(r - 0.2) < 0.2 * 1e-4, (s, r)
        assert abs(mon[i] - 0.2) < 0.2 * 1e-5, (s, mon[i])
    i = min(range(len(wl.shapes)), key=lambda k: wl.shapes[k][0] * wl.shapes[k][1])
    o = O.newton_schulz(host(g[i]))
    ref = -HP.lr * 0.2 * o / math.sqrt(float(np.mean(o * o)))
    err, line = assert_ns_close(host(w[i]), ref, wl.shapes[i], i)
    log(f"  matrix {i} {wl.shapes[i]}: update rel err {err:.3e}, worst line {line:.3e}")


def test_fullsize_monitor_periodic_cycle_15b(torch_dev):
    """Eq. 4 monitor over a K = 3 cycle of the 15B-scale set: refresh steps read
    0.2 RMS(O) sqrt(max(A, B)), inside Lemma 1's band; RowNorm steps read 0.2 gamma."""
    torch, dev = torch_dev
    wl = WL.LAYER_SET_15B_H5120
    w, m, g = fill_state(torch, dev, wl)
    ws = B.make_workspace(wl.shapes, dev)
    rms = torch.zeros(len(wl.shapes), dtype=torch.float32, device=dev)
    hp = B.default_hparams(period_k=3)
    for step in range(3):
        B.muon_step(w, m, g, step, hp, ws, update_rms=rms)
        torch.cuda.synchronize()
        mon = host(rms)
        log(f"step {step}: monitor {np.round(mon, 5).tolist()}")
        for i, s in enumerate(wl.shapes):
            if step == 0:
                if s[0] != s[1]:
                    assert 0.2 * 0.68 <= mon[i] <= 0.2 * 1.21, (s, mon[i])
            else:
                assert abs(mon[i] - 0.2 * HP.gamma) < 0.2 * HP.gamma * 1e-5, (s, mon[i])
