"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (relative Frobenius error):
  * Newton-Schulz output, and the refresh-step update recovered with W = 0:
    2e-2. The GEMMs take bf16 operands (8-bit mantissa, unit roundoff 2^-9) with
    fp32 accumulation; five iterations of three products accumulate to about 1%.
    Every line of the output (row of a flat matrix, column of a tall one) is also
    held to a per-line bound, 6e-2 at the workloads' sizes, so that one wrong row
    cannot hide in the whole-matrix error. Inputs with min(A, B) < 64 get the wider
    bands of tolerances.py, set from a sweep of the CPU emulation of the same bf16
    recipe against the oracle.
  * Momentum, the RowNorm step's W and its update (W = 0 probe): 1e-5. These are
    fp32 element-wise maps plus fp32 tree reductions (error ~ log2(n) * 2^-24).
Inputs are seeded (matrix_orthogonalising_optimizer_02_amd.workloads); nothing
the oracle sees comes from the HIP path except, in the teacher-forced multi-step
runs, the previous step's state, which both sides then advance by one step.
"""
import math
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import FP32_TOL, NS_TOL, assert_ns_close

pytestmark = pytest.mark.gpu

HP = O.OracleHParams()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()  # raises when the HIP library is missing: no fallback
    return torch, torch.device("cuda:0")


def to_dev(torch, dev, x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def to_host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def gauss(key, idx, shape, std=1.0, step=0):
    return WL.host_normal(key, WL.ROLE_G, idx, shape, std, step)


# ------------------------------------------------------------------ NS5 ----

NS_SHAPES = [(128, 512), (512, 128), (1, 7), (7, 1), (2, 2), (33, 77), (77, 33), (300, 700),
             (700, 300), (256, 256), (257, 513), (129, 1000), (1000, 129), (64, 64)]


def test_ns5_batched_small_and_ragged_vs_oracle(torch_dev):
    torch, dev = torch_dev
    xs = [gauss(100, i, s) for i, s in enumerate(NS_SHAPES)]
    log(f"ns5_batched: {len(xs)} matrices {NS_SHAPES}")
    outs = B.ns5_batched([to_dev(torch, dev, x) for x in xs])
    torch.cuda.synchronize()
    for s, x, o in zip(NS_SHAPES, xs, outs):
        err, line = assert_ns_close(to_host(o), O.newton_schulz(x), s)
        log(f"  {s}: rel err {err:.3e}, worst line {line:.3e}")


def test_ns5_more_than_one_group_and_mixed_m(torch_dev):
    torch, dev = torch_dev
    shapes = [(96 + 32 * (i % 5), 160 + 64 * (i % 3)) if i % 2 == 0 else (200 + 16 * i, 90 + 8 * (i % 4))
              for i in range(21)]
    xs = [gauss(101, i, s) for i, s in enumerate(shapes)]
    log(f"ns5_batched: {len(xs)} matrices in several groups")
    outs = B.ns5_batched([to_dev(torch, dev, x) for x in xs])
    torch.cuda.synchronize()
    errs = [assert_ns_close(to_host(o), O.newton_schulz(x), s) for s, x, o in zip(shapes, xs, outs)]
    log(f"  max rel err {max(e[0] for e in errs):.3e}, worst line {max(e[1] for e in errs):.3e}")


def test_ns5_apply_on_one_round_of_big_tiles(torch_dev):
    """Three [2048, 2048] matrices: 192 big Apply tiles (24 per XCD, one round) against 768
    small ones (96 per XCD, two rounds), so the Apply runs on 256-wide tiles, the Gram
    and polynomial on 128-wide ones. Against the oracle at the bf16 tolerance; and equal
    bit for bit to the same matrix alone (192 / 3 = 64 big tiles, 256 small ones: 8 and
    32 per XCD, so it stays on 128-wide tiles), since both tiles accumulate over K in the
    same order."""
    torch, dev = torch_dev
    shapes = [(2048, 2048)] * 3
    xs = [gauss(104, i, s) for i, s in enumerate(shapes)]
    outs = B.ns5_batched([to_dev(torch, dev, x) for x in xs])
    alone = B.ns5_batched([to_dev(torch, dev, xs[2])])
    torch.cuda.synchronize()
    assert torch.equal(outs[2], alone[0])
    for i in (0, 2):
        err, line = assert_ns_close(to_host(outs[i]), O.newton_schulz(xs[i]), shapes[i], i)
        log(f"  three [2048, 2048], matrix {i}: rel err {err:.3e}, worst line {line:.3e}")


def test_ns5_stages_on_big_tiles_by_rounds(torch_dev):
    """Five [2304, 2304] matrices: the Gram and polynomial need one round of 256-wide
    tiles (25 to 30 upper tiles per XCD) against two of 128-wide ones (105 to 110), the
    Apply two rounds (50 to 55 tiles) against four (200 to 205), so all three stages run
    on 256-wide tiles; no XCD's last round is short enough to be split. One such matrix
    alone (at most 6, 22, 11 and 41 tiles per XCD: one round either way) keeps 128-wide
    tiles. The outputs are equal bit for bit, as both tiles accumulate over K in the same
    order, and match the oracle."""
    torch, dev = torch_dev
    shapes = [(2304, 2304)] * 5
    xs = [gauss(105, i, s) for i, s in enumerate(shapes)]
    outs = B.ns5_batched([to_dev(torch, dev, x) for x in xs])
    alone = B.ns5_batched([to_dev(torch, dev, xs[4])])
    torch.cuda.synchronize()
    assert torch.equal(outs[4], alone[0])
    err, line = assert_ns_close(to_host(outs[4]), O.newton_schulz(xs[4]), shapes[4])
    log(f"  five [2304, 2304], matrix 4: rel err {err:.3e}, worst line {line:.3e}")


def test_ns5_wide_cast_tiles_ragged_tall(torch_dev):
    """Three [8450, 2046] matrices and one [8450, 2048]: 144 upper tiles of 256, so the
    Gram reads X_c alone and the cast writes no transposed copy; it then takes its wide
    16 x 256 tiles, here with ragged rows (8450 of 8704) and, for the first three,
    columns that are not a multiple of 4 (2046: the element-wise path; the padded
    columns of X_c must be zeros). The first and last matrix against the oracle."""
    torch, dev = torch_dev
    shapes = [(8450, 2046)] * 3 + [(8450, 2048)]
    plan = B.ns5_plan(shapes)
    assert len(plan) == 1 and plan[0]["gram"][0] == 256
    xs = [gauss(111, i, s) for i, s in enumerate(shapes)]
    log(f"ns5_batched: {shapes}")
    outs = B.ns5_batched([to_dev(torch, dev, x) for x in xs])
    torch.cuda.synchronize()
    for i in (0, 3):
        err, line = assert_ns_close(to_host(outs[i]), O.newton_schulz(xs[i]), shapes[i], i)
        log(f"  matrix {i} {shapes[i]}: rel err {err:.3e}, worst line {line:.3e}")


def test_ns5_in_place_zero_and_degenerate(torch_dev):
    torch, dev = torch_dev
    x = gauss(102, 0, (300, 200))
    t = to_dev(torch, dev, x)
    log("ns5_batched in place")
    B.ns5_batched([t], [t])
    torch.cuda.synchronize()
    assert_ns_close(to_host(t), O.newton_schulz(x), x.shape)
    z = torch.zeros(70, 90, device=dev)
    log("ns5_batched zero matrix and rank-one row")
    (oz,) = B.ns5_batched([z])
    torch.cuda.synchronize()
    assert torch.count_nonzero(oz).item() == 0
    r = gauss(102, 1, (1, 4099))
    (orow,) = B.ns5_batched([to_dev(torch, dev, r)])
    torch.cuda.synchronize()
    assert_ns_close(to_host(orow), O.newton_schulz(r), r.shape)


@pytest.mark.parametrize("steps", [1, 2, 10])
def test_ns5_iteration_count(torch_dev, steps):
    """N = 10 ("Muon is Scalable", Sec. 2.2 other hyper-parameters) as well as 5.

    Every iteration rounds X, A and B to bf16 again and the polynomial map does not
    contract those errors (its iterates oscillate around 1), so the error grows about
    linearly with N: the bound is 2e-2 * max(1, N / 5).
    """
    torch, dev = torch_dev
    x = gauss(103, steps, (160, 480))
    hp = B.default_hparams(ns_steps=steps)
    log(f"ns5_batched ns_steps={steps}")
    (o,) = B.ns5_batched([to_dev(torch, dev, x)], hp=hp)
    torch.cuda.synchronize()
    err, line = assert_ns_close(to_host(o), O.newton_schulz(x, steps=steps), x.shape, scale=max(1.0, steps / 5))
    log(f"  rel err {err:.3e}, worst line {line:.3e}")


# --------------------------------------------------------- vanilla step ----

def test_vanilla_step_single_128x512(torch_dev):
    """One vanilla step on the 128x512 workload: M' at 1e-5, the update at 2e-2."""
    torch, dev = torch_dev
    wl = WL.SINGLE_128x512
    w, mp, g = WL.host_inputs(wl, 0)
    hp = B.default_hparams(period_k=1)
    w_ref, m_ref = O.muon_step(w, mp, g, 0, HP)
    # real W
    wt, mt, gt = (to_dev(torch, dev, a) for a in (w, mp, g))
    log("muon_step vanilla 128x512")
    B.muon_step([wt], [mt], [gt], 0, hp)
    torch.cuda.synchronize()
    assert rel_fro(to_host(mt), m_ref) < FP32_TOL
    decay = 1.0 - HP.lr * HP.weight_decay
    upd_gpu = to_host(wt) - decay * w.astype(np.float64)
    upd_ref = w_ref - decay * w.astype(np.float64)
    err, line = assert_ns_close(upd_gpu, upd_ref, w.shape)
    log(f"  update rel err {err:.3e}, worst line {line:.3e}")
    # W = 0 probe isolates the update exactly
    w0, mt, gt = (to_dev(torch, dev, a) for a in (np.zeros_like(w), mp, g))
    B.muon_step([w0], [mt], [gt], 0, hp)
    torch.cuda.synchronize()
    w0_ref, _ = O.muon_step(np.zeros_like(w), mp, g, 0, HP)
    assert_ns_close(to_host(w0), w0_ref, w.shape)


def test_vanilla_step_mixed_shapes_w0_probe(torch_dev):
    torch, dev = torch_dev
    shapes = [(130, 520), (520, 130), (200, 200), (1, 64), (64, 1), (45, 300)]
    mps = [gauss(104, i, s, 0.02) for i, s in enumerate(shapes)]
    gs = [gauss(105, i, s, 0.02) for i, s in enumerate(shapes)]
    ws = [torch.zeros(s, device=dev) for s in shapes]
    ms = [to_dev(torch, dev, a) for a in mps]
    log("muon_step vanilla mixed shapes, W = 0")
    B.muon_step(ws, ms, [to_dev(torch, dev, a) for a in gs], 0, B.default_hparams(period_k=1))
    torch.cuda.synchronize()
    for s, w, m, mp, g in zip(shapes, ws, ms, mps, gs):
        w_ref, m_ref = O.muon_step(np.zeros(s), mp, g, 0, HP)
        assert rel_fro(to_host(m), m_ref) < FP32_TOL
        err, line = assert_ns_close(to_host(w), w_ref, s)
        log(f"  {s}: update rel err {err:.3e}, worst line {line:.3e}")


# -------------------------------------------------------------- RowNorm ----

# flat rows up to 8192 floats take 256-thread blocks, longer ones up to 32768 (a multiple
# of 4) 1024-thread blocks (9000, 20480, 24000, 32768 here), longer still the re-reading
# kernel (40000)
RN_SHAPES = [(128, 512), (512, 128), (256, 256), (33, 77), (77, 33), (1, 4096), (4096, 1),
             (3, 40000), (300, 2048), (2048, 300), (64, 20480), (20480, 64), (5, 1023), (1023, 5),
             (700, 257), (11, 9000), (6, 24000), (9, 32768)]


@pytest.mark.parametrize("entry", ["rownorm_update", "muon_step"])
def test_rownorm_step_vs_oracle(torch_dev, entry):
    torch, dev = torch_dev
    hp = B.default_hparams()
    ws_h = [WL.host_normal(106, 0, i, s, 0.02) for i, s in enumerate(RN_SHAPES)]
    mp_h = [WL.host_normal(106, 1, i, s, 0.02) for i, s in enumerate(RN_SHAPES)]
    g_h = [WL.host_normal(106, 2, i, s, 1e-3) for i, s in enumerate(RN_SHAPES)]
    for probe in (False, True):
        w_in = [np.zeros(s, np.float32) if probe else a for s, a in zip(RN_SHAPES, ws_h)]
        wt = [to_dev(torch, dev, a) for a in w_in]
        mt = [to_dev(torch, dev, a) for a in mp_h]
        gt = [to_dev(torch, dev, a) for a in g_h]
        log(f"{entry} RowNorm step, W = 0 probe: {probe}")
        if entry == "rownorm_update":
            B.rownorm_update(wt, mt, gt, hp)
        else:
            B.muon_step(wt, mt, gt, 4, hp)  # 4 % 3 != 0: a RowNorm step
        torch.cuda.synchronize()
        for s, w, m, a, mp, g in zip(RN_SHAPES, wt, mt, w_in, mp_h, g_h):
            w_ref, m_ref = O.rownorm_step(a, mp, g, HP)
            em, ew = rel_fro(to_host(m), m_ref), rel_fro(to_host(w), w_ref)
            assert em < FP32_TOL, (s, em)
            assert ew < FP32_TOL, (s, probe, ew)


def test_rownorm_zero_lines_and_gamma(torch_dev):
    torch, dev = torch_dev
    for shape in [(40, 96), (96, 40)]:
        g = gauss(107, 0, shape, 1e-3)
        if shape[0] < shape[1]:
            g[5, :] = 0.0
        else:
            g[:, 7] = 0.0
        for gamma in (0.15, 1.0):
            hp = B.default_hparams(gamma=gamma)
            w = torch.zeros(shape, device=dev)
            m = torch.zeros(shape, device=dev)
            log(f"rownorm zero line {shape} gamma={gamma}")
            B.rownorm_update([w], [m], [to_dev(torch, dev, g)], hp)
            torch.cuda.synchronize()
            ref, _ = O.rownorm_step(np.zeros(shape), np.zeros(shape), g, O.OracleHParams(gamma=gamma))
            assert rel_fro(to_host(w), ref) < FP32_TOL
            out = to_host(w)
            assert np.all(out[5, :] == 0.0) if shape[0] < shape[1] else np.all(out[:, 7] == 0.0)


# ----------------------------------------------------- multi-step Periodic ----

def test_periodic_twelve_steps_reduced_bucket(torch_dev):
    """The mixed flat/tall bucket at reduced size, 12 steps with K = 3, teacher forced."""
    torch, dev = torch_dev
    shapes = [(256, 1024) if i % 2 == 0 else (1024, 256) for i in range(16)]
    hp = B.default_hparams(period_k=3, gamma=0.15)
    w = [to_dev(torch, dev, WL.host_normal(108, 0, i, s, 0.02)) for i, s in enumerate(shapes)]
    m = [torch.zeros(s, device=dev) for s in shapes]
    ws = B.make_workspace(shapes, dev)
    decay = 1.0 - HP.lr * HP.weight_decay
    for step in range(12):
        g_h = [WL.host_normal(108, 2, i, s, 1e-3, step) for i, s in enumerate(shapes)]
        w_prev = [to_host(x) for x in w]
        m_prev = [to_host(x) for x in m]
        log(f"periodic step {step} ({'refresh' if step % 3 == 0 else 'rownorm'})")
        B.muon_step(w, m, [to_dev(torch, dev, a) for a in g_h], step, hp, ws)
        torch.cuda.synchronize()
        worst_w = worst_m = 0.0
        for i in range(16):
            w_ref, m_ref = O.muon_step(w_prev[i], m_prev[i], g_h[i], step, HP)
            worst_m = max(worst_m, rel_fro(to_host(m[i]), m_ref))
            if step % 3 == 0:
                worst_w = max(worst_w, assert_ns_close(to_host(w[i]) - decay * w_prev[i], w_ref - decay * w_prev[i],
                                                       shapes[i], f"step {step}")[0])
            else:
                worst_w = max(worst_w, rel_fro(to_host(w[i]), w_ref))
        log(f"  M' {worst_m:.2e}  {'update' if step % 3 == 0 else 'W'} {worst_w:.2e}")
        assert worst_m < FP32_TOL
        assert worst_w < (NS_TOL if step % 3 == 0 else FP32_TOL)


def test_k1_is_vanilla_bitwise_and_deterministic(torch_dev):
    torch, dev = torch_dev
    shapes = [(200, 600), (600, 200), (128, 128)]
    w0 = [WL.host_normal(109, 0, i, s, 0.02) for i, s in enumerate(shapes)]
    m0 = [WL.host_normal(109, 1, i, s, 0.02) for i, s in enumerate(shapes)]
    g0 = [WL.host_normal(109, 2, i, s, 1e-3) for i, s in enumerate(shapes)]

    def run(step, k):
        w = [to_dev(torch, dev, a) for a in w0]
        m = [to_dev(torch, dev, a) for a in m0]
        B.muon_step(w, m, [to_dev(torch, dev, a) for a in g0], step, B.default_hparams(period_k=k))
        torch.cuda.synchronize()
        return [to_host(x) for x in w + m]

    log("K = 1 vs refresh step, repeat runs")
    ref = run(0, 3)
    for step in (1, 2, 5):
        out = run(step, 1)
        assert all(np.array_equal(a, b) for a, b in zip(out, ref))
    assert all(np.array_equal(a, b) for a, b in zip(run(0, 3), ref))
    rn1, rn2 = run(1, 3), run(1, 3)
    assert all(np.array_equal(a, b) for a, b in zip(rn1, rn2))


def test_resume_is_bitwise(torch_dev):
    torch, dev = torch_dev
    shapes = [(96, 320), (320, 96)]
    grads = [[to_dev(torch, dev, WL.host_normal(110, 2, i, s, 1e-3, t)) for i, s in enumerate(shapes)]
             for t in range(12)]

    def fresh():
        return [to_dev(torch, dev, WL.host_normal(110, 0, i, s, 0.02)) for i, s in enumerate(shapes)]

    log("resume: 12 straight steps vs 6 + save/load + 6")
    p1 = fresh()
    opt1 = B.MuonOptimizer(p1)
    for t in range(12):
        opt1.step(grads[t])
    p2 = fresh()
    opt2 = B.MuonOptimizer(p2)
    for t in range(6):
        opt2.step(grads[t])
    state = opt2.state_dict()
    saved_w = [x.clone() for x in p2]
    p3 = [x.clone() for x in saved_w]
    opt3 = B.MuonOptimizer(p3)
    opt3.load_state_dict(state)
    for t in range(6, 12):
        opt3.step(grads[t])
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(p1, p3))
    assert all(torch.equal(a, b) for a, b in zip(opt1.momenta, opt3.momenta))


def test_nan_propagates_and_stays_local(torch_dev):
    torch, dev = torch_dev
    shapes = [(64, 256), (256, 64)]
    for step in (0, 1):
        w = [torch.zeros(s, device=dev) for s in shapes]
        m = [torch.zeros(s, device=dev) for s in shapes]
        g = [to_dev(torch, dev, gauss(111, i, s, 1e-3)) for i, s in enumerate(shapes)]
        g[0][3, 5] = float("nan")
        log(f"NaN propagation, step {step}")
        B.muon_step(w, m, g, step, B.default_hparams())
        torch.cuda.synchronize()
        assert torch.isnan(w[0]).any().item()
        assert torch.isfinite(w[1]).all().item() and torch.isfinite(m[1]).all().item()
        if step == 1:  # RowNorm of a flat matrix: only row 3 is touched
            assert torch.isnan(w[0][3]).all().item()
            assert torch.isfinite(w[0][:3]).all().item() and torch.isfinite(w[0][4:]).all().item()
