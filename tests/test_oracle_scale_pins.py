"""Pins of the oracle's update-scale rules and update-RMS monitor.

"Muon is Scalable for LLM Training", Sec. 3.1 (consistent update RMS) lists three
ways to scale the orthogonalised update: Eq. 5 (0.2 sqrt(H), H the hidden size),
Eq. 6 (0.2 O / RMS(O)) and Eq. 7 (0.2 sqrt(max(A, B)), the same as Eq. 4 of
Sec. 2.2). Each rule is pinned here to closed forms the pages and the mathematics
fix, not to a retyped copy of the oracle's formula:

* Lemma 1 (Sec. 2.2): a full-rank matrix with orthonormal rows or columns has RMS
  1 / sqrt(max(A, B)); exact orthonormal factors come from LAPACK's QR here.
* The Sec. 3.1 analysis: for an [H, 4H] matrix, Eq. 4 / Eq. 7 give twice the update
  RMS of Eq. 5, since sqrt(max(H, 4H)) / sqrt(H) = 2; for [H, H] they agree.
* Eq. 6 makes the update RMS exactly 0.2 for any non-zero O.
* RowNorm outputs have unit rows (columns), so their RMS is exact (reading R2).
The monitor value is checked against the RMS recomputed from the step's W output.
"""
import dataclasses
import math

import numpy as np
import pytest

from oracle import muon_oracle as O

HP = O.OracleHParams()


def gaussian(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def orthonormal(shape, seed):
    """An exact (to rounding) matrix with orthonormal rows (flat) or columns (tall)."""
    a, b = shape
    g = gaussian((max(a, b), min(a, b)), seed)
    q, _ = np.linalg.qr(g)              # [max, min], orthonormal columns
    return q if a > b else q.T


def rms_np(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x)))


def hp_with(**kw):
    return dataclasses.replace(HP, **kw)


def update_from_w(w_old, w_new, hp):
    """The scaled direction c U recovered from a step's W output (lambda removed)."""
    return ((1.0 - hp.lr * hp.weight_decay) * np.asarray(w_old) - np.asarray(w_new)) / hp.lr


@pytest.mark.parametrize("shape", [(32, 128), (128, 32), (48, 48)])
def test_lemma1_rms_of_orthonormal_factors(shape):
    q = orthonormal(shape, 1)
    assert abs(O.rms(q) - 1.0 / math.sqrt(max(shape))) < 1e-14


@pytest.mark.parametrize("shape", [(32, 128), (128, 32), (48, 48)])
def test_eq6_on_orthonormal_direction_equals_eq4(shape):
    """Lemma 1: RMS(O) = 1/sqrt(max(A,B)), so Eq. 6's factor is Eq. 4's."""
    q = orthonormal(shape, 2)
    c6 = O.direction_scale(q, shape, "ns5", hp_with(scale_mode="rms"))
    c4 = O.direction_scale(q, shape, "ns5", HP)
    assert abs(c4 - 0.2 * math.sqrt(max(shape))) < 1e-12
    assert abs(c6 / c4 - 1.0) < 1e-12


def test_eq5_vs_eq4_on_h_by_4h_and_h_by_h():
    """Sec. 3.1 analysis: sqrt(max(H, 4H)) / sqrt(H) = 2 for the MLP, 1 for attention q."""
    h = 32
    for shape, ratio in (((h, 4 * h), 2.0), ((h, h), 1.0), ((4 * h, h), 2.0)):
        q = orthonormal(shape, 3)
        u4 = O.direction_scale(q, shape, "ns5", HP) * O.rms(q)
        u5 = O.direction_scale(q, shape, "ns5", hp_with(scale_mode="hidden", hidden=h)) * O.rms(q)
        assert abs(u4 - 0.2) < 1e-12            # Eq. 4 makes every shape 0.2 (Lemma 1)
        assert abs(u4 / u5 - ratio) < 1e-12


def test_eq5_with_hidden_equal_to_max_dim_is_eq4():
    """Sec. 3.1: for most matrices max(A, B) equals H, and then Eq. 5 is Eq. 4."""
    for shape in ((64, 256), (256, 64)):
        w, m, g = gaussian(shape, 4, 0.02), gaussian(shape, 5, 0.02), gaussian(shape, 6, 1e-3)
        hp5 = hp_with(scale_mode="hidden", hidden=max(shape))
        for step in (0, 1):
            a = O.muon_step(w, m, g, step, HP)[0]
            b = O.muon_step(w, m, g, step, hp5)[0]
            assert np.array_equal(a, b)


@pytest.mark.parametrize("shape", [(64, 256), (256, 64), (96, 96)])
def test_eq6_refresh_update_rms_is_exactly_point_two(shape):
    """W = 0 probe: the Eq. 6 update is -lr 0.2 O / RMS(O), RMS exactly lr * 0.2,
    and its direction is that of the SVD closed form of NS5 (not the oracle's loop)."""
    hp6 = hp_with(scale_mode="rms")
    m = gaussian(shape, 7)
    w_new, _ = O.vanilla_step(np.zeros(shape), np.zeros(shape), m, hp6)
    assert abs(rms_np(w_new) / hp6.lr - 0.2) < 1e-12
    x = m.T if shape[0] > shape[1] else m
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    fx = s / math.sqrt(float(np.sum(s * s)))
    for _ in range(5):
        fx = HP.ns_a * fx + HP.ns_b * fx ** 3 + HP.ns_c * fx ** 5
    o = (u * fx) @ vt
    o = o.T if shape[0] > shape[1] else o
    ref = -hp6.lr * 0.2 * o / rms_np(o)
    assert np.linalg.norm(w_new - ref) / np.linalg.norm(ref) < 1e-10


def test_eq6_zero_momentum_gives_pure_decay():
    """R14: division by max(RMS(O), eps): a zero direction leaves only weight decay."""
    shape = (32, 96)
    w = gaussian(shape, 8, 0.02)
    w_new, m = O.vanilla_step(w, np.zeros(shape), np.zeros(shape), hp_with(scale_mode="rms"))
    assert np.all(np.isfinite(w_new))
    assert np.array_equal(w_new, w - HP.lr * (0.0 + HP.weight_decay * w))


def test_eq6_rownorm_step_is_eq4_rownorm_step():
    """R15: on RowNorm steps Eq. 6 uses the exact RMS of R, i.e. Eq. 4's factor."""
    for shape in ((64, 256), (256, 64)):
        w, m, g = gaussian(shape, 9, 0.02), gaussian(shape, 10, 0.02), gaussian(shape, 11, 1e-3)
        a = O.rownorm_step(w, m, g, HP)[0]
        b = O.rownorm_step(w, m, g, hp_with(scale_mode="rms"))[0]
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["max_dim", "hidden", "rms"])
@pytest.mark.parametrize("step", [0, 1])
@pytest.mark.parametrize("shape", [(64, 256), (256, 64)])
def test_monitor_equals_rms_of_the_applied_update(mode, step, shape):
    hp = hp_with(scale_mode=mode, hidden=128)
    w, m, g = gaussian(shape, 12, 0.02), gaussian(shape, 13, 0.02), gaussian(shape, 14, 1e-3)
    w_new, _, mon = O.muon_step_monitored(w, m, g, step, hp)
    assert abs(mon / rms_np(update_from_w(w, w_new, hp)) - 1.0) < 1e-9


@pytest.mark.parametrize("shape", [(64, 256), (256, 64), (80, 80)])
def test_monitor_rownorm_closed_form(shape):
    """Unit lines: RMS(R) = 1/sqrt(max(A, B)) exactly, so the monitor reads 0.2 gamma."""
    w, m, g = gaussian(shape, 15, 0.02), gaussian(shape, 16, 0.02), gaussian(shape, 17, 1e-3)
    for mode in ("max_dim", "rms"):
        _, _, mon = O.muon_step_monitored(w, m, g, 1, hp_with(scale_mode=mode))
        assert abs(mon - 0.2 * HP.gamma) < 1e-12
    _, _, mon5 = O.muon_step_monitored(w, m, g, 1, hp_with(scale_mode="hidden", hidden=64))
    assert abs(mon5 - 0.2 * HP.gamma * math.sqrt(64 / max(shape))) < 1e-12


def test_monitor_refresh_in_lemma1_band():
    """Full-rank Gaussian input: NS5's singular values lie in about [0.68, 1.21], so the
    Eq. 4 monitor, 0.2 RMS(O) sqrt(max(A, B)), lies in [0.2 * 0.68, 0.2 * 1.21]."""
    for shape in ((64, 256), (256, 64), (128, 128)):
        m = gaussian(shape, 18)
        _, _, mon = O.muon_step_monitored(np.zeros(shape), np.zeros(shape), m, 0, HP)
        assert 0.2 * 0.68 <= mon <= 0.2 * 1.21, (shape, mon)


def test_scale_rule_argument_checks():
    with pytest.raises(ValueError):
        O.direction_scale(np.ones((2, 3)), (2, 3), "ns5", hp_with(scale_mode="hidden", hidden=0))
    with pytest.raises(ValueError):
        O.direction_scale(np.ones((2, 3)), (2, 3), "ns5", hp_with(scale_mode="unknown"))


def _mutant_scale(kind_of_mistake):
    def f(u, shape, kind, hp):
        if kind_of_mistake == "eq5_uses_max_dim" and hp.scale_mode == "hidden":
            return hp.rms_scale * math.sqrt(max(shape))
        if kind_of_mistake == "eq6_uses_fro" and hp.scale_mode == "rms" and kind == "ns5":
            return hp.rms_scale / max(float(np.linalg.norm(u)), hp.eps)
        if kind_of_mistake == "eq6_on_rownorm_measured" and hp.scale_mode == "rms" and kind == "rownorm":
            return hp.rms_scale / max(O.rms(u), hp.eps)
        return _ORIG_SCALE(u, shape, kind, hp)
    return f


_ORIG_SCALE = O.direction_scale


@pytest.mark.parametrize("mistake", ["eq5_uses_max_dim", "eq6_uses_fro", "eq6_on_rownorm_measured"])
def test_pins_reject_planted_scale_mistakes(mistake, monkeypatch):
    monkeypatch.setattr(O, "direction_scale", _mutant_scale(mistake))
    pins = [test_eq5_vs_eq4_on_h_by_4h_and_h_by_h,
            lambda: test_eq6_refresh_update_rms_is_exactly_point_two((64, 256)),
            test_eq6_rownorm_step_is_eq4_rownorm_step,
            lambda: test_monitor_rownorm_closed_form((64, 256))]
    failures = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, mistake
