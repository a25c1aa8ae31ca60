"""Pins of the AdamW oracle (the hybrid optimizer's companion for non-matrix parameters).

The pages name AdamW without restating it, so the oracle is pinned to what fixes it
independently:
* torch.optim.AdamW run in float64 on the CPU: a library implementation of the same
  algorithm (decoupled weight decay, bias-corrected moments);
* closed forms: the first step from zero state moves each element by
  lr * g / (|g| + eps); under a constant gradient the bias-corrected moments are
  exactly g and g^2 at every step, so W follows a scalar recursion;
* zero gradients leave pure weight decay;
* the parameter-group rule of "Scaling Muon for Diffusion Transformers" (setup
  paragraph) on named shapes.
Planted mistakes (no bias correction, eps under the square root, weight decay
coupled into the gradient) are rejected.
"""
import dataclasses

import numpy as np
import pytest

from oracle import adamw_oracle as A

HP = A.AdamWHParams()


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def torch_adamw_reference(w0, grads, hp):
    import torch
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay)
    out = []
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        out.append(p.detach().numpy().copy())
    return out


def run_oracle(w0, grads, hp, step_fn=None):
    step_fn = step_fn or A.adamw_step
    w, m, v = np.asarray(w0, np.float64), np.zeros_like(w0), np.zeros_like(w0)
    out = []
    for s, g in enumerate(grads):
        w, m, v = step_fn(w, g, m, v, s, hp)
        out.append(w)
    return out


@pytest.mark.parametrize("hp", [HP, A.AdamWHParams(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0)])
def test_matches_torch_adamw_float64(hp):
    w0 = rnd((7, 33), 1, 0.02)
    grads = [rnd((7, 33), 10 + s, 1e-3) for s in range(6)]
    ref = torch_adamw_reference(w0, grads, hp)
    got = run_oracle(w0, grads, hp)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) < 1e-15 + 1e-12 * np.max(np.abs(b))


def test_first_step_closed_form():
    w0, g = rnd((50,), 2, 0.02), rnd((50,), 3, 1e-3)
    w1, m1, v1 = A.adamw_step(w0, g, np.zeros(50), np.zeros(50), 0, HP)
    expect = w0 - HP.lr * (g / (np.abs(g) + HP.eps) + HP.weight_decay * w0)
    assert np.allclose(w1, expect, rtol=0, atol=1e-18)
    assert np.allclose(m1, (1 - HP.beta1) * g) and np.allclose(v1, (1 - HP.beta2) * g * g)
    # |g| >> eps: every element moves by about lr (Adam's sign-like first step)
    assert abs(A.update_rms(w0, w1, HP) - 1.0) < 1e-4


def test_constant_gradient_scalar_recursion():
    w0, g = rnd((40,), 4, 0.02), rnd((40,), 5, 1e-3)
    steps = 25
    w, m, v = w0.copy(), np.zeros(40), np.zeros(40)
    for s in range(steps):
        w, m, v = A.adamw_step(w, g, m, v, s, HP)
    u = g / (np.abs(g) + HP.eps)
    d = 1.0 - HP.lr * HP.weight_decay
    expect = d ** steps * w0 - HP.lr * u * sum(d ** k for k in range(steps))
    assert np.max(np.abs(w - expect)) < 1e-15


def test_zero_gradient_is_pure_decay():
    w0 = rnd((3, 4), 6, 0.02)
    w1, m1, v1 = A.adamw_step(w0, np.zeros((3, 4)), np.zeros((3, 4)), np.zeros((3, 4)), 4, HP)
    assert np.array_equal(m1, np.zeros((3, 4))) and np.array_equal(v1, np.zeros((3, 4)))
    assert np.allclose(w1, w0 * (1 - HP.lr * HP.weight_decay), rtol=1e-15, atol=0)


def test_step_argument():
    with pytest.raises(ValueError):
        A.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), -1, HP)


def test_parameter_group_rule():
    """[DiT] setup: 2-D weights inside transformer blocks go to Muon; biases,
    normalisation weights and everything outside the blocks go to AdamW."""
    cases = [("blocks.0.img.attn.qkv.weight", (3072, 1024), True),
             ("blocks.3.txt.mlp.down.weight", (1024, 4096), True),
             ("blocks.0.img.attn.qkv.bias", (3072,), False),
             ("blocks.0.img.attn.q_norm.weight", (64,), False),
             ("x_embedder.weight", (1024, 64), False),
             ("final_layer.linear.weight", (64, 1024), False),
             ("pos_embed", (1, 4096, 1024), False)]
    for name, shape, muon in cases:
        assert A.goes_to_muon(name, shape) is muon, name


def _no_bias_correction(w, g, m, v, step, hp):
    w, g, m, v = (np.asarray(x, dtype=np.float64) for x in (w, g, m, v))
    m = hp.beta1 * m + (1 - hp.beta1) * g
    v = hp.beta2 * v + (1 - hp.beta2) * g * g
    return w - hp.lr * (m / (np.sqrt(v) + hp.eps) + hp.weight_decay * w), m, v


def _eps_inside_sqrt(w, g, m, v, step, hp):
    w, g, m, v = (np.asarray(x, dtype=np.float64) for x in (w, g, m, v))
    t = step + 1
    m = hp.beta1 * m + (1 - hp.beta1) * g
    v = hp.beta2 * v + (1 - hp.beta2) * g * g
    mh, vh = m / (1 - hp.beta1 ** t), v / (1 - hp.beta2 ** t)
    return w - hp.lr * (mh / np.sqrt(vh + hp.eps) + hp.weight_decay * w), m, v


def _coupled_decay(w, g, m, v, step, hp):
    g = np.asarray(g, np.float64) + hp.weight_decay * np.asarray(w, np.float64)
    return A.adamw_step(w, g, m, v, step, dataclasses.replace(hp, weight_decay=0.0))


@pytest.mark.parametrize("mutant", [_no_bias_correction, _eps_inside_sqrt, _coupled_decay])
def test_torch_pin_rejects_planted_mistakes(mutant):
    w0 = rnd((7, 33), 1, 0.02)
    grads = [rnd((7, 33), 10 + s, 1e-3) for s in range(6)]
    ref = torch_adamw_reference(w0, grads, HP)
    got = run_oracle(w0, grads, HP, mutant)
    assert max(np.max(np.abs(a - b)) for a, b in zip(got, ref)) > 1e-9
