"""Seeded synthetic workloads: matrix shapes and input distributions.

This module holds no arithmetic of the optimizer itself. It only names the
matrix sets the optimizer is exercised on and draws seeded random inputs for
them, so that the HIP path and the float64 oracle see identical arrays.

Shapes follow the diffusion-transformer blocks of "Scaling Muon for Diffusion
Transformers" (dual-stream MMDiT with Muon on the 2-D block weights): at hidden
size H, qkv [3H, H], output projection [H, H], MLP up [4H, H] and down [H, 4H],
adaLN modulation [6H, H]. Distributions: weights N(0, 0.02^2), gradients
N(0, 1e-3^2) or 1e-3 * Student-t(3) (heavy-tailed), initial momentum 0.

Host draws use numpy's PCG64 seeded with SeedSequence([config, role, matrix,
step]) so any single matrix can be regenerated independently; role 0 = W,
1 = previous momentum, 2 = gradient. Device draws (used only where the CPU
would take too long to fill several GB) use a seeded torch generator on the
GPU and are never compared against the oracle element by element.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

ROLE_W, ROLE_M, ROLE_G = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named set of [rows, cols] fp32 matrices and how their inputs are drawn."""

    key: int                       # seed component identifying the workload
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    w_std: float = 0.02
    g_std: float = 1e-3
    g_dist: str = "normal"         # "normal" or "t3" (1e-3 * Student-t, nu = 3)
    m0_std: float = 0.0            # previous momentum std (0 -> zeros)
    steps: int = 1
    period_k: int = 1

    @property
    def elements(self) -> int:
        return sum(a * b for a, b in self.shapes)


def dit_block_shapes(h: int) -> List[Tuple[int, int]]:
    """qkv, out-proj, MLP up, MLP down, adaLN modulation of one DiT stream at hidden size h."""
    return [(3 * h, h), (h, h), (4 * h, h), (h, 4 * h), (6 * h, h)]


SINGLE_128x512 = Workload(
    key=1, name="single 128x512, one vanilla step",
    shapes=((128, 512),), w_std=0.02, g_std=0.02, m0_std=0.02, steps=1, period_k=1)

DIT_BLOCK_H2048 = Workload(
    key=2, name="DiT block H=2048 (qkv, out, up, down, adaLN), one vanilla step",
    shapes=tuple(dit_block_shapes(2048)), steps=1, period_k=1)

MIXED_BUCKET_H2048 = Workload(
    key=3, name="16-matrix bucket, even [2048,8192] / odd [8192,2048], 12 steps K=3",
    shapes=tuple((2048, 8192) if i % 2 == 0 else (8192, 2048) for i in range(16)),
    steps=12, period_k=3)

MMDIT_PAIR_H3072 = Workload(
    key=4, name="dual-stream MMDiT block pair H=3072, 6 steps K=3",
    shapes=tuple(dit_block_shapes(3072) * 2), steps=6, period_k=3)

LAYER_SET_15B_H5120 = Workload(
    key=5, name="15B-scale layer set H=5120, both streams, t3 gradients, K=3",
    shapes=tuple(dit_block_shapes(5120) * 2), g_dist="t3", steps=3, period_k=3)

WORKLOADS = (SINGLE_128x512, DIT_BLOCK_H2048, MIXED_BUCKET_H2048,
             MMDIT_PAIR_H3072, LAYER_SET_15B_H5120)


def rng(key: int, role: int, index: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, role, index, step])))


def host_normal(key: int, role: int, index: int, shape: Sequence[int], std: float,
                step: int = 0) -> np.ndarray:
    """float32 array of N(0, std^2) drawn in float64 then rounded."""
    if std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    return (rng(key, role, index, step).standard_normal(shape) * std).astype(np.float32)


def host_student_t3(key: int, role: int, index: int, shape: Sequence[int], scale: float,
                    step: int = 0) -> np.ndarray:
    """float32 array of scale * T, T ~ Student-t with 3 degrees of freedom."""
    return (rng(key, role, index, step).standard_t(3.0, size=shape) * scale).astype(np.float32)


def host_inputs(wl: Workload, index: int, step: int = 0, shape=None):
    """(W, M_prev, G) float32 host arrays for matrix `index` of workload `wl` at `step`."""
    shape = tuple(shape or wl.shapes[index])
    w = host_normal(wl.key, ROLE_W, index, shape, wl.w_std)
    m = host_normal(wl.key, ROLE_M, index, shape, wl.m0_std)
    g = host_gradient(wl, index, step, shape)
    return w, m, g


def host_gradient(wl: Workload, index: int, step: int, shape=None) -> np.ndarray:
    shape = tuple(shape or wl.shapes[index])
    if wl.g_dist == "t3":
        return host_student_t3(wl.key, ROLE_G, index, shape, wl.g_std, step)
    return host_normal(wl.key, ROLE_G, index, shape, wl.g_std, step)


def device_fill(tensor, key: int, role: int, index: int, std: float, dist: str = "normal",
                step: int = 0):
    """Fill a float32 CUDA tensor in place from a seeded torch generator (bench only)."""
    import torch

    gen = torch.Generator(device=tensor.device)
    gen.manual_seed((((key * 8 + role) * 4096 + index) * 65536 + step) & 0x7FFFFFFFFFFFFFFF)
    if std == 0.0:
        tensor.zero_()
        return tensor
    if dist == "t3":
        # Student-t(3) = Z / sqrt(chi2_3 / 3), chi2_3 = sum of three squared standard normals.
        z = torch.randn(tensor.shape, generator=gen, device=tensor.device, dtype=torch.float32)
        chi = torch.zeros_like(z)
        for _ in range(3):
            e = torch.randn(tensor.shape, generator=gen, device=tensor.device, dtype=torch.float32)
            chi.addcmul_(e, e)
            del e
        tensor.copy_(z / torch.sqrt(chi / 3.0) * std)
        return tensor
    tensor.normal_(0.0, std, generator=gen)
    return tensor
