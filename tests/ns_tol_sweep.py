"""Sweep of the bf16 Newton-Schulz rounding error against the float64 oracle.

For working sizes m = min(A, B) from 1 to 63, and a grid of larger m, it draws
seeded Gaussian and Student-t(3) matrices of random shape (the other side up to 600,
or a small multiple of m; flat and tall), runs the oracle's Newton-Schulz and the CPU
emulation of the GPU's bf16 recipe (tests/bf16_emulation.py) on the same float32
input, and records per m the largest relative Frobenius error of the whole output and
the largest relative l2 error of one of its lines (rows of a flat output, columns of a
tall one). tests/tolerances.py sets the parity tolerances from these maxima.

Run as a script for the full sweep (about a minute on one core):
    python tests/ns_tol_sweep.py [draws_small] [draws_large] [seed]
(seeds 2024 and 7777 give the two sweeps tests/tolerances.py quotes)
The CPU test suite runs a smaller sweep with other seeds and checks every draw
against the tolerances.
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

from oracle import muon_oracle as O  # noqa: E402
from bf16_emulation import newton_schulz_bf16  # noqa: E402
from tolerances import ns_errors  # noqa: E402

LARGE_M = (64, 72, 96, 128, 160, 200, 256, 300, 384, 450, 512, 600)


def draw(rng, m, d, max_side=600):
    """Draw d of working size m: a random shape with min side m, flat or tall, from a
    Gaussian (three draws in four) or Student-t(3) distribution, as float32."""
    if d % 3:
        n = int(rng.integers(m, max(m, max_side) + 1))
    else:
        n = m * int(rng.integers(1, 5))
    shape = (m, n) if d % 2 else (n, m)
    if d % 4 == 3:
        x = rng.standard_t(3, size=shape)
    else:
        x = rng.standard_normal(shape)
    return x.astype(np.float32)


def measure(x):
    """(relative Frobenius error, largest relative line error) of the bf16 recipe."""
    return ns_errors(newton_schulz_bf16(x), O.newton_schulz(x))


def sweep(ms, draws, seed):
    """{m: (max whole-matrix error, mean whole-matrix error, max line error)}."""
    out = {}
    for m in ms:
        rng = np.random.default_rng([seed, m])
        fro, line = [], []
        for d in range(draws):
            f, ln = measure(draw(rng, m, d))
            fro.append(f)
            line.append(ln)
        out[m] = (max(fro), float(np.mean(fro)), max(line))
    return out


def main():
    import torch
    torch.set_num_threads(1)
    small = int(sys.argv[1]) if len(sys.argv) > 1 else 400
    large = int(sys.argv[2]) if len(sys.argv) > 2 else 40
    seed = int(sys.argv[3]) if len(sys.argv) > 3 else 2024
    res = sweep(range(1, 64), small, seed)
    res.update(sweep(LARGE_M, large, seed + 1))
    for m, (mx, mean, line) in res.items():
        print(f"m {m:4d}: max {mx:.4f}  mean {mean:.4f}  line max {line:.4f}", flush=True)
    bands = [(1, 12), (13, 31), (32, 63), (64, 255), (256, 600)]
    for lo, hi in bands:
        sel = [v for m, v in res.items() if lo <= m <= hi]
        print(f"m {lo}..{hi}: whole max {max(v[0] for v in sel):.4f}, line max {max(v[2] for v in sel):.4f}")


if __name__ == "__main__":
    main()
