"""The GEMM kernels' block -> (matrix, tile, K chunk) mapping, restated on the CPU and
checked against the library's plans.

For a stage launch the kernel reads, per XCD x (block b runs on XCD b mod 8, slot
b div 8): the rotation of each matrix's eighths (XCD x takes eighth (x + r) mod 8 of
every matrix's tile sequence, matrices in group order), and for split launches
xfull[x], xtail[x], xsplit[x] and xpbase[x]: slots from xfull on are chunk u mod S of
tile xfull + u div S while u = slot - xfull < xtail S (partial tile xpbase + u), then
the tiles after the split ones, whole. A tail split has xfull = the XCD's tile count
minus its split tiles; a head split has xfull = 0. The fixup launch takes split tile t
of the XCDs in order. This test rebuilds those arguments from ns5_plan and the
planning rules of tests/test_plan_cpu.py and checks, for every stage of every group:
every tile of every matrix is computed exactly once, whole or as all of its chunks;
partial tiles are numbered 0 .. units - 1 without gaps or repeats; the grid (8 x the
largest per-XCD block count) covers every block; the fixup finds each split tile's
chunks; a head split stays within one round of 32 blocks per XCD.
"""
import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
import test_plan_cpu as P


def rotations(mats, stage, width):
    """(tiles, r) per matrix, as the deal the planner takes for the stage."""
    bal = P.rotated_deal(mats, stage, width, True)
    use_bal = P.deal(mats, stage, width) == bal
    load = [0] * 8
    out = []
    for m, n in mats:
        t = m // width
        total = t * (n // width) if stage == "apply" else t * (t + 1) // 2
        k = (n if stage == "gram" else m) // 256
        e = P.eighths(total)
        r = 0
        if use_bal:
            r = min(range(8), key=lambda r: (sum((load[x] + e[(x + r) % 8] * k) ** 2 for x in range(8)), r))
        out.append((total, r))
        for x in range(8):
            load[x] += e[(x + r) % 8] * k
    return out


def xcd_slot(desc, x, sl):
    for g, (total, r) in enumerate(desc):
        j = (x + r) & 7
        lo = (j * total) >> 3
        c = (((j + 1) * total) >> 3) - lo
        if sl < c:
            return g, lo + sl
        sl -= c
    return -1, 0


def check_plan(shapes):
    plan = B.ns5_plan(shapes)
    splits = 0
    for grp in plan:
        mats = [(P.ceil_div(min(shapes[i]), 256) * 256, P.ceil_div(max(shapes[i]), 256) * 256) for i in grp["indices"]]
        for st in ("gram", "poly", "apply"):
            width, sp = grp[st]
            desc = rotations(mats, st, width)
            cnt = [sum(P.eighths(total)[(x + r) & 7] for total, r in desc) for x in range(8)]
            xfull, xtail, xsplit, xpbase = [0] * 8, [0] * 8, [1] * 8, [0] * 8
            base = 0
            head = any(h < 0 for h, _ in sp.values())
            for x in range(8):
                h, S = sp.get(x, (0, 1))
                xtail[x] = abs(h)
                xfull[x] = 0 if h < 0 or (head and h == 0) else cnt[x] - h
                xsplit[x] = S
                xpbase[x] = base
                base += xtail[x] * S
            total_blocks = 8 * max(cnt[x] + xtail[x] * (xsplit[x] - 1) for x in range(8))
            if head:
                assert total_blocks // 8 <= 32, (shapes, st)
            got, units = {}, set()
            for b in range(total_blocks):
                x, sl, chunk = b & 7, b >> 3, -1
                if sp and sl >= xfull[x]:
                    u, nt, S = sl - xfull[x], xtail[x], xsplit[x]
                    if u < nt * S:
                        chunk, sl = u % S, xfull[x] + u // S
                        unit = xpbase[x] + u
                        assert unit not in units
                        units.add(unit)
                    else:
                        sl = xfull[x] + nt + (u - nt * S)
                gi, loc = xcd_slot(desc, x, sl)
                if gi >= 0:
                    got.setdefault((gi, loc), []).append((x, sl, chunk))
            assert len(got) == sum(total for total, _ in desc), (shapes, st)
            for (gi, loc), v in got.items():
                x0, sl0 = v[0][0], v[0][1]
                split = bool(sp) and xfull[x0] <= sl0 < xfull[x0] + xtail[x0]
                assert sorted(c for _, _, c in v) == (list(range(xsplit[x0])) if split else [-1]), (shapes, st, gi, loc)
            assert units == set(range(base)), (shapes, st)
            for t0 in range(sum(xtail)):
                t, x = t0, 0
                while t >= xtail[x]:
                    t -= xtail[x]
                    x += 1
                gi, loc = xcd_slot(desc, x, xfull[x] + t)
                assert gi >= 0 and all(c >= 0 for _, _, c in got[(gi, loc)])
            splits += sum(xtail)
    return splits


def mapping_sets():
    sets = [list(w.shapes) for w in WL.WORKLOADS] + P.bench_and_test_sets()
    sets += [[(2048, 8192)] + [(2048, 2048)] * 4, [(6144, 3072), (3072, 3072)], [(9216, 1536)] + [(1536, 1536)] * 6,
             [(2560, 2560)] * 6, [(8450, 2046)] * 3 + [(8450, 2048)]]
    rng = np.random.default_rng(20241204)
    for _ in range(60):
        m = int(rng.choice([1024, 1536, 2048, 2304, 2560, 3072]))
        ns = [int(rng.choice([1, 2, 3, 4, 6, 8])) * m + int(rng.choice([0, 0, 100])) for _ in range(int(rng.integers(2, 4)))]
        sh = []
        for _ in range(int(rng.integers(2, 12))):
            n = ns[int(rng.integers(0, len(ns)))]
            sh.append((m, n) if rng.random() < 0.5 else (n, m))
        sets.append(sh)
    return sets


def test_split_block_mapping_covers_every_tile_once():
    P._lib_or_skip()
    total = sum(check_plan(s) for s in mapping_sets())
    assert total > 500  # the sets exercise tail and head splits, not only whole-tile launches
