"""GPU parity of the split tiles of the NS5 GEMM stages: the tail split and the head split.

When a group's Gram, polynomial or non-final Apply stage runs on 256-wide tiles and
every matrix of the group has the same K for it, an XCD whose tile count leaves a last
round of at most 16 tiles (of its 32 compute units) runs those tiles as K chunks that
write fp32 partial tiles; a fixup launch adds each tile's chunks in chunk order and
applies the stage's epilogue. The split is taken only when the modelled time it saves
exceeds the cost of its partial tiles (the library's planning rule).
Four sets exercise it:
  * 16 x [2048, 2048] (576 upper tiles): in the Gram and polynomial, XCDs 1, 3, 5 and
    7 hold 80 tiles and split their last 16 (from matrices 12 to 15) in 2 chunks; the
    Apply (128 tiles per XCD) does not split;
  * 10 x [2560, 2560] (550 upper tiles): in the Gram and polynomial, XCDs 1 to 7 hold
    70 tiles and split their last 6 (all from matrix 9) in 5 chunks (the plain deal: the
    balanced one, 68 or 69 tiles everywhere, models slower); the Apply's balanced deal
    gives every XCD 125 tiles, whose last round of 29 does not split;
  * [2048, 8448] and [8448, 2048]: the Gram and polynomial run on 128-wide tiles (72
    big upper tiles, one round either way), so the Apply also writes the row-major X'_r; every XCD holds 66
    Apply tiles and splits its last 2 (from the second matrix) in 8 chunks;
  * 2 x [4096, 4096]: only 272 upper tiles of 256, but two rounds of them per XCD (34
    tiles) against three of 128-wide ones (132), so the Gram and polynomial run on
    256-wide tiles and every XCD splits its last 2 (from the second matrix) in 8
    chunks; the Apply (64 tiles per XCD) does not split.
When the group's matrices differ in K and every XCD's tiles fit one round, the XCD
instead runs its first (longest) tiles as K chunks, the head split. Three sets exercise it:
  * [2048, 8192] and 4 x [2048, 2048] (180 upper tiles; K 32 and 8 units of 256): every
    XCD runs its 4 or 5 tiles of the first matrix as 3 chunks of 10 to 11 units (uneven
    chunks), its longest block 32 -> 11 units;
  * [6144, 3072] and [3072, 3072] (156 upper tiles; K 24 and 12 units): XCDs run their 9
    or 10 tiles of the first matrix as 2 chunks, 24 -> 12 units;
  * [9216, 1536] and 6 x [1536, 1536] (147 upper tiles; K 36 and 6 units): XCDs run
    their 2 or 3 tiles of the first matrix as 5 chunks of 7 to 8 units.
The matrices with split tiles and the first one are checked against the float64
oracle's Newton-Schulz at the bf16 tolerance, and each call is repeated to check
that the fixed-order chunk sums make it bitwise repeatable. The library's plan
(ns5_plan) must be the split listed here, so a change of rule that stops exercising
it fails the test; the rule itself is checked on the CPU over many sets. A seeded
sweep of six further sets (sides 2048 to 3072, one or two shapes, up to 16 matrices,
kept when the plan splits a tail or takes 256-wide tiles below 512 of them) checks the
first and last matrix of each against the oracle and every output for repeatability;
a seeded sweep of four sets that take the head split (sides 1024 to 2048, some ragged,
both orientations) does the same.
"""
import sys

import numpy as np
import pytest

from oracle import muon_oracle as O
from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL
from tolerances import assert_ns_close

pytestmark = pytest.mark.gpu

# shapes, matrices checked against the oracle, split of the symmetric stages (XCD ->
# (tail tiles, chunks)), split of the Apply
CASES = [
    ([(2048, 2048)] * 16, [0, 12, 13, 14, 15], {1: (16, 2), 3: (16, 2), 5: (16, 2), 7: (16, 2)}, {}),
    ([(2560, 2560)] * 10, [0, 9], {x: (6, 5) for x in range(1, 8)}, {}),
    ([(2048, 8448), (8448, 2048)], [0, 1], {}, {x: (2, 8) for x in range(8)}),
    ([(4096, 4096)] * 2, [1], {x: (2, 8) for x in range(8)}, {}),
]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("case", range(len(CASES)))
def test_split_tail_tiles_vs_oracle_and_repeatable(torch_dev, case):
    torch, dev = torch_dev
    shapes, checked, split, split_apply = CASES[case]
    plan = B.ns5_plan(shapes)
    assert len(plan) == 1 and plan[0]["apply"][0] == 256
    assert plan[0]["gram"][1] == plan[0]["poly"][1] == split
    assert plan[0]["apply"][1] == split_apply and plan[0]["apply_final"][1] == {}
    xs = [WL.host_normal(7 + case, WL.ROLE_G, i, s, 1e-3) for i, s in enumerate(shapes)]
    ins = [torch.from_numpy(x.astype(np.float32)).to(dev) for x in xs]
    log(f"ns5_batched: {shapes}, split tail tiles {split}, Apply {split_apply}")
    outs = B.ns5_batched(ins)
    outs2 = B.ns5_batched(ins)
    torch.cuda.synchronize()
    for i, (o, o2) in enumerate(zip(outs, outs2)):
        assert torch.equal(o, o2), f"matrix {i}: two calls differ"
    for i in checked:
        ref = O.newton_schulz(xs[i].astype(np.float32).astype(np.float64))
        oh = outs[i].detach().cpu().numpy().astype(np.float64)
        err, line = assert_ns_close(oh, ref, shapes[i], i)
        log(f"  matrix {i} {shapes[i]}: rel err {err:.3e}, worst line {line:.3e}")


HEAD_CASES = [
    ([(2048, 8192)] + [(2048, 2048)] * 4, [0, 4], {x: (-4 - (x & 1), 3) for x in range(8)}),
    ([(6144, 3072), (3072, 3072)], [0, 1], {x: (-9 if x in (0, 4) else -10, 2) for x in range(8)}),
    ([(9216, 1536)] + [(1536, 1536)] * 6, [0, 6], {x: (-2 if x in (0, 2, 5) else -3, 5) for x in range(8)}),
]


@pytest.mark.parametrize("case", range(len(HEAD_CASES)))
def test_split_head_tiles_vs_oracle_and_repeatable(torch_dev, case):
    torch, dev = torch_dev
    shapes, checked, split = HEAD_CASES[case]
    plan = B.ns5_plan(shapes)
    assert len(plan) == 1 and plan[0]["gram"] == (256, split)
    xs = [WL.host_normal(17 + case, WL.ROLE_G, i, s, 1e-3) for i, s in enumerate(shapes)]
    ins = [torch.from_numpy(x.astype(np.float32)).to(dev) for x in xs]
    log(f"ns5_batched: {shapes}, Gram head split {split}, polynomial {plan[0]['poly']}, Apply {plan[0]['apply']}")
    outs = B.ns5_batched(ins)
    outs2 = B.ns5_batched(ins)
    torch.cuda.synchronize()
    for i, (o, o2) in enumerate(zip(outs, outs2)):
        assert torch.equal(o, o2), f"matrix {i}: two calls differ"
    for i in checked:
        ref = O.newton_schulz(xs[i].astype(np.float32).astype(np.float64))
        oh = outs[i].detach().cpu().numpy().astype(np.float64)
        err, line = assert_ns_close(oh, ref, shapes[i], i)
        log(f"  matrix {i} {shapes[i]}: rel err {err:.3e}, worst line {line:.3e}")


def random_big_sets(count=6, seed=20241202):
    """Seeded sets on 256-wide tiles: m from 2048 to 3072, n = m, m + 256 or 2 m, random
    orientation, 1 to 16 matrices of one or two shapes; a set is kept when the library's
    plan splits tiles (tail or head) in some stage or takes 256-wide tiles for a stage with fewer than
    512 of them (the fewer-rounds rule)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        kinds = int(rng.integers(1, 3))
        m = int(rng.choice([2048, 2304, 2560, 2816, 3072]))
        pool = []
        for _ in range(kinds):
            n = int(rng.choice([m, m + 256, 2 * m]))
            pool.append((m, n) if rng.random() < 0.5 else (n, m))
        shapes = [pool[int(rng.integers(0, kinds))] for _ in range(int(rng.integers(1, 17)))]
        plan = B.ns5_plan(shapes)
        split = any(g[st][1] for g in plan for st in ("gram", "poly", "apply"))
        few = False
        for g in plan:
            mats = [(min(shapes[i]), max(shapes[i])) for i in g["indices"]]
            ms = [(-(-a // 256), -(-b // 256)) for a, b in mats]
            if g["gram"][0] == 256 and sum(t * (t + 1) // 2 for t, _ in ms) < 512:
                few = True
            if g["apply"][0] == 256 and sum(t * u for t, u in ms) < 512:
                few = True
        if split or few:
            out.append((shapes, split, few))
    return out


@pytest.mark.parametrize("case", range(6))
def test_random_big_sets_vs_oracle(torch_dev, case):
    torch, dev = torch_dev
    sets = random_big_sets()
    assert sum(1 for _, s, _ in sets if s) >= 3 and sum(1 for _, _, f in sets if f) >= 1
    shapes, split, few = sets[case]
    plan = B.ns5_plan(shapes)
    xs = [WL.host_normal(31 + case, WL.ROLE_G, i, s, 1e-3) for i, s in enumerate(shapes)]
    ins = [torch.from_numpy(x.astype(np.float32)).to(dev) for x in xs]
    log(f"ns5_batched: {len(shapes)} matrices {sorted(set(shapes))}, split {split}, fewer-rounds tiles {few}")
    outs = B.ns5_batched(ins)
    outs2 = B.ns5_batched(ins)
    torch.cuda.synchronize()
    for i, (o, o2) in enumerate(zip(outs, outs2)):
        assert torch.equal(o, o2), f"matrix {i}: two calls differ"
    checked = sorted({plan[0]["indices"][0], plan[-1]["indices"][-1]})
    for i in checked:
        ref = O.newton_schulz(xs[i].astype(np.float32).astype(np.float64))
        oh = outs[i].detach().cpu().numpy().astype(np.float64)
        err, line = assert_ns_close(oh, ref, shapes[i], i)
        log(f"  matrix {i} {shapes[i]}: rel err {err:.3e}, worst line {line:.3e}")


def random_head_sets(count=4, seed=20241205):
    """Seeded sets that take the head split: m from 1024 to 2048, two or three values of
    n (1 to 4 times m, some ragged by 100), random orientation, 3 to 9 matrices; kept
    when the Gram's plan splits the first tiles of some XCD."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m = int(rng.choice([1024, 1536, 2048]))
        ns = [int(rng.choice([1, 2, 3, 4])) * m + int(rng.choice([0, 0, 100])) for _ in range(int(rng.integers(2, 4)))]
        shapes = []
        for _ in range(int(rng.integers(3, 10))):
            n = ns[int(rng.integers(0, len(ns)))]
            shapes.append((m, n) if rng.random() < 0.5 else (n, m))
        plan = B.ns5_plan(shapes)
        if any(h < 0 for g in plan for h, _ in g["gram"][1].values()):
            out.append(shapes)
    return out


@pytest.mark.parametrize("case", range(4))
def test_random_head_split_sets_vs_oracle(torch_dev, case):
    """The head split on seeded sets with ragged sides and both orientations: every
    output bitwise repeatable; the group's first matrix (whose tiles are the split ones)
    and its last against the oracle."""
    torch, dev = torch_dev
    shapes = random_head_sets()[case]
    plan = B.ns5_plan(shapes)
    xs = [WL.host_normal(41 + case, WL.ROLE_G, i, s, 1e-3) for i, s in enumerate(shapes)]
    ins = [torch.from_numpy(x.astype(np.float32)).to(dev) for x in xs]
    log(f"ns5_batched: {shapes}, Gram {plan[0]['gram']}")
    outs = B.ns5_batched(ins)
    outs2 = B.ns5_batched(ins)
    torch.cuda.synchronize()
    for i, (o, o2) in enumerate(zip(outs, outs2)):
        assert torch.equal(o, o2), f"matrix {i}: two calls differ"
    for i in sorted({plan[0]["indices"][0], plan[-1]["indices"][-1]}):
        ref = O.newton_schulz(xs[i].astype(np.float32).astype(np.float64))
        oh = outs[i].detach().cpu().numpy().astype(np.float64)
        err, line = assert_ns_close(oh, ref, shapes[i], i)
        log(f"  matrix {i} {shapes[i]}: rel err {err:.3e}, worst line {line:.3e}")
