"""Host-side planning of the Newton-Schulz GEMM stages, checked on the CPU.

The library's own plan (the host-only ns5_plan query, which runs the code the launches
run) is compared with the planning rules as stated here, written independently of the
library's C++:
  * grouping: nonempty matrices, working shape m = min(rows, cols), n = max(rows, cols),
    each padded up to a multiple of 256; a stable sort by (m, n), both descending;
    groups of at most 16;
  * tiles: the Gram and polynomial count the upper triangle of a [m, m] tile grid
    (diagonal included), the Apply every tile of [m, n]; each of the 8 XCDs takes a
    contiguous eighth of every matrix's tiles, XCD x eighth (x + r) mod 8. In the
    balanced deal each matrix in group order takes the r in 0..7 that leaves the XCDs'
    loads (tiles times K / 256, K = n for the Gram and m otherwise) with the smallest
    sum of squares, the smallest r on a tie; in the plain deal r = 0. 128-wide tiles
    take the balanced deal; 256-wide tiles take it only when its modelled cost is lower:
    the busiest XCD's span in K steps (q full rounds of K plus the last round's tiles or
    their largest chunk under the split rules below; the longest block when a stage
    with mixed K fits one round; otherwise a list schedule of the XCD's tiles, in order,
    on 32 compute units) times 0.86 us, plus 0.13 us per partial tile and 10 us when the
    stage splits;
  * tile width per stage: 256 when the stage has at least 512 such tiles (128 for the
    Gram); otherwise,
    when every matrix of the group has the same K for the stage (n for the Gram, m for
    the polynomial and the Apply), 256 when the busiest XCD needs fewer rounds of them
    (32 per round, one block per compute unit) than of 128-wide tiles (64 per round, two
    blocks per compute unit); 128 otherwise;
  * tail split, for a stage on 256-wide tiles whose matrices share K: an XCD whose last
    round holds r <= 16 tiles runs them as S = min(8, 32 // r, K / 256) chunks of K
    (S >= 2), taken only when (1 - 1 / S_min) of a tile's K steps at 0.86 us each exceeds
    0.13 us per partial tile plus 10 us; the partial-tile region is sized for the stage
    that splits the most tiles, and the last Apply never splits;
  * head split, for a stage on 256-wide tiles whose matrices do not share K and whose
    XCDs hold at most 32 tiles each: an XCD may run its first h tiles (K units of 256
    k_0, k_1, ...) as S in 2..8 chunks each, when h S plus its other tiles stay within
    32 and each split tile has at least S units; its longest block is then the largest
    of ceil(k_i / S) over the split tiles and k_i over the rest. The target is the
    largest over the XCDs of each one's best; each XCD above it takes the (h, S) that
    reaches it with the fewest partial tiles h S, then the smallest S; taken when the
    units saved on the longest XCD, 8 K steps at 0.86 us each, beat the same partial
    cost. Reported as (-h, S).
Sets: the benchmark workloads, the GPU tests' sets, and a seeded sweep of random sets.
"""
import ctypes
import heapq
import os

import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL

PAD, GROUP, XCDS, CUS = 256, 16, 8, 32


def _lib_or_skip():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmuon_rocm.so is not built")
    return B.load_library()


def ceil_div(a, b):
    return -(-a // b)


def eighths(total):
    return [((x + 1) * total >> 3) - (x * total >> 3) for x in range(XCDS)]


def rotated_deal(mats, stage, width, balance):
    """Per XCD, the K (units of 256) of each tile it takes, in order: XCD x takes eighth
    (x + r) mod 8 of each matrix, r = 0 or, balanced, the r that leaves the XCDs' loads
    (tiles times K) with the smallest sum of squares (the smallest r on a tie)."""
    seqs = [[] for _ in range(XCDS)]
    load = [0] * XCDS
    for m, n in mats:
        t = m // width
        total = t * (n // width) if stage == "apply" else t * (t + 1) // 2
        k = (n if stage == "gram" else m) // 256
        e = eighths(total)
        r = 0
        if balance:
            r = min(range(XCDS), key=lambda r: (sum((load[x] + e[(x + r) % XCDS] * k) ** 2 for x in range(XCDS)), r))
        for x in range(XCDS):
            seqs[x] += [k] * e[(x + r) % XCDS]
            load[x] += e[(x + r) % XCDS] * k
    return seqs


def shared_k(mats, stage):
    ks = {n if stage == "gram" else m for m, n in mats}
    return ks.pop() if len(ks) == 1 else None


def tail_split_of(counts, ksteps):
    """(partial tiles, {XCD: (tail tiles, chunks)}) for per-XCD tile counts of one K."""
    out = {}
    for x, c in enumerate(counts):
        r = c % CUS
        if 0 < r <= CUS // 2:
            s = min(8, CUS // r, ksteps // 8)
            if s >= 2:
                out[x] = (r, s)
    if not out:
        return 0, {}
    units = sum(r * s for r, s in out.values())
    s_min = min(s for _, s in out.values())
    if (1.0 - 1.0 / s_min) * ksteps * 0.86 <= units * 0.13 + 10.0:
        return 0, {}
    return units, out


def head_split_of(seqs):
    """(partial tiles, {XCD: (-h, chunks)}, longest block in units of 256 or None when
    the tiles do not fit one round)."""
    if max(len(v) for v in seqs) > CUS:
        return 0, {}, None

    def options(v):
        # (longest block, partial tiles, S, h) of every allowed split, and no split
        yield max(v, default=0), 0, 1, 0
        for S in range(2, 9):
            for h in range(1, len(v) + 1):
                if h * S + len(v) - h > CUS or min(v[:h]) < S:
                    break
                yield max([ceil_div(k, S) for k in v[:h]] + v[h:]), h * S, S, h

    before = max(max(v, default=0) for v in seqs)
    target = max(min(o[0] for o in options(v)) for v in seqs)
    out = {}
    for x, v in enumerate(seqs):
        if max(v, default=0) <= target:
            continue
        _, units, S, h = min((o for o in options(v) if o[0] <= target and o[1] > 0), key=lambda o: (o[1], o[2]))
        out[x] = (-h, S)
    units = sum(-h * S for h, S in out.values())
    if not out or (before - target) * 8 * 0.86 <= units * 0.13 + 10.0:
        return 0, {}, before
    return units, out, target


def list_schedule(durations):
    """Finish time of blocks taken in order, each by the first free of CUS units."""
    free = [0] * CUS
    heapq.heapify(free)
    end = 0
    for d in durations:
        t = heapq.heappop(free) + d
        end = max(end, t)
        heapq.heappush(free, t)
    return end


def modelled_cost(seqs, k):
    """Busiest XCD's span in K steps times 86 plus 13 per partial tile plus 1000 when the
    stage splits (hundredths of a microsecond)."""
    if k is not None:
        ksteps = k // 32
        units, split = tail_split_of([len(v) for v in seqs], ksteps)
        span = 0
        for x, v in enumerate(seqs):
            q, r = divmod(len(v), CUS)
            if x in split:
                last = ceil_div(ksteps // 8, split[x][1]) * 8
            else:
                last = ksteps if r else 0
            span = max(span, q * ksteps + last)
    else:
        units, split, longest = head_split_of(seqs)
        if longest is not None:
            span = longest * 8
        else:
            span = max(list_schedule([8 * kk for kk in v]) for v in seqs)
    return span * 86 + (units * 13 + 1000 if units else 0)


def deal(mats, stage, width):
    """The deal a stage uses: balanced, except on 256-wide tiles when the plain deal's
    modelled cost is not above the balanced one's (the plain deal when both are equal)."""
    bal = rotated_deal(mats, stage, width, True)
    if width != 256:
        return bal
    plain = rotated_deal(mats, stage, width, False)
    if plain == bal:
        return bal
    k = shared_k(mats, stage)
    return bal if modelled_cost(bal, k) < modelled_cost(plain, k) else plain


def per_xcd(mats, stage, width):
    return [len(v) for v in deal(mats, stage, width)]


def tile_width(mats, stage):
    big = per_xcd(mats, stage, 256)
    if sum(big) >= (128 if stage == "gram" else 512):
        return 256
    if shared_k(mats, stage) is None:
        return 128
    small = per_xcd(mats, stage, 128)
    return 256 if max(big) > 0 and ceil_div(max(big), CUS) < ceil_div(max(small), 2 * CUS) else 128


def split_of(mats, stage):
    """(partial tiles, {XCD: (tiles, chunks)}) of a stage on 256-wide tiles."""
    seqs = deal(mats, stage, 256)
    k = shared_k(mats, stage)
    if k is not None:
        return tail_split_of([len(v) for v in seqs], k // 32)
    units, split, _ = head_split_of(seqs)
    return units, split


def expected_plan(shapes):
    work = []
    for i, (a, b) in enumerate(shapes):
        if a == 0 or b == 0:
            continue
        work.append((ceil_div(min(a, b), PAD) * PAD, ceil_div(max(a, b), PAD) * PAD, min(a, b), max(a, b), i))
    work.sort(key=lambda w: (-w[2], -w[3]))  # stable: equal shapes keep their order
    groups = []
    for g0 in range(0, len(work), GROUP):
        grp = work[g0:g0 + GROUP]
        mats = [(w[0], w[1]) for w in grp]
        tiles = {st: tile_width(mats, st) for st in ("gram", "poly", "apply")}
        splits = {st: split_of(mats, st) if tiles[st] == 256 else (0, {}) for st in tiles}
        rec = {"indices": [w[4] for w in grp]}
        for st in ("gram", "poly", "apply"):
            rec[st] = (tiles[st], splits[st][1])
        rec["apply_final"] = (tiles["apply"], {})
        groups.append(rec)
    return groups


def bench_and_test_sets():
    sets = [list(wl.shapes) for wl in WL.WORKLOADS]
    sets += [
        [(2048, 2048)] * 16, [(2560, 2560)] * 10, [(2048, 8448), (8448, 2048)], [(4096, 4096)] * 2,
        [(2304, 2304)] * 5, [(2304, 2304)], [(2048, 2048)] * 3, [(3072, 3072)] * 2, [(6144, 6144)],
        [(2048, 8192)] * 20, [(0, 5), (300, 70), (7, 0), (70, 300)],
    ]
    return sets


@pytest.mark.parametrize("case", range(len(bench_and_test_sets())))
def test_plan_of_bench_and_test_sets(case):
    _lib_or_skip()
    shapes = bench_and_test_sets()[case]
    assert B.ns5_plan(shapes) == expected_plan(shapes)


def test_plan_of_random_sets():
    """Seeded random sets: sizes around the tile and padding edges, 1 to 40 matrices,
    shapes repeated so that groups often share K."""
    _lib_or_skip()
    rng = np.random.default_rng(20240607)
    sizes = [1, 100, 128, 255, 256, 257, 512, 1000, 1536, 2048, 2304, 2560, 3072, 3840, 4096, 5120, 6144, 8192]
    splits = 0
    chosen = {True: 0, False: 0}
    for trial in range(300):
        kinds = int(rng.integers(1, 4))
        pool = [(int(rng.choice(sizes)), int(rng.choice(sizes))) for _ in range(kinds)]
        shapes = [pool[int(rng.integers(0, kinds))] for _ in range(int(rng.integers(1, 41)))]
        want = expected_plan(shapes)
        assert B.ns5_plan(shapes) == want, (trial, shapes)
        splits += sum(1 for g in want for st in ("gram", "poly", "apply") if g[st][1])
        for g in want:
            mats = [(ceil_div(min(shapes[i]), PAD) * PAD, ceil_div(max(shapes[i]), PAD) * PAD) for i in g["indices"]]
            for st in ("gram", "poly", "apply"):
                bal = rotated_deal(mats, st, 256, True)
                if bal != rotated_deal(mats, st, 256, False):
                    chosen[deal(mats, st, 256) == bal] += 1
    assert splits > 20  # the sweep exercises the split rule, not only the tile rule
    assert min(chosen.values()) > 50  # and both outcomes of the deal choice


def test_plan_of_random_mixed_k_sets():
    """Seeded random sets that share m but differ in n (the Gram's K), few enough tiles
    for one round: the sets the head split is for. The sweep must take it often, with
    more than one chunk count."""
    _lib_or_skip()
    rng = np.random.default_rng(20241203)
    heads, chunks = 0, set()
    for trial in range(300):
        m = int(rng.choice([1024, 1536, 2048, 2304, 2560, 3072, 3328]))
        ns = [int(rng.choice([1, 2, 3, 4, 6, 8])) * m + int(rng.choice([0, 0, 100])) for _ in range(int(rng.integers(2, 4)))]
        shapes = []
        for _ in range(int(rng.integers(2, 9))):
            n = ns[int(rng.integers(0, len(ns)))]
            shapes.append((m, n) if rng.random() < 0.5 else (n, m))
        want = expected_plan(shapes)
        assert B.ns5_plan(shapes) == want, (trial, shapes)
        for g in want:
            for h, S in g["gram"][1].values():
                if h < 0:
                    heads += 1
                    chunks.add(S)
    assert heads > 50 and len(chunks) >= 2


def test_record_size_matches_the_header():
    import re
    header = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "muon_rocm.h")
    text = open(header).read()
    m = re.search(r"#define MUON_PLAN_RECORD_INTS (\d+)", text)
    assert m and int(m.group(1)) == B.PLAN_RECORD_INTS == 1 + GROUP + 4 * 17


def test_plan_argument_errors():
    lib = _lib_or_skip()
    rows = (ctypes.c_int64 * 2)(64, 128)
    cols = (ctypes.c_int64 * 2)(64, 256)
    ng = ctypes.c_int32(-1)
    assert lib.ns5_plan(rows, cols, 2, None, 0, None) == B.MUON_ERR_INVALID_ARG
    assert lib.ns5_plan(rows, cols, -1, None, 0, ctypes.byref(ng)) == B.MUON_ERR_INVALID_ARG
    assert lib.ns5_plan(None, None, 1, None, 0, ctypes.byref(ng)) == B.MUON_ERR_INVALID_ARG
    assert lib.ns5_plan(rows, cols, 2, None, 5, ctypes.byref(ng)) == B.MUON_ERR_INVALID_ARG
    short = (ctypes.c_int32 * (B.PLAN_RECORD_INTS - 1))()
    assert lib.ns5_plan(rows, cols, 2, short, B.PLAN_RECORD_INTS - 1, ctypes.byref(ng)) == B.MUON_ERR_INVALID_ARG
    assert lib.ns5_plan(rows, cols, 2, None, 0, ctypes.byref(ng)) == B.MUON_OK and ng.value == 1
    assert lib.ns5_plan(None, None, 0, None, 0, ctypes.byref(ng)) == B.MUON_OK and ng.value == 0
    bad = (ctypes.c_int64 * 1)(1 << 31)
    assert lib.ns5_plan(bad, cols, 1, None, 0, ctypes.byref(ng)) == B.MUON_ERR_TOO_LARGE
    neg = (ctypes.c_int64 * 1)(-3)
    assert lib.ns5_plan(neg, cols, 1, None, 0, ctypes.byref(ng)) == B.MUON_ERR_INVALID_ARG
