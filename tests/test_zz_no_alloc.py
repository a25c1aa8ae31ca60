"""rownorm_update_noalloc: the RowNorm step on the library's fixed device scratch.

It must give what rownorm_update gives on the same inputs, bit for bit (the same
kernels in the same order, only the workspace address differs): W, M and the
update-RMS monitor. Two calls in a row, the second on a smaller set, so the second
runs on scratch that still holds the first call's data. Then the call captured in a
HIP graph (it allocates nothing) and replayed three times against three eager
rownorm_update steps.
"""
import sys

import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL

pytestmark = pytest.mark.gpu

FIRST = [(3072, 1024), (1024, 3072), (8192, 2048), (777, 333), (333, 777), (512, 512), (5000, 12), (12, 5000)]
SECOND = [(1000, 300), (300, 1000), (64, 64)]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


def state(torch, dev, key, shapes):
    out = []
    for role, std in ((WL.ROLE_W, 0.02), (WL.ROLE_M, 0.02), (WL.ROLE_G, 1e-3)):
        out.append([torch.from_numpy(WL.host_normal(key, role, i, s, std)).to(dev) for i, s in enumerate(shapes)])
    return out


def compare(torch, dev, key, shapes):
    hp = B.default_hparams()
    w1, m1, g1 = state(torch, dev, key, shapes)
    w2, m2, g2 = state(torch, dev, key, shapes)
    r1 = torch.full((len(shapes),), -1.0, device=dev)
    r2 = torch.full((len(shapes),), -1.0, device=dev)
    B.rownorm_update(w1, m1, g1, hp, B.make_workspace(shapes, dev), update_rms=r1)
    B.rownorm_update_noalloc(w2, m2, g2, hp, update_rms=r2)
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        assert torch.equal(w1[i], w2[i]), (s, "W")
        assert torch.equal(m1[i], m2[i]), (s, "M")
    assert torch.equal(r1, r2), (r1, r2)
    assert bool((r2 > 0).all())
    # and without the monitor
    B.rownorm_update(w1, m1, g1, hp, B.make_workspace(shapes, dev))
    B.rownorm_update_noalloc(w2, m2, g2, hp)
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        assert torch.equal(w1[i], w2[i]), (s, "W, second step")
        assert torch.equal(m1[i], m2[i]), (s, "M, second step")


def test_noalloc_matches_rownorm_update_twice(torch_dev):
    torch, dev = torch_dev
    log(f"rownorm_update_noalloc vs rownorm_update: {FIRST}")
    compare(torch, dev, 501, FIRST)
    log(f"again on a smaller set: {SECOND}")
    compare(torch, dev, 502, SECOND)


def test_noalloc_full_size_15b_set(torch_dev):
    """The 15B-scale set's RowNorm step: six tall matrices up to [30720, 5120] in one
    group (about 43 MB of scratch)."""
    torch, dev = torch_dev
    wl = WL.LAYER_SET_15B_H5120
    hp = B.default_hparams()
    log(f"15B-scale set: {wl.shapes}")
    outs = []
    for use_noalloc in (False, True):
        w = [torch.empty(s, dtype=torch.float32, device=dev) for s in wl.shapes]
        m = [torch.empty_like(x) for x in w]
        g = [torch.empty_like(x) for x in w]
        for i in range(len(w)):
            WL.device_fill(w[i], wl.key, WL.ROLE_W, i, wl.w_std)
            WL.device_fill(m[i], wl.key, WL.ROLE_M, i, 1e-3)
            WL.device_fill(g[i], wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist)
        if use_noalloc:
            B.rownorm_update_noalloc(w, m, g, hp)
        else:
            B.rownorm_update(w, m, g, hp, B.make_workspace(wl.shapes, dev))
        torch.cuda.synchronize()
        outs.append((w, m))
        del g
    for i, s in enumerate(wl.shapes):
        assert torch.equal(outs[0][0][i], outs[1][0][i]), (s, "W")
        assert torch.equal(outs[0][1][i], outs[1][1][i]), (s, "M")


def test_noalloc_in_a_graph(torch_dev):
    torch, dev = torch_dev
    hp = B.default_hparams()
    shapes = [(2048, 512), (512, 2048), (300, 300)]
    w1, m1, g1 = state(torch, dev, 503, shapes)
    w2, m2, g2 = state(torch, dev, 503, shapes)
    ws = B.make_workspace(shapes, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    log("capture rownorm_update_noalloc")
    with torch.cuda.graph(graph, stream=side):
        B.rownorm_update_noalloc(w2, m2, g2, hp)
    torch.cuda.synchronize()
    for rep in range(3):
        B.rownorm_update(w1, m1, g1, hp, ws)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert bool(torch.isfinite(junk))
        for i, s in enumerate(shapes):
            assert torch.equal(w1[i], w2[i]), (rep, s, "W")
            assert torch.equal(m1[i], m2[i]), (rep, s, "M")
    del graph
