"""HIP graph capture of the optimizer step, through the C ABI.

The library only enqueues kernels (no memset, allocation, copy or synchronisation
inside a step), so a Periodic cycle of muon_step calls can be captured once and
replayed: small matrix sets are launch-bound and gain most from it. The step index
decides refresh versus RowNorm on the host at capture time, so a captured K-step cycle
replays the same schedule (a refresh, then K - 1 RowNorm steps).

Each replay must equal eager execution of the same steps bit for bit (the same kernels
in the same order on the same data). Between replays the program runs eager work of
its own and synchronises, and every replay is checked, not only the first.
"""
import sys

import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


def make_state(torch, dev, shapes, key):
    w = [torch.from_numpy(WL.host_normal(key, WL.ROLE_W, i, s, 0.02)).to(dev) for i, s in enumerate(shapes)]
    m = [torch.from_numpy(WL.host_normal(key, WL.ROLE_M, i, s, 0.02)).to(dev) for i, s in enumerate(shapes)]
    g = [[torch.from_numpy(WL.host_normal(key, WL.ROLE_G, i, s, 1e-3, step)).to(dev) for i, s in enumerate(shapes)]
         for step in range(3)]
    return w, m, g


# the third set runs its Gram, polynomial and Apply stages with split tail tiles and
# their fixup launches (six [2560, 2560] matrices: the Gram and polynomial split the
# last 9 or 10 of each XCD's 41 or 42 upper tiles in 3 chunks, the Apply the last 11 of
# 75 in 2); the last, [2048, 8192] and four [2048, 2048], runs its Gram with the head
# split (each XCD's tiles of the first matrix in 3 chunks) and its fixup
@pytest.mark.parametrize("shapes", [[(128, 512)],
                                    [(768, 256), (256, 256), (1024, 256), (256, 1024), (1536, 256)],
                                    [(2560, 2560)] * 6,
                                    [(2048, 8192)] + [(2048, 2048)] * 4])
def test_captured_periodic_cycle_replays_bitwise(torch_dev, shapes):
    torch, dev = torch_dev
    hp = B.default_hparams(period_k=3)
    w0, m0, g = make_state(torch, dev, shapes, 800 + len(shapes))
    ws_e = B.make_workspace(shapes, dev)
    ws_g = B.make_workspace(shapes, dev)

    def cycle(w, m, ws, base):
        for j in range(3):
            B.muon_step(w, m, g[j], base + j, hp, ws)

    # eager reference: three cycles (steps 0..8), a snapshot after each
    w_e, m_e = [x.clone() for x in w0], [x.clone() for x in m0]
    snaps = []
    for r in range(3):
        cycle(w_e, m_e, ws_e, 3 * r)
        torch.cuda.synchronize()
        snaps.append(([x.clone() for x in w_e], [x.clone() for x in m_e]))

    # capture one cycle (steps 0, 1, 2: a refresh, then two RowNorm steps)
    w_g, m_g = [x.clone() for x in w0], [x.clone() for x in m0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        cycle(w_g, m_g, ws_g, 0)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(w_g, w0)), "capture must not execute the step"

    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        noise = torch.randn(1 << 20, device=dev)  # the program's own eager work between replays
        _ = (noise * 2.0).sum().item()
        for i, s in enumerate(shapes):
            assert torch.equal(w_g[i], snaps[r][0][i]), (s, r, "W")
            assert torch.equal(m_g[i], snaps[r][1][i]), (s, r, "M")
        log(f"{len(shapes)} matrices: replay {r} equals eager cycle {r} bit for bit")


def test_captured_ns5_batched_replays_bitwise(torch_dev):
    torch, dev = torch_dev
    shapes = [(300, 700), (700, 300)]
    hp = B.default_hparams()
    x = [torch.from_numpy(WL.host_normal(810, WL.ROLE_M, i, s, 1.0)).to(dev) for i, s in enumerate(shapes)]
    ws = B.make_workspace(shapes, dev)
    ref = B.ns5_batched(x, None, hp, ws)
    torch.cuda.synchronize()
    outs = [torch.zeros_like(t) for t in x]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        B.ns5_batched(x, outs, hp, ws)
    for r in range(3):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(o, e) for o, e in zip(outs, ref)), r
