"""The binding's own workspace on a side stream.

When no workspace is passed, the binding allocates one for the call. It must be
allocated on the stream the call enqueues on: torch's caching allocator hands a
freed block out again only to allocations on its own stream, in that stream's order.
These tests enqueue the step on a side stream without a workspace, then at once
allocate and overwrite memory on the default stream while the side stream may still
run, and compare with the same step run on the default stream with an explicit
workspace: bit for bit, since the kernels and their order are the same.
"""
import sys

import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B
from matrix_orthogonalising_optimizer_02_amd import workloads as WL

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 3072), (3072, 1024), (512, 512)]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


def state(torch, dev, key):
    w = [torch.from_numpy(WL.host_normal(key, WL.ROLE_W, i, s, 0.02)).to(dev) for i, s in enumerate(SHAPES)]
    m = [torch.from_numpy(WL.host_normal(key, WL.ROLE_M, i, s, 0.02)).to(dev) for i, s in enumerate(SHAPES)]
    g = [torch.from_numpy(WL.host_normal(key, WL.ROLE_G, i, s, 1e-3)).to(dev) for i, s in enumerate(SHAPES)]
    return w, m, g


@pytest.mark.parametrize("step", [0, 1], ids=["refresh", "rownorm"])
def test_side_stream_without_workspace(torch_dev, step):
    torch, dev = torch_dev
    hp = B.default_hparams(period_k=3)
    w_ref, m_ref, g_ref = state(torch, dev, 77)
    ws = B.make_workspace(SHAPES, dev)
    for _ in range(3):
        B.muon_step(w_ref, m_ref, g_ref, step, hp, ws)
    torch.cuda.synchronize()
    w, m, g = state(torch, dev, 77)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    log(f"step {step} three times on a side stream, binding-allocated workspace")
    for _ in range(3):
        B.muon_step(w, m, g, step, hp, stream=side)
        # the default stream allocates and writes while the side stream may still run
        junk = torch.empty(B.workspace_bytes(SHAPES) // 4 + 1024, dtype=torch.float32, device=dev)
        junk.fill_(float("nan"))
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for i, s in enumerate(SHAPES):
        assert torch.equal(w[i], w_ref[i]), (s, "W")
        assert torch.equal(m[i], m_ref[i]), (s, "M")
        assert bool(torch.isfinite(w[i]).all()), s


def test_side_stream_ns5_without_workspace(torch_dev):
    torch, dev = torch_dev
    xs = [torch.from_numpy(WL.host_normal(78, WL.ROLE_G, i, s, 1.0)).to(dev) for i, s in enumerate(SHAPES)]
    ref = B.ns5_batched(xs, workspace=B.make_workspace(SHAPES, dev))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = B.ns5_batched(xs, stream=side)
    junk = torch.empty(B.workspace_bytes(SHAPES) // 4 + 1024, dtype=torch.float32, device=dev)
    junk.fill_(float("nan"))
    side.synchronize()
    torch.cuda.synchronize()
    for s, o, r in zip(SHAPES, outs, ref):
        assert torch.equal(o, r), s
    assert np.isfinite(junk.cpu().numpy()).sum() == 0
