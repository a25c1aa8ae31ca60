"""The ceiling yardsticks the benchmark reports beside the spec peaks: the streaming
copy kernel copies exactly, including a ragged tail, and the MFMA loop's checksums
match a host recomputation of its register operands' products."""
import numpy as np
import pytest

from matrix_orthogonalising_optimizer_02_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a visible GPU"
    B.load_library()
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("n", [1, 4095, 4096, 4097, 3 * 4096 + 17, 1 << 22])
def test_copy_is_exact(torch_dev, n):
    torch, dev = torch_dev
    src = torch.randn(n, device=dev)
    dst = torch.full_like(src, float("nan"))
    B.ceiling_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def _bf16_bits_to_float(bits):
    return np.asarray(bits, np.uint32).astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)


def test_mfma_checksum(torch_dev):
    """The loop's operands follow a fixed per-lane word sequence (start from the lane
    index, then add 0x00250025, keep sign and mantissa bits, set the exponent of [0.5, 1)
    every round). Each round every one of the 16 accumulators adds A B^T of the
    32 x 32 x 16 operand blocks the lanes form (lane l holds row l % 32, k = 8 (l // 32)
    .. + 7 of both), so a wave's checksum is 16 times the sum over rounds of the
    entries of A B^T, recomputed here from the same sequence."""
    torch, dev = torch_dev
    blocks, iters = 3, 7
    out = torch.zeros(4 * blocks, device=dev)
    flops = B.ceiling_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 16 * 32 * 32 * 16 * 2
    mask, expo, step = 0x807F807F, 0x3F003F00, 0x00250025
    lanes = np.arange(64, dtype=np.uint64)
    a = np.stack([((lanes * 0x01030107 + e * 0x00110013) & mask) | expo for e in range(4)], 1) & 0xFFFFFFFF
    b = np.stack([((lanes * 0x02050309 + e * 0x00170019) & mask) | expo for e in range(4)], 1) & 0xFFFFFFFF
    total = 0.0
    for _ in range(iters):
        am = np.zeros((32, 16))
        bm = np.zeros((32, 16))
        for lane in range(64):
            for e in range(4):
                for half in range(2):  # element 2e + half of the lane's 8 bf16 values
                    k = 8 * (lane // 32) + 2 * e + half
                    am[lane % 32, k] = _bf16_bits_to_float((int(a[lane, e]) >> (16 * half)) & 0xFFFF)
                    bm[lane % 32, k] = _bf16_bits_to_float((int(b[lane, e]) >> (16 * half)) & 0xFFFF)
        total += float((am @ bm.T).sum())
        a = (((a + step) & 0xFFFFFFFF) & mask) | expo
        b = (((b + step) & 0xFFFFFFFF) & mask) | expo
    want = 16 * total
    got = out.cpu().numpy().astype(np.float64)
    assert np.allclose(got, want, rtol=1e-4, atol=1e-2), (got, want)
