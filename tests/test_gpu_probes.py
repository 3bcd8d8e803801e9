"""GPU checks of the measurement probes whose results bench.py reports as the
device's measured ceilings: the copy moves every byte (main loop and tail),
the read folds every word it is said to read, and the MFMA loop runs the
iterations, and so the FLOP, it reports.  A probe that skipped work would
report a ceiling above what the hardware does."""
import numpy as np
import pytest
import torch

from fp8_packed_reduced_amd import binding as B

pytestmark = pytest.mark.gpu

THREADS = 256  # threads per block of the copy and read probes


def _bytes(n: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)


@pytest.mark.parametrize("nbytes, blocks", [((1 << 20) + 48, 8), (4096 + 16, 3), (16, 1)])
def test_probe_copy_moves_every_byte(nbytes, blocks):
    src = _bytes(nbytes, 11).cuda()
    dst = torch.zeros_like(src)
    B.probe_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(src.cpu(), dst.cpu())


@pytest.mark.parametrize("nbytes, blocks", [((1 << 20) + 48, 8), (4096 + 16, 3)])
def test_probe_read_folds_every_word(nbytes, blocks):
    host = _bytes(nbytes, 12)
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    B.probe_read(host.cuda(), out, blocks)
    torch.cuda.synchronize()
    # each thread XORs the four words of every 16-byte element it strides
    # over; a block keeps the largest (unsigned) of its threads' values
    words = host.numpy().view(np.uint32).reshape(-1, 4)
    elem = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    stride = blocks * THREADS
    per_thread = np.zeros(stride, dtype=np.uint32)
    for i, x in enumerate(elem):
        per_thread[i % stride] ^= x
    expect = per_thread.reshape(blocks, THREADS).max(axis=1)
    got = out.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, expect)


def test_probe_mfma_runs_its_iterations():
    blocks = 4
    out3 = torch.zeros(blocks * 8, dtype=torch.float32, device="cuda")
    out6 = torch.zeros_like(out3)
    f3 = B.probe_mfma(blocks, 3, out3)
    f6 = B.probe_mfma(blocks, 6, out6)
    torch.cuda.synchronize()
    # 8 waves per block, 4 MFMAs per iteration, 2 * 32 * 32 * 64 FLOP each
    assert f3 == blocks * 8 * 3 * 4 * 2 * 32 * 32 * 64
    assert f6 == 2 * f3
    a3, a6 = out3.cpu().double(), out6.cpu().double()
    assert torch.isfinite(a3).all() and (a3 != 0).all()
    # twice the iterations accumulate twice the same products
    assert torch.allclose(a6, 2 * a3, rtol=1e-5, atol=0)
