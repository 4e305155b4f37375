"""The MFMA throughput probe (a measurement aid for the bench) computes what it
claims: per wave, iters rounds of a 4 x 4 block of 32x32x16 bf16 products of
its register-held fragments.  With operands in {-1, 0, 1} every product and
sum is exact in fp32, so the sum over a wave's lanes must equal the closed
form of the header exactly: each 16-deep contraction splits into the lanes
0..31 and 32..63 halves, and the sum of all entries of A.B is the sum over
the contraction index of (column sums of A) x (row sums of B).  The copy
probe (the HBM-side measurement aid) must reproduce its source byte for
byte, whatever the load/store hints and grid, tail included."""
import numpy as np
import pytest
import torch

from routing_permute_groupgemm_amd import _lib

pytestmark = pytest.mark.gpu


def expected_wave_sums(ops, iters):
    """ops int [waves, 8, 64, 8]: fragments 0..3 are A, 4..7 are B."""
    o = ops.astype(np.float64).reshape(ops.shape[0], 8, 2, 32, 8)  # [w, frag, half, lane%32, j]
    col = o.sum(axis=3)                                              # [w, frag, half, j]
    a, b = col[:, :4], col[:, 4:]
    return iters * np.einsum("wmhj,wnhj->w", a, b)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 7), (256, 64)])
def test_probe_matches_closed_form(blocks, iters):
    rng = np.random.default_rng(blocks * 1000 + iters)
    ops = rng.integers(-1, 2, size=(blocks * 4, 8, 64, 8))
    dev = torch.from_numpy(ops.astype(np.float32)).to(torch.bfloat16).cuda()
    out = _lib.moe_probe_mfma(dev, iters)
    torch.cuda.synchronize()
    got = out.double().sum(dim=1).cpu().numpy()
    np.testing.assert_array_equal(got, expected_wave_sums(ops, iters))


def test_probe_zero_iterations_writes_zeros():
    ops = torch.ones((8, 8, 64, 8), dtype=torch.bfloat16, device="cuda")
    out = torch.full((8, 64), 7.0, dtype=torch.float32, device="cuda")
    _lib.moe_probe_mfma(ops, 0, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def expected_wave_sums16(ops, iters):
    """ops int [waves, 16, 64, 8]: fragments 0..7 are A, 8..15 are B; lanes in groups of 16 share a k-set."""
    o = ops.astype(np.float64).reshape(ops.shape[0], 16, 4, 16, 8)  # [w, frag, group, lane%16, j]
    col = o.sum(axis=3)                                               # [w, frag, group, j]
    a, b = col[:, :8], col[:, 8:]
    return iters * np.einsum("wmgj,wngj->w", a, b)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 7), (256, 64)])
def test_probe16_matches_closed_form(blocks, iters):
    rng = np.random.default_rng(blocks * 1000 + iters + 1)
    ops = rng.integers(-1, 2, size=(blocks * 4, 16, 64, 8))
    dev = torch.from_numpy(ops.astype(np.float32)).to(torch.bfloat16).cuda()
    out = _lib.moe_probe_mfma16(dev, iters)
    torch.cuda.synchronize()
    got = out.double().sum(dim=1).cpu().numpy()
    np.testing.assert_array_equal(got, expected_wave_sums16(ops, iters))


@pytest.mark.parametrize("nbytes,nontemporal,blocks", [
    (16, 0, 0), (16 * (3 * 1024 + 17), 1, 0), (16 * (3 * 1024 + 17), 2, 3), (16 * 1024 * 1024 + 48, 3, 0),
    (16 * 5000, 3, 1)])
def test_copy_probe_copies_exactly(nbytes, nontemporal, blocks):
    g = torch.Generator().manual_seed(nbytes + nontemporal)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    pad = 4096
    dst = torch.full((nbytes + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    _lib.moe_probe_copy(src, dst[:nbytes], nontemporal=nontemporal, blocks=blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes].cpu(), src.cpu())
    assert bool((dst[nbytes:] == 0xA5).all())  # nothing past the end
