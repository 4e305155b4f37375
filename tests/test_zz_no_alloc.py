"""moe_permute_noalloc (the permutation with its count matrix in the library's
own device array instead of a caller's workspace) against moe_permute, bit
for bit, through the C ABI: two calls in a row, the second on a smaller,
different input, so that anything the first call left in the array and the
second read before writing would show."""
import numpy as np
import pytest
import torch

from routing_permute_groupgemm_amd import _lib

pytestmark = pytest.mark.gpu


def topk_pairs(T, E, K, seed):
    """K distinct experts per token, from a seeded random ranking (host-side input generation)."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


def buffers(T, K, e_local, cap, H, dev):
    e = lambda *s, dt=torch.int32: torch.full(s, -7, dtype=dt, device=dev)  # noqa: E731
    return dict(counts=e(max(e_local, 1)), offsets=e(e_local + 1), pos=e(T, K), src=e(max(cap, 1)),
                status=e(4), x_perm=torch.zeros((max(cap, 1), H), dtype=torch.bfloat16, device=dev))


def run_both(T, E, K, e_begin, e_local, H, seed, dev, copy_rows=True):
    idx = torch.from_numpy(topk_pairs(T, E, K, seed)).to(dev)
    gen = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn((T, H), device=dev, generator=gen).to(torch.bfloat16)
    cap = T * K
    ref = buffers(T, K, e_local, cap, H, dev)
    got = buffers(T, K, e_local, cap, H, dev)
    ws = torch.empty(max(_lib.moe_permute_workspace_size(T, K, e_local), 256), dtype=torch.uint8, device=dev)
    _lib.moe_permute(idx, e_begin, e_local, x, cap, out=ref, ws=ws, copy_rows=copy_rows)
    _lib.moe_permute_noalloc(idx, e_begin, e_local, x, cap, out=got, copy_rows=copy_rows)
    torch.cuda.synchronize()
    R = int(ref["offsets"][e_local].item())
    for name in ("counts", "offsets", "pos", "status"):
        a, b = ref[name], got[name]
        if name == "counts":
            a, b = a[:e_local], b[:e_local]
        if name == "status":
            a, b = a[:1], b[:1]
        assert torch.equal(a, b), f"{name} differs (T={T}, e_local={e_local}, seed={seed})"
    assert torch.equal(ref["src"][:R], got["src"][:R]), f"src differs (T={T}, seed={seed})"
    if copy_rows:
        assert torch.equal(ref["x_perm"][:R].view(torch.int16), got["x_perm"][:R].view(torch.int16)), \
            f"x_perm differs (T={T}, seed={seed})"
    return R


# (first call, second call): each pair goes from a larger to a smaller input; the count matrix is laid out
# by the second call's block count, so stale entries of the first would land in its reads
CASES = [
    # all 128 experts local, 256-token blocks and the one-block scan; then a 32-of-256 share whose
    # 64-token blocks take the scan inside the rank kernel
    ((16384, 128, 8, 0, 128, 256, 1), (3000, 256, 8, 32, 32, 128, 2)),
    # the largest routing size of the layer's workloads (131072 tokens, 32 of 256 experts), then a
    # small one on the same path
    ((131072, 256, 8, 0, 32, 64, 3), (9000, 256, 8, 0, 32, 64, 4)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_path_on_two_calls(dev, first, second):
    for T, E, K, e_begin, e_local, H, seed in (first, second):
        print(f"noalloc case T={T} E={E} K={K} e_begin={e_begin} e_local={e_local} H={H} seed={seed}", flush=True)
        R = run_both(T, E, K, e_begin, e_local, H, seed, dev)
        assert R > 0


def test_noalloc_index_only_and_empty(dev):
    # the index-only permutation (no row copy), then zero tokens, then again a real call
    print("noalloc index-only / empty", flush=True)
    run_both(5000, 64, 4, 0, 64, 64, 5, dev, copy_rows=False)
    run_both(0, 64, 4, 0, 64, 64, 6, dev)
    run_both(777, 64, 4, 16, 8, 64, 7, dev)


def test_noalloc_rejects_oversize_before_launching(dev):
    # T=2^20 with 64 local experts needs 2 MiB of count matrix, over the 1 MiB array
    T, K, e_local = 1 << 20, 2, 64
    assert _lib.moe_permute_workspace_size(T, K, e_local) > (1 << 20)
    lib = _lib.load()
    fake = 0x10000  # never dereferenced: the size check fails first
    rc = lib.moe_permute_noalloc(fake, T, K, 0, e_local, fake, 64, T * K, fake, fake, fake, fake, fake, fake, None)
    assert rc == -4
