"""Router projection and its backward on the GPU against the CPU oracle.

logits = x . W_r + bias (fp32), and from a score gradient dlogits:
dx = bf16(bf16(dlogits) . W_r^T), dW_r = x^T . bf16(dlogits) (fp32).  Floating
outputs must satisfy |gpu - oracle| <= 1e-2 + 1e-2*|oracle| (and the logits a
tighter fp32-sum bound); reruns must be bitwise identical.  The GPU's top-k
on its own logits is checked as a property (the chosen set is the exact
top-K of those fp32 values under score desc, id asc), not against the
oracle, since no oracle input may come from the GPU."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# (shape, why): contraction split or not, E of 64/128/256/320, ragged T, long H
SMALL = [
    (W["ep_share_4k"].scaled(T=512, H=256), "E=256, weight gradient in 2 row chunks"),
    (W["ep_share_4k"].scaled(T=512, H=1024), "E=256, contraction in 4 chunks"),
    (W["skew_8k"].scaled(T=1000, H=256), "E=128, skew bias, ragged T"),
    (synth.MoeShape("e64", 91, T=2048, H=128, F=64, E=64, K=4), "E=64"),
    (W["ep_share_4k"].scaled(T=64, H=7168), "few rows, long contraction"),
    (W["fwdbwd_16k"].scaled(T=4096, H=192), "many rows, short contraction"),
    (synth.MoeShape("e320s", 92, T=2048, H=64, F=64, E=320, K=4),
     "E=320 on 128-column tiles: three column tiles, the last half full, bias in the GEMM epilogue"),
    (synth.MoeShape("e320", 93, T=32768, H=128, F=64, E=320, K=4),
     "E=320 on 256-column tiles: two column tiles, bias in the GEMM epilogue"),
]


def bits(t):
    return pipeline.to_numpy_bits(t)


def dlogits_for(T, E, seed):
    return (np.random.default_rng(seed).standard_normal((T, E)) * 0.1).astype(np.float32)


def topk_property(logits, idx):
    """idx[t] must be the first K experts of logits[t] under (score desc, id asc)."""
    T, E = logits.shape
    K = idx.shape[1]
    s = logits.astype(np.float64) + 0.0  # -0 and +0 compare equal
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -s), axis=1)
    assert_equal("topk_idx (property)", idx, order[:, :K].astype(np.int32))


@pytest.mark.parametrize("k", range(len(SMALL)))
def test_router_logits_and_backward(k):
    shape, why = SMALL[k]
    T, H, E = shape.T, shape.H, shape.E
    print(f"[router] {why}: T={T} H={H} E={E} ws={_lib.moe_router_workspace_size(T, H, E)}", flush=True)
    inp = synth.make_inputs(shape, seed=2, weights=False, router=True)
    dev = pipeline.to_device(inp)
    logits = _lib.moe_router_logits(dev["x"], dev["w_router"], dev["router_bias"])
    logits2 = _lib.moe_router_logits(dev["x"], dev["w_router"], dev["router_bias"])
    dl = dlogits_for(T, E, 5)
    dx, dw = _lib.moe_router_backward(dev["x"], dev["w_router"], torch.from_numpy(dl).cuda())
    dx2, dw2 = _lib.moe_router_backward(dev["x"], dev["w_router"], torch.from_numpy(dl).cuda())
    idx, _ = _lib.moe_route(logits, shape.K)
    torch.cuda.synchronize()
    ref = oracle.router_logits(inp["x"], inp["w_router"], inp["router_bias"])
    got = bits(logits)
    assert_close("logits", got, ref)
    # the fp32 sums in chunk order against the fp64 sum: far inside the layer tolerance
    assert np.max(np.abs(got.astype(np.float64) - ref) / (1e-3 + np.abs(ref))) < 1e-3
    assert_equal("logits rerun", got, bits(logits2))
    topk_property(got, bits(idx))
    rdx, rdw = oracle.router_backward(inp["x"], inp["w_router"], dl)
    assert_close("dx", bits(dx), rdx)
    assert_close("dw_r", bits(dw), rdw)
    assert_equal("dx rerun", bits(dx), bits(dx2))
    assert_equal("dw_r rerun", bits(dw), bits(dw2))


def test_router_without_bias_and_zero_tokens():
    shape = SMALL[0][0]
    inp = synth.make_inputs(shape, seed=3, weights=False, router=True)
    dev = pipeline.to_device(inp)
    logits = _lib.moe_router_logits(dev["x"], dev["w_router"])
    torch.cuda.synchronize()
    assert_close("logits", bits(logits), oracle.router_logits(inp["x"], inp["w_router"]))
    # T = 0: no logits; the weight gradient of no tokens is exactly 0
    x0 = dev["x"][:0]
    l0 = _lib.moe_router_logits(x0, dev["w_router"])
    dw = torch.full((shape.H, shape.E), 7.0, device="cuda")
    _, dw = _lib.moe_router_backward(x0, dev["w_router"], torch.empty((0, shape.E), device="cuda"), dw_r=dw)
    torch.cuda.synchronize()
    assert l0.shape == (0, shape.E)
    assert torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("name", ["ep_share_4k", "skew_8k", "fwdbwd_16k", "ep_share_128k"])
def test_router_full_size_sampled(name):
    """Full workload sizes: logits and dx on sampled tokens, dW_r on sampled experts, reruns bitwise."""
    shape = W[name]
    T, H, E = shape.T, shape.H, shape.E
    print(f"[router] {name}: T={T} H={H} E={E}", flush=True)
    inp = synth.make_inputs(shape, seed=0, weights=False, router=True)
    dev = pipeline.to_device(inp)
    dl = dlogits_for(T, E, 6)
    ws = torch.empty(_lib.moe_router_workspace_size(T, H, E), dtype=torch.uint8, device="cuda")
    logits = _lib.moe_router_logits(dev["x"], dev["w_router"], dev["router_bias"], ws=ws)
    dx, dw = _lib.moe_router_backward(dev["x"], dev["w_router"], torch.from_numpy(dl).cuda(), ws=ws)
    logits2 = _lib.moe_router_logits(dev["x"], dev["w_router"], dev["router_bias"], ws=ws)
    idx, _ = _lib.moe_route(logits, shape.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 40)]))
    cols = np.unique(np.concatenate([[0, E - 1], rng.integers(0, E, 4)]))
    ref = oracle.router_logits(inp["x"], inp["w_router"], inp["router_bias"], rows=rows)
    got = bits(logits)
    assert_close("logits", got[rows], ref[rows])
    assert_equal("logits rerun", got, bits(logits2))
    topk_property(got[rows], bits(idx)[rows])
    rdx, rdw = oracle.router_backward(inp["x"], inp["w_router"], dl, rows=rows, cols=cols)
    assert_close("dx", bits(dx)[rows], rdx[rows])
    assert_close("dw_r", bits(dw)[:, cols], rdw[:, cols])


# (T, E, K): K of 1..16 (lanes per token 1, 2, 4, 8, 16; K not a power of two), E not a multiple of 4,
# E past 256 (the larger LDS slice), T ragged against the 8- and 4-token groups and past one pass of the grid
RB_CASES = [(1, 8, 1), (7, 8, 2), (13, 100, 3), (4099, 256, 8), (1001, 257, 5), (333, 320, 16), (2050, 512, 13),
            (65537, 128, 8), (9, 7, 4), (300000, 64, 2)]


@pytest.mark.parametrize("T,E,K", RB_CASES)
def test_route_backward_shapes(T, E, K):
    """dlogits from distinct top-K experts, gates and gate gradients against the oracle: zeros exactly where no
    expert was chosen, the chosen entries within tolerance; a rerun is bitwise identical."""
    print(f"[route_backward] T={T} E={E} K={K}", flush=True)
    rng = np.random.default_rng(T * 7 + E * 3 + K)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    g = rng.random((T, K)).astype(np.float32)
    g /= g.sum(axis=1, keepdims=True)
    dg = rng.standard_normal((T, K)).astype(np.float32)
    d_idx, d_g, d_dg = (torch.from_numpy(a).cuda() for a in (idx, g, dg))
    dl = _lib.moe_route_backward(d_idx, d_g, d_dg, E)
    torch.cuda.synchronize()
    got = dl.cpu().numpy()
    ref = oracle.route_backward(idx, g, dg, E)
    chosen = np.zeros((T, E), bool)
    np.put_along_axis(chosen, idx, True, axis=1)
    assert np.all(got[~chosen] == 0.0), "non-zero score gradient at an expert that was not chosen"
    assert_close("dlogits", got, ref)
    again = _lib.moe_route_backward(d_idx, d_g, d_dg, E)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy().view(np.uint32), got.view(np.uint32))


def _int_bits(rng, shape, lo, hi):
    table = np.array([np.float32(v).view(np.uint32) >> 16 for v in range(lo, hi + 1)], np.uint16)
    return table[rng.integers(0, hi - lo + 1, shape, dtype=np.int8)]


@pytest.mark.parametrize("k", range(len(SMALL)))
def test_router_exact_on_integer_operands(k):
    """The router projection and its backward on small-integer x, W_r, bias and dlogits: every product and
    sum is exact in fp32 in any order (the contraction chunks and their partial sums included), so logits,
    dx and dW_r must equal the oracle's bits exactly."""
    shape, why = SMALL[k]
    T, H, E = shape.T, shape.H, shape.E
    rng = np.random.default_rng(41 + k)
    x = _int_bits(rng, (T, H), -2, 2)
    w = _int_bits(rng, (H, E), -1, 1)
    bias = rng.integers(-3, 4, E).astype(np.float32)
    dl = rng.integers(-2, 3, (T, E)).astype(np.float32)
    dev = pipeline.to_device(dict(x=x, w=w, b=bias))
    logits = _lib.moe_router_logits(dev["x"], dev["w"], dev["b"])
    dx, dw = _lib.moe_router_backward(dev["x"], dev["w"], torch.from_numpy(dl).cuda())
    torch.cuda.synchronize()
    ref = oracle.router_logits(x, w, bias)
    assert_equal("logits", bits(logits), ref.astype(np.float32))
    rdx, rdw = oracle.router_backward(x, w, dl)
    assert_equal("dx", bits(dx), rdx)
    assert_equal("dw_r", bits(dw), rdw)
