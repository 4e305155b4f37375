"""The weight-gradient entry points beside moe_wgrad.  The non-bitwise weight
gradient (moe_wgrad_split: each expert's rows in fixed chunks whose fp32
partials are added in chunk order) against the oracle
element by element, its run-to-run determinism, and its chunk semantics:
it equals, bit for bit, moe_wgrad over the refined row groups followed by
fp32 adds in chunk order.  The paired dW_gate/dW_up pass (moe_wgrad_gate_up)
against two moe_wgrad calls, bit for bit.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu

# empty experts, single rows, exact and ragged multiples of the 32-row step and of the 256-row tile
COUNTS = np.array([0, 130, 1, 64, 0, 257, 1000, 33], np.int32)


def operands(M, N, seed):
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    R = int(offsets[-1])
    a = synth.f32_to_bf16_bits(rng.standard_normal((R, M)).astype(np.float32))
    b = synth.f32_to_bf16_bits(rng.standard_normal((R, N)).astype(np.float32))
    return a, b, offsets, R


def refined_offsets(offsets, S):
    """Host restatement of the documented chunking: chunk c of expert j starts at
    off[j] + min(c * len, n), len = ceil(n / S) rounded up to 32 rows."""
    out = []
    for j in range(len(offsets) - 1):
        lo, n = int(offsets[j]), int(offsets[j + 1] - offsets[j])
        ln = ((n + S - 1) // S + 31) // 32 * 32
        out += [lo + min(c * ln, n) for c in range(S)]
    out.append(int(offsets[-1]))
    return np.array(out, np.int32)


@pytest.mark.parametrize("S,M,N", [(2, 192, 128), (3, 128, 256), (4, 320, 64)])
def test_split_matches_oracle_and_reruns(S, M, N):
    print(f"[wgrad_split] S={S} M={M} N={N}", flush=True)
    a, b, offsets, R = operands(M, N, seed=S)
    dev = pipeline.to_device(dict(a=a, b=b, offsets=offsets))
    EL = len(COUNTS)
    dw = torch.full((EL, M, N), float("nan"), dtype=torch.float32, device="cuda")
    _lib.moe_wgrad_split(dev["a"], M, dev["b"], N, dev["offsets"], EL, M, N, R, S, dw=dw)
    dw2 = _lib.moe_wgrad_split(dev["a"], M, dev["b"], N, dev["offsets"], EL, M, N, R, S)
    torch.cuda.synchronize()
    ref = oracle.wgrad(a, M, b, N, offsets, M, N, R)
    assert_close("dw", dw.cpu().numpy(), ref)
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32)), "rerun differs"
    for j in np.nonzero(COUNTS == 0)[0]:
        assert torch.all(dw[j] == 0).item(), f"empty expert {j} not zero"


@pytest.mark.parametrize("S", [2, 3])
def test_split_is_chunk_partials_added_in_order(S):
    M, N = 128, 192
    a, b, offsets, R = operands(M, N, seed=10 + S)
    dev = pipeline.to_device(dict(a=a, b=b, offsets=offsets, off2=refined_offsets(offsets, S)))
    EL = len(COUNTS)
    got = _lib.moe_wgrad_split(dev["a"], M, dev["b"], N, dev["offsets"], EL, M, N, R, S)
    part = _lib.moe_wgrad(dev["a"], M, dev["b"], N, dev["off2"], EL * S, M, N, R)
    want = part.view(EL, S, M, N)[:, 0].clone()
    for c in range(1, S):
        want += part.view(EL, S, M, N)[:, c]
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), "not the chunk partials in chunk order"


def test_split_one_is_the_bitwise_path():
    M, N = 64, 128
    a, b, offsets, R = operands(M, N, seed=21)
    dev = pipeline.to_device(dict(a=a, b=b, offsets=offsets))
    EL = len(COUNTS)
    got = _lib.moe_wgrad_split(dev["a"], M, dev["b"], N, dev["offsets"], EL, M, N, R, 1)
    want = _lib.moe_wgrad(dev["a"], M, dev["b"], N, dev["offsets"], EL, M, N, R)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))


@pytest.mark.parametrize("H,F", [(192, 64), (128, 192), (320, 128)])
def test_gate_up_pair_is_two_bitwise_wgrads(H, F):
    """dW_gate and dW_up from one pass over [da | db] equal the two separate weight gradients bit for bit
    (same fixed order per output element), including the empty experts' zeros; and the oracle within
    tolerance."""
    print(f"[wgrad_gate_up] H={H} F={F}", flush=True)
    a, dab, offsets, R = operands(H, 2 * F, seed=H + F)
    dev = pipeline.to_device(dict(a=a, dab=dab, offsets=offsets))
    EL = len(COUNTS)
    g0 = torch.full((EL, H, F), float("nan"), dtype=torch.float32, device="cuda")
    u0 = torch.full_like(g0, float("nan"))
    g, u = _lib.moe_wgrad_gate_up(dev["a"], dev["dab"], dev["offsets"], EL, R, dw_gate=g0, dw_up=u0)
    wg = _lib.moe_wgrad(dev["a"], H, dev["dab"], 2 * F, dev["offsets"], EL, H, F, R)
    wu = _lib.moe_wgrad(dev["a"], H, dev["dab"], 2 * F, dev["offsets"], EL, H, F, R, b_col0=F)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int32), wg.view(torch.int32)), "dW_gate differs from moe_wgrad"
    assert torch.equal(u.view(torch.int32), wu.view(torch.int32)), "dW_up differs from moe_wgrad"
    ref_g = oracle.wgrad(a, H, dab, 2 * F, offsets, H, F, R)
    ref_u = oracle.wgrad(a, H, np.ascontiguousarray(dab[:, F:]), F, offsets, H, F, R)
    assert_close("dw_gate", g.cpu().numpy(), ref_g)
    assert_close("dw_up", u.cpu().numpy(), ref_u)


@pytest.mark.parametrize("S", [2, 3, 5])
def test_split_exact_on_integer_operands(S):
    """The non-bitwise weight gradient on small-integer operands: the chunk partials and their sum are
    exact in fp32, so dW must equal the oracle's (bitwise path's) bits, whatever the chunking."""
    M, N = 192, 320
    rng = np.random.default_rng(60 + S)
    counts = COUNTS
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    table = np.array([np.float32(v).view(np.uint32) >> 16 for v in range(-2, 3)], np.uint16)
    a = table[rng.integers(0, 5, (R, M), dtype=np.int8)]
    b = table[rng.integers(0, 5, (R, N), dtype=np.int8)]
    dev = pipeline.to_device(dict(a=a, b=b, offsets=offsets))
    dw = _lib.moe_wgrad_split(dev["a"], M, dev["b"], N, dev["offsets"], len(counts), M, N, R, S)
    torch.cuda.synchronize()
    assert_equal("dw", dw.cpu().numpy(), oracle.wgrad(a, M, b, N, offsets, M, N, R))
