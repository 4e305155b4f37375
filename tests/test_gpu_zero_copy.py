"""Zero-copy dispatch (MoonEP page, "How Redundant Expert Planning Achieves
Perfect Balance"): the gate/up GroupGEMM reads each row of the
expert-grouped order straight from the tokens, x[src[r] // K], after an
index-only permutation.  Its h and ab_save must be bit-identical to the
copy path (same kernel, same accumulation order, only the address of the A
rows differs) and within tolerance of the oracle; the whole zero-copy
forward must give the copy path's output bit for bit.  The backward half:
the gate/up weight gradient reads its contraction rows through src too, so
a whole training step runs with no x_perm, bit for bit the copy path's."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SHAPES = {
    "tiny": W["tiny"].scaled(),
    "ep_share_small": W["ep_share_4k"].scaled(T=512, H=256, F=192),
    "skew_small": W["skew_8k"].scaled(T=1024, H=256, F=128),
    "long_small": W["ep_share_128k"].scaled(T=2048, H=128, F=64),
}


def bits(t):
    return pipeline.to_numpy_bits(t)


def gate_up_both_ways(shape, inp, cap):
    """-> (copy-path buffers, zero-copy permutation, zero-copy h, zero-copy ab)."""
    dev = pipeline.to_device(inp)
    ref = pipeline.MoeBuffers.allocate(shape, cap=cap, backward=True)
    pipeline.route(ref, dev["logits"])
    pipeline.permute(ref, dev["x"])
    pipeline.expert_up(ref, dev["w_gate"], dev["w_up"])
    pm = _lib.moe_permute(ref.topk_idx, shape.e_begin, shape.EL, dev["x"], cap, copy_rows=False)
    assert pm["x_perm"] is None
    h = torch.zeros_like(ref.h)
    ab = torch.zeros_like(ref.ab)
    _lib.moe_grouped_gemm_swiglu_gather(dev["x"], pm["src"], shape.K, dev["w_gate"], dev["w_up"], pm["offsets"],
                                        cap, h=h, ab_save=ab)
    torch.cuda.synchronize()
    return ref, pm, h, ab


@pytest.mark.parametrize("tile", ["auto", "256", "192", "128"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_gather_gate_up_equals_copy_path(name, tile, monkeypatch):
    if tile != "auto":
        monkeypatch.setenv("MOE_GEMM_TILE", tile)
    shape = SHAPES[name]
    print(f"[zero-copy] {name} tile={tile} T={shape.T} H={shape.H} F={shape.F} EL={shape.EL}", flush=True)
    inp = synth.make_inputs(shape, seed=6)
    ref, pm, h, ab = gate_up_both_ways(shape, inp, shape.cap)
    R = min(int(bits(ref.offsets)[-1]), shape.cap)
    assert_equal("offsets", bits(pm["offsets"]), bits(ref.offsets))
    assert_equal("src", bits(pm["src"])[:R], bits(ref.src)[:R])
    assert_equal("h", bits(h)[:R], bits(ref.h)[:R])
    assert_equal("ab_save", bits(ab)[:R], bits(ref.ab)[:R])
    # and against the oracle directly
    o = oracle.forward(inp, shape.e_begin, shape.EL, shape.K, shape.cap)
    assert_close("h", bits(h)[:R], o["h"][:R])
    assert_close("ab_save", bits(ab)[:R], o["ab"][:R])


@pytest.mark.parametrize("name", ["ep_share_small", "skew_small"])
def test_gather_with_dropped_rows(name):
    """Capacity below R: the rows past cap_rows are dropped on both paths."""
    shape = SHAPES[name]
    inp = synth.make_inputs(shape, seed=8)
    idx, _ = oracle.route(inp["logits"], shape.K)
    R_full = int(oracle.permute(idx, shape.e_begin, shape.EL, inp["x"], shape.cap)["offsets"][-1])
    cap = max(R_full // 2 + 7, 1)
    ref, pm, h, ab = gate_up_both_ways(shape, inp, cap)
    assert int(bits(pm["status"])[0]) == 1
    assert_equal("h", bits(h)[:cap], bits(ref.h)[:cap])
    assert_equal("ab_save", bits(ab)[:cap], bits(ref.ab)[:cap])


@pytest.mark.parametrize("name", list(SHAPES))
def test_zero_copy_forward_equals_copy_forward(name):
    shape = SHAPES[name]
    inp = synth.make_inputs(shape, seed=9)
    dev = pipeline.to_device(inp)
    a = pipeline.MoeBuffers.allocate(shape, backward=False)
    b = pipeline.MoeBuffers.allocate(shape, backward=False, zero_copy=True)
    assert b.x_perm is None
    pipeline.forward(a, dev)
    pipeline.forward(b, dev)
    torch.cuda.synchronize()
    R = min(int(bits(a.offsets)[-1]), shape.cap)
    assert_equal("h", bits(b.h)[:R], bits(a.h)[:R])
    assert_equal("y", bits(b.y)[:R], bits(a.y)[:R])
    assert_equal("out", bits(b.out), bits(a.out))
    o = oracle.forward(inp, shape.e_begin, shape.EL, shape.K, shape.cap)
    assert_close("out", bits(b.out), o["out"])


@pytest.mark.parametrize("K", [1, 3, 5, 16])
def test_gather_every_topk(K):
    """The row of pair index src = t*K + k is t = src / K, computed with a reciprocal and one correction:
    other K than the workloads' 2 and 8, including K = 1 and the largest K."""
    shape = synth.MoeShape(f"zc_k{K}", 95, T=333, H=128, F=64, E=max(16, K), K=K)
    inp = synth.make_inputs(shape, seed=K)
    ref, pm, h, ab = gate_up_both_ways(shape, inp, shape.cap)
    R = min(int(bits(ref.offsets)[-1]), shape.cap)
    assert_equal("h", bits(h)[:R], bits(ref.h)[:R])
    assert_equal("ab_save", bits(ab)[:R], bits(ref.ab)[:R])


def wgrad_both_ways(shape, inp, cap, seed):
    """dW_gate, dW_up from x_perm (copy path) and from x through src (zero-copy), on a seeded [da | db]."""
    dev = pipeline.to_device(inp)
    ref = pipeline.MoeBuffers.allocate(shape, cap=cap, backward=False)
    pipeline.route(ref, dev["logits"])
    pipeline.permute(ref, dev["x"])
    capn = max(cap, 1)
    dab = pipeline.to_device(dict(d=synth.operand_bf16((capn, 2 * shape.F), seed=seed, tag=41)))["d"]
    gw, uw = _lib.moe_wgrad_gate_up(ref.x_perm, dab, ref.offsets, shape.EL, cap)
    gz, uz = _lib.moe_wgrad_gate_up_gather(dev["x"], ref.src, shape.K, dab, ref.offsets, shape.EL, cap)
    torch.cuda.synchronize()
    return ref, (gw, uw), (gz, uz)


# experts of every size around a stage (32 rows), empty ones among them, many tiles per workgroup
SPARSE = synth.MoeShape("zc_sparse", 96, T=700, H=192, F=64, E=64, K=2, e_begin=3, e_local=40, zipf_s=1.5)


@pytest.mark.parametrize("tile", ["auto", "128"])
@pytest.mark.parametrize("name", list(SHAPES) + ["sparse"])
def test_gather_wgrad_equals_copy_path(name, tile, monkeypatch):
    """The weight gradient of gate/up reading its rows through src: bit for bit the copy path's, which the
    oracle pins (tests/test_gpu_parity.py); here also sampled against the oracle directly."""
    if tile != "auto":
        monkeypatch.setenv("MOE_GEMM_TILE", tile)
    shape = SPARSE if name == "sparse" else SHAPES[name]
    print(f"[zero-copy wgrad] {name} tile={tile} T={shape.T} H={shape.H} F={shape.F} EL={shape.EL}", flush=True)
    inp = synth.make_inputs(shape, seed=16)
    ref, (gw, uw), (gz, uz) = wgrad_both_ways(shape, inp, shape.cap, seed=16)
    assert torch.equal(gw.view(torch.int32), gz.view(torch.int32))
    assert torch.equal(uw.view(torch.int32), uz.view(torch.int32))
    counts = bits(ref.counts)
    assert (counts == 0).any() or name != "sparse"  # empty experts are skipped by the schedule


@pytest.mark.parametrize("name", ["ep_share_small", "sparse"])
def test_gather_wgrad_with_dropped_rows(name):
    """Capacity below R: rows past cap_rows take part in neither path."""
    shape = SPARSE if name == "sparse" else SHAPES[name]
    inp = synth.make_inputs(shape, seed=17)
    idx, _ = oracle.route(inp["logits"], shape.K)
    R_full = int(oracle.permute(idx, shape.e_begin, shape.EL, inp["x"], shape.cap)["offsets"][-1])
    cap = max(R_full // 2 + 5, 1)
    ref, (gw, uw), (gz, uz) = wgrad_both_ways(shape, inp, cap, seed=17)
    assert int(bits(ref.status)[0]) == 1
    assert torch.equal(gw.view(torch.int32), gz.view(torch.int32))
    assert torch.equal(uw.view(torch.int32), uz.view(torch.int32))


@pytest.mark.parametrize("K", [1, 3, 16])
def test_gather_wgrad_every_topk(K):
    shape = synth.MoeShape(f"zcw_k{K}", 97, T=333, H=128, F=64, E=max(16, K), K=K)
    inp = synth.make_inputs(shape, seed=K + 30)
    _, (gw, uw), (gz, uz) = wgrad_both_ways(shape, inp, shape.cap, seed=K)
    assert torch.equal(gw.view(torch.int32), gz.view(torch.int32))
    assert torch.equal(uw.view(torch.int32), uz.view(torch.int32))


@pytest.mark.parametrize("name", ["ep_share_small", "long_small", "sparse"])
def test_zero_copy_training_step_equals_copy_step(name):
    """A whole forward and backward with no x_perm at all: every output of the step bit for bit the copy
    path's, and the weight gradients within tolerance of the oracle."""
    shape = SPARSE if name == "sparse" else SHAPES[name]
    inp = synth.make_inputs(shape, seed=19, d_out=True)
    dev = pipeline.to_device(inp)
    a = pipeline.MoeBuffers.allocate(shape, backward=True)
    b = pipeline.MoeBuffers.allocate(shape, backward=True, zero_copy=True)
    assert b.x_perm is None
    for buf in (a, b):
        pipeline.forward(buf, dev)
        pipeline.backward(buf, dev)
    torch.cuda.synchronize()
    for f in ("out", "dx", "dlogits"):
        assert torch.equal(getattr(a, f).view(torch.int16 if getattr(a, f).dtype == torch.bfloat16 else torch.int32),
                           getattr(b, f).view(torch.int16 if getattr(b, f).dtype == torch.bfloat16 else torch.int32)), f
    for f in ("dw_gate", "dw_up", "dw_down"):
        assert torch.equal(getattr(a, f).view(torch.int32), getattr(b, f).view(torch.int32)), f
    o = oracle.forward(inp, shape.e_begin, shape.EL, shape.K, shape.cap)
    ob = oracle.backward(inp, o, shape.cap)
    assert_close("dw_gate", bits(b.dw_gate), ob["dw_gate"])
    assert_close("dw_up", bits(b.dw_up), ob["dw_up"])
