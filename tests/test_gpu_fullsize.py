"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same pipeline calls, same capacity).

Index outputs are compared in full against the oracle; the row copy by a
property (x_perm[r] == x[src[r] // K] for every row); the floating-point
steps on sampled rows/tokens/columns that the oracle computes one by one.
Per-step inputs downstream of the permutation are seeded synthetic operands
of the real shapes fed identically to both sides, so no oracle input comes
from the GPU."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu


def bits(t):
    return pipeline.to_numpy_bits(t)


class Case:
    pass


@pytest.fixture(scope="module", params=list(synth.WORKLOADS))
def case(request):
    name = request.param
    shape = synth.WORKLOADS[name]
    print(f"\n[fullsize] {name}: generating inputs", flush=True)
    c = Case()
    c.shape = shape
    c.inp = synth.make_inputs(shape, seed=0, d_out=shape.backward)
    c.dev = pipeline.to_device(c.inp)
    c.buf = pipeline.MoeBuffers.allocate(shape, backward=shape.backward)
    print(f"[fullsize] {name}: running GPU forward{'+backward' if shape.backward else ''}", flush=True)
    pipeline.forward(c.buf, c.dev)
    if shape.backward:
        pipeline.backward(c.buf, c.dev)
    torch.cuda.synchronize()
    c.ref_idx, c.ref_g = oracle.route(c.inp["logits"], shape.K)
    c.ref_pm = oracle.permute(c.ref_idx, shape.e_begin, shape.EL, c.inp["x"], shape.cap)
    c.R = min(int(c.ref_pm["offsets"][-1]), shape.cap)
    c.rng = np.random.default_rng(7)
    yield c
    del c.buf, c.dev
    torch.cuda.empty_cache()


def sample_rows(c, n_random=128, whole_tiles=False):
    """Rows at the ends and middle of the first, last, largest and smallest experts plus random rows;
    with whole_tiles, also every row of five whole 256-row GEMM tiles: the largest expert's first tile,
    the last expert's last (ragged) tile, the smallest expert's first tile and a tile in the middle of
    each of two randomly chosen experts, so that every lane, MFMA row block and epilogue row of those
    tiles is compared element by element."""
    off = c.ref_pm["offsets"]
    counts = np.diff(off)
    nz = np.nonzero(counts)[0]
    pick = {nz[0], nz[-1], nz[np.argmax(counts[nz])], nz[np.argmin(counts[nz])]}
    rows = set()
    for j in pick:
        lo, hi = int(off[j]), int(min(off[j + 1], c.shape.cap))
        if lo < hi:
            rows |= {lo, hi - 1, (lo + hi) // 2}
    rows |= set(c.rng.integers(0, c.R, n_random).tolist())
    if whole_tiles:
        j = nz[np.argmax(counts[nz])]
        lo, hi = int(off[j]), int(min(off[j + 1], c.shape.cap))
        rows |= set(range(lo, min(hi, lo + 256)))
        j = nz[-1]
        lo, hi = int(off[j]), int(min(off[j + 1], c.shape.cap))
        rows |= set(range(lo + (hi - lo - 1) // 256 * 256, hi))
        j = nz[np.argmin(counts[nz])]
        lo, hi = int(off[j]), int(min(off[j + 1], c.shape.cap))
        rows |= set(range(lo, min(hi, lo + 256)))
        for j in c.rng.choice(nz, 2):
            lo, hi = int(off[j]), int(min(off[j + 1], c.shape.cap))
            t0 = lo + ((hi - lo) // 2) // 256 * 256
            rows |= set(range(t0, min(hi, t0 + 256)))
    return np.array(sorted(r for r in rows if r < c.R), np.int64)


def test_route_full(case):
    assert_equal("topk_idx", bits(case.buf.topk_idx), case.ref_idx)
    assert_close("gates", bits(case.buf.gates), case.ref_g)


def test_permute_full(case):
    c, pm = case, case.ref_pm
    assert_equal("counts", bits(c.buf.counts)[:c.shape.EL], pm["counts"])
    assert_equal("offsets", bits(c.buf.offsets), pm["offsets"])
    assert_equal("pos", bits(c.buf.pos), pm["pos"])
    assert_equal("src", bits(c.buf.src)[:c.R], pm["src"][:c.R])
    assert int(bits(c.buf.status)[0]) == pm["status"] == 0
    # the row copy, checked for every row on the device
    src = c.buf.src[:c.R].long()
    assert torch.equal(c.buf.x_perm[:c.R].view(torch.int16), c.dev["x"][src // c.shape.K].view(torch.int16))
    counts = pm["counts"]
    print(f"[fullsize] {c.shape.name}: R={c.R} rows/expert {counts.min()}..{counts.max()} "
          f"maxvio={synth.maxvio(counts, c.shape.T, c.shape.K, c.shape.E):.2f}", flush=True)


def test_expert_up_sampled_rows(case):
    c = case
    rows = sample_rows(c, whole_tiles=True)
    h, ab = oracle.expert_up(c.ref_pm["x_perm"], c.inp["w_gate"], c.inp["w_up"], c.ref_pm["offsets"],
                             c.shape.cap, rows=rows, want_ab=True)
    assert_close("h", bits(c.buf.h)[rows], h[rows])
    if c.buf.ab is not None:
        assert_close("ab_save", bits(c.buf.ab)[rows], ab[rows])


def test_zero_copy_gate_up_full(case):
    """The zero-copy gate/up GroupGEMM (rows read from x through src) at full size, in the bench's
    launch configuration: bit-identical to the copy path's h (and ab_save) for every row."""
    c = case
    s = c.shape
    h = torch.zeros_like(c.buf.h)
    ab = torch.zeros_like(c.buf.ab) if c.buf.ab is not None else None
    _lib.moe_grouped_gemm_swiglu_gather(c.dev["x"], c.buf.src, s.K, c.dev["w_gate"], c.dev["w_up"], c.buf.offsets,
                                        c.buf.cap, h=h, ab_save=ab)
    torch.cuda.synchronize()
    assert torch.equal(h[:c.R].view(torch.int16), c.buf.h[:c.R].view(torch.int16))
    if ab is not None:
        assert torch.equal(ab[:c.R].view(torch.int16), c.buf.ab[:c.R].view(torch.int16))
    del h, ab


def test_expert_down_sampled_rows(case):
    c = case
    s = c.shape
    hin = synth.operand_bf16((s.cap, s.F), seed=0, tag=1)
    dh = pipeline.to_device(dict(h=hin))["h"]
    y = torch.empty((s.cap, s.H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(dh, c.dev["w_down"], None, 0, c.buf.offsets, s.F, s.H, s.cap, y)
    torch.cuda.synchronize()
    rows = sample_rows(c, whole_tiles=True)
    ref = oracle.expert_down(hin, c.inp["w_down"], c.ref_pm["offsets"], s.cap, rows=rows)
    assert_close("y", bits(y)[rows], ref[rows])


def test_combine_sampled_tokens(case):
    c = case
    s = c.shape
    yin = synth.operand_bf16((s.cap, s.H), seed=0, tag=2)
    yd = pipeline.to_device(dict(y=yin))["y"]
    out = _lib.moe_combine(yd, c.buf.pos, c.buf.gates)
    out1 = _lib.moe_combine(yd, c.buf.pos, None)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, s.T - 1], c.rng.integers(0, s.T, 512),
                                     np.nonzero(np.all(c.ref_pm["pos"] < 0, axis=1))[0][:4]])).astype(np.int64)
    # gates: the oracle's own (bit-exact indices; gate values are the oracle's)
    ref = oracle.combine(yin, c.ref_pm["pos"], c.ref_g, tokens=toks)
    ref1 = oracle.combine(yin, c.ref_pm["pos"], None, tokens=toks)
    assert_close("out", bits(out)[toks], ref[toks])
    assert_close("out_ungated", bits(out1)[toks], ref1[toks])


def _bwd_only(c):
    if not c.shape.backward:
        pytest.skip("forward-only workload")


def test_gather_sampled_rows(case):
    c = case
    _bwd_only(c)
    s = c.shape
    rows = sample_rows(c, whole_tiles=True)
    ref = oracle.bwd_gather(c.inp["d_out"], c.ref_pm["src"], c.ref_pm["offsets"], c.ref_g, s.K, s.cap)
    assert_close("dy_perm", bits(c.buf.dy_perm)[rows], ref[rows])


def test_dgrad_down_swiglu_sampled_rows(case):
    c = case
    _bwd_only(c)
    s = c.shape
    dy = synth.operand_bf16((s.cap, s.H), seed=0, tag=3, std=0.125)
    ab = synth.operand_bf16((s.cap, 2 * s.F), seed=0, tag=4)
    d = pipeline.to_device(dict(dy=dy, ab=ab))
    dab = torch.empty((s.cap, 2 * s.F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d["dy"], c.dev["w_down"], None, 1, c.buf.offsets, s.H, s.F, s.cap, dab,
                          epilogue=_lib.MOE_EPI_SWIGLU_BWD, ab=d["ab"])
    torch.cuda.synchronize()
    rows = sample_rows(c, whole_tiles=True)
    ref = oracle.bwd_down(dy, c.inp["w_down"], ab, c.ref_pm["offsets"], s.cap, rows=rows)
    assert_close("dab", bits(dab)[rows], ref[rows])


def test_dgrad_up_sampled_rows(case):
    c = case
    _bwd_only(c)
    s = c.shape
    dabin = synth.operand_bf16((s.cap, 2 * s.F), seed=0, tag=5, std=0.1)
    d = pipeline.to_device(dict(dab=dabin))
    dx = torch.empty((s.cap, s.H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d["dab"], c.dev["w_gate"], c.dev["w_up"], 1, c.buf.offsets, s.F, s.H, s.cap, dx)
    torch.cuda.synchronize()
    rows = sample_rows(c, whole_tiles=True)
    ref = oracle.bwd_up(dabin, c.inp["w_gate"], c.inp["w_up"], c.ref_pm["offsets"], s.cap, rows=rows)
    assert_close("dx_perm", bits(dx)[rows], ref[rows])


@pytest.mark.parametrize("which", ["gate", "down"])
def test_wgrad_sampled(case, which):
    c = case
    _bwd_only(c)
    s = c.shape
    if which == "gate":
        M, N, lda, ldb = s.H, s.F, s.H, 2 * s.F
        A = synth.operand_bf16((s.cap, s.H), seed=0, tag=6)
        B = synth.operand_bf16((s.cap, 2 * s.F), seed=0, tag=7, std=0.1)
    else:
        M, N, lda, ldb = s.F, s.H, s.F, s.H
        A = synth.operand_bf16((s.cap, s.F), seed=0, tag=8)
        B = synth.operand_bf16((s.cap, s.H), seed=0, tag=9, std=0.1)
    d = pipeline.to_device(dict(A=A, B=B))
    dw = _lib.moe_wgrad(d["A"], lda, d["B"], ldb, c.buf.offsets, s.EL, M, N, s.cap)
    dw2 = _lib.moe_wgrad(d["A"], lda, d["B"], ldb, c.buf.offsets, s.EL, M, N, s.cap)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32)), "wgrad rerun differs"
    counts = c.ref_pm["counts"]
    groups = np.unique([int(np.argmax(counts)), int(np.argmin(counts)), 0, s.EL - 1,
                        *c.rng.integers(0, s.EL, 3).tolist()]).astype(np.int32)
    # both ends, the columns on either side of each of the first 256-column tile edges, and random ones
    edges = [e + d for e in range(256, min(N, 1024), 256) for d in (-1, 0)]
    cols = np.unique(np.concatenate([[0, N - 1], edges, c.rng.integers(0, N, 64)])).astype(np.int32)
    ref = np.zeros((s.EL, M, N), np.float32)
    oracle.wgrad(A, lda, B, ldb, c.ref_pm["offsets"], M, N, s.cap, groups=groups, cols=cols, out=ref)
    got = dw.cpu().numpy()
    for j in groups:
        assert_close(f"dw[{j}]", got[j][:, cols], ref[j][:, cols])


def test_zero_copy_wgrad_gate_up_full(case):
    """The gate/up weight gradient reading its rows from x through src, at full size in the bench's launch
    configuration: bit-identical to the copy path's dW_gate and dW_up of the same backward."""
    c = case
    _bwd_only(c)
    s = c.shape
    gz, uz = _lib.moe_wgrad_gate_up_gather(c.dev["x"], c.buf.src, s.K, c.buf.dab, c.buf.offsets, s.EL, c.buf.cap)
    torch.cuda.synchronize()
    assert torch.equal(gz.view(torch.int32), c.buf.dw_gate.view(torch.int32))
    assert torch.equal(uz.view(torch.int32), c.buf.dw_up.view(torch.int32))
    del gz, uz


def test_wgrad_split_sampled(case):
    """The non-bitwise weight gradient (two row chunks per expert) at full size: sampled experts and
    columns against the oracle's serial sum, and a bitwise rerun."""
    c = case
    _bwd_only(c)
    s = c.shape
    M, N, lda, ldb = s.H, s.F, s.H, 2 * s.F
    A = synth.operand_bf16((s.cap, s.H), seed=0, tag=6)
    B = synth.operand_bf16((s.cap, 2 * s.F), seed=0, tag=7, std=0.1)
    d = pipeline.to_device(dict(A=A, B=B))
    ws = torch.empty(_lib.moe_wgrad_split_workspace_size(s.EL, M, N, 2), dtype=torch.uint8, device="cuda")
    dw = _lib.moe_wgrad_split(d["A"], lda, d["B"], ldb, c.buf.offsets, s.EL, M, N, s.cap, 2, ws=ws)
    dw2 = _lib.moe_wgrad_split(d["A"], lda, d["B"], ldb, c.buf.offsets, s.EL, M, N, s.cap, 2, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32)), "split wgrad rerun differs"
    counts = c.ref_pm["counts"]
    groups = np.unique([int(np.argmax(counts)), int(np.argmin(counts)), 1]).astype(np.int32)
    cols = np.unique(np.concatenate([[0, N - 1], c.rng.integers(0, N, 10)])).astype(np.int32)
    ref = np.zeros((s.EL, M, N), np.float32)
    oracle.wgrad(A, lda, B, ldb, c.ref_pm["offsets"], M, N, s.cap, groups=groups, cols=cols, out=ref)
    got = dw.cpu().numpy()
    for j in groups:
        assert_close(f"dw[{j}]", got[j][:, cols], ref[j][:, cols])


def test_gate_grad_and_route_backward_full(case):
    """Router backward at full size: dgates for every token from the same seeded d_out and y on both
    sides, the fused kernel's dy_perm equal to moe_gather's, and dlogits for every token from the same
    seeded dgates."""
    c = case
    s = c.shape
    d_out = c.inp["d_out"] if "d_out" in c.inp else synth.operand_bf16((s.T, s.H), seed=0, tag=10)
    yin = synth.operand_bf16((s.cap, s.H), seed=0, tag=11, std=0.05)
    d = pipeline.to_device(dict(d_out=d_out, y=yin))
    dy = torch.empty((s.cap, s.H), dtype=torch.bfloat16, device="cuda")
    dy2 = torch.empty_like(dy)
    _, dg = _lib.moe_gather_gate_grad(d["d_out"], c.buf.pos, c.buf.gates, d["y"], dy)
    _lib.moe_gather(d["d_out"], c.buf.pos, c.buf.gates, dy2)
    dgin = synth.operand_bf16((s.T, s.K), seed=0, tag=12)
    dgin = synth.bf16_bits_to_f32(dgin)
    dl = _lib.moe_route_backward(c.buf.topk_idx, c.buf.gates, torch.from_numpy(dgin).cuda(), s.E)
    torch.cuda.synchronize()
    R = c.R
    assert torch.equal(dy[:R].view(torch.int16), dy2[:R].view(torch.int16)), "fused gather differs"
    assert_close("dgates", bits(dg), oracle.gate_grad(d_out, yin, c.ref_pm["pos"]))
    # gates: the oracle's own (indices are bit-exact; gate values within tolerance)
    assert_close("dlogits", bits(dl), oracle.route_backward(c.ref_idx, c.ref_g, dgin, s.E))


def test_full_layer_rerun_bitwise(case):
    c = case
    s = c.shape
    b2 = pipeline.MoeBuffers.allocate(s, backward=s.backward)
    pipeline.forward(b2, c.dev)
    if s.backward:
        pipeline.backward(b2, c.dev)
    torch.cuda.synchronize()
    fields = ["topk_idx", "gates", "pos", "out"] + (["dx", "dw_gate", "dw_up", "dw_down", "dgates", "dlogits"]
                                                      if s.backward else [])
    for f in fields:
        assert torch.equal(getattr(c.buf, f).view(torch.uint8), getattr(b2, f).view(torch.uint8)), f
    R = c.R
    for f in ["src", "x_perm", "h", "y"] + (["ab", "dy_perm", "dab", "dx_perm"] if s.backward else []):
        assert torch.equal(getattr(c.buf, f)[:R].view(torch.uint8), getattr(b2, f)[:R].view(torch.uint8)), f
    del b2


def test_literal_zipf_bias_full_size_forward():
    """skew_8k's shape with the recipe read literally (alpha = 1, one expert gets most of the 65536 rows):
    indices and permutation in full, gate/up and the combine on sampled rows and tokens."""
    shape = synth.WORKLOADS["skew_8k"]
    inp = synth.make_inputs(shape, seed=0, alpha=1.0)
    dev = pipeline.to_device(inp)
    buf = pipeline.MoeBuffers.allocate(shape, backward=False)
    pipeline.forward(buf, dev)
    torch.cuda.synchronize()
    idx, g = oracle.route(inp["logits"], shape.K)
    pm = oracle.permute(idx, shape.e_begin, shape.EL, inp["x"], shape.cap)
    counts = pm["counts"]
    print(f"[fullsize] literal skew: rows per expert {counts.min()}..{counts.max()}", flush=True)
    assert counts.max() > 4000
    assert_equal("topk_idx", bits(buf.topk_idx), idx)
    assert_equal("offsets", bits(buf.offsets), pm["offsets"])
    assert_equal("pos", bits(buf.pos), pm["pos"])
    R = min(int(pm["offsets"][-1]), shape.cap)
    hot = int(np.argmax(counts))
    lo, hi = int(pm["offsets"][hot]), int(pm["offsets"][hot + 1])
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[lo, hi - 1, (lo + hi) // 2, 0, R - 1], rng.integers(0, R, 16)]))
    h, _ = oracle.expert_up(pm["x_perm"], inp["w_gate"], inp["w_up"], pm["offsets"], shape.cap, rows=rows,
                            want_ab=False)
    assert_close("h", bits(buf.h)[rows], h[rows])


def _int_bits(rng, shape, lo, hi):
    """bf16 bits of integers drawn from [lo, hi] (|v| <= 2: exact in bf16), built through a lookup table."""
    table = np.array([np.float32(v).view(np.uint32) >> 16 for v in range(lo, hi + 1)], np.uint16)
    return table[rng.integers(0, hi - lo + 1, shape, dtype=np.int8)]


def test_integer_operands_exact_at_full_size(case):
    """The GroupGEMMs at full size on small-integer operands (products and sums exact in fp32 in any order,
    so the stored bits must equal the oracle's exactly): the saved (a, b) of the gate/up GEMM and the down
    GEMM on the sampled rows and whole tiles, and for training workloads the gate/up dgrad, the down
    dgrad at a saved a of 0 (its SwiGLU backward then exact) and dW_gate, dW_up, dW_down on the sampled
    experts and columns."""
    c = case
    s = c.shape
    rng = np.random.default_rng(23)
    R = c.R
    x = _int_bits(rng, (s.cap, s.H), -2, 2)
    x[R:] = 0
    wg = _int_bits(rng, (s.EL, s.H, s.F), -1, 1)
    wu = _int_bits(rng, (s.EL, s.H, s.F), -1, 1)
    wd = _int_bits(rng, (s.EL, s.F, s.H), -1, 1)
    hin = _int_bits(rng, (s.cap, s.F), -2, 2)
    d = pipeline.to_device(dict(x=x, wg=wg, wu=wu, wd=wd, h=hin))
    h = torch.empty((s.cap, s.F), dtype=torch.bfloat16, device="cuda")
    ab = torch.empty((s.cap, 2 * s.F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm_swiglu(d["x"], d["wg"], d["wu"], c.buf.offsets, s.cap, h=h, ab_save=ab)
    y = torch.empty((s.cap, s.H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d["h"], d["wd"], None, 0, c.buf.offsets, s.F, s.H, s.cap, y)
    torch.cuda.synchronize()
    rows = sample_rows(c, whole_tiles=True)
    off = c.ref_pm["offsets"]
    _, ref_ab = oracle.expert_up(x, wg, wu, off, s.cap, rows=rows, want_ab=True)
    assert_equal("ab_save", bits(ab)[rows], ref_ab[rows])
    ref_y = oracle.expert_down(hin, wd, off, s.cap, rows=rows)
    assert_equal("y", bits(y)[rows], ref_y[rows])
    del h, ab, y
    if not s.backward:
        return
    dab = _int_bits(rng, (s.cap, 2 * s.F), -2, 2)
    dab[R:] = 0
    d2 = pipeline.to_device(dict(dab=dab))
    dx = torch.empty((s.cap, s.H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d2["dab"], d["wg"], d["wu"], 1, c.buf.offsets, s.F, s.H, s.cap, dx)
    dwg, dwu = _lib.moe_wgrad_gate_up(d["x"], d2["dab"], c.buf.offsets, s.EL, s.cap)
    dwd = _lib.moe_wgrad(d["h"], s.F, d["x"], s.H, c.buf.offsets, s.EL, s.F, s.H, s.cap)
    # the down dgrad with a saved a of 0 (sigmoid 1/2 exactly): exact da = dh * b / 2 and db = 0
    ab0 = dab.copy()
    ab0[:, :s.F] = 0
    dy = _int_bits(rng, (s.cap, s.H), -2, 2)
    d3 = pipeline.to_device(dict(ab0=ab0, dy=dy))
    dab_o = torch.empty((s.cap, 2 * s.F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d3["dy"], d["wd"], None, 1, c.buf.offsets, s.H, s.F, s.cap, dab_o,
                          epilogue=_lib.MOE_EPI_SWIGLU_BWD, ab=d3["ab0"])
    torch.cuda.synchronize()
    ref_dx = oracle.bwd_up(dab, wg, wu, off, s.cap, rows=rows)
    assert_equal("dx_perm", bits(dx)[rows], ref_dx[rows])
    ref_dab = oracle.bwd_down(dy, wd, ab0, off, s.cap, rows=rows)
    assert_equal("dab (a = 0)", bits(dab_o)[rows], ref_dab[rows])
    del dab_o, d3
    counts = c.ref_pm["counts"]
    groups = np.unique([int(np.argmax(counts)), int(np.argmin(counts)), 0, s.EL - 1,
                        *c.rng.integers(0, s.EL, 2).tolist()]).astype(np.int32)
    for name, got, A, lda, B, ldb, M, N in (
            ("dW_gate", dwg, x, s.H, dab, 2 * s.F, s.H, s.F),
            ("dW_up", dwu, x, s.H, dab.reshape(-1)[s.F:], 2 * s.F, s.H, s.F),
            ("dW_down", dwd, hin, s.F, x, s.H, s.F, s.H)):
        edges = [e + dd for e in range(256, min(N, 1024), 256) for dd in (-1, 0)]
        cols = np.unique(np.concatenate([[0, N - 1], edges, c.rng.integers(0, N, 32)])).astype(np.int32)
        ref = np.zeros((s.EL, M, N), np.float32)
        oracle.wgrad(A, lda, B, ldb, off, M, N, s.cap, groups=groups, cols=cols, out=ref)
        g = got.cpu().numpy()
        for j in groups:
            assert_equal(f"{name}[{j}]", g[j][:, cols], ref[j][:, cols])
    del dx, dwg, dwu, dwd
