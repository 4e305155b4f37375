"""GPU parity of the whole layer (forward + backward) against the CPU oracle
at sizes the oracle finishes in seconds, plus edge cases and determinism.

Integer outputs (top-k indices, counts, offsets, pos, src) and the row copy
x_perm must be bit-exact; floating outputs must satisfy
|gpu - oracle| <= 1e-2 + 1e-2*|oracle| elementwise; GPU reruns must be
bitwise identical.  Every call goes through the C ABI (libmoe.so)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# Scaled-down copies of every workload: same E, K, routing recipe; several
# row tiles per expert, ragged tails, N not always a multiple of 128.
SMALL = {
    "tiny": W["tiny"].scaled(backward=True),
    "ep_share_small": W["ep_share_4k"].scaled(T=512, H=256, F=192, backward=True),
    "skew_small": W["skew_8k"].scaled(T=1024, H=256, F=128, backward=True),
    "fwdbwd_small": W["fwdbwd_16k"].scaled(T=1024, H=192, F=128),
    "long_small": W["ep_share_128k"].scaled(T=2048, H=128, F=64),
}


def bits(t):
    return pipeline.to_numpy_bits(t)


def run_gpu(shape, inp, cap=None):
    dev = pipeline.to_device(inp)
    buf = pipeline.MoeBuffers.allocate(shape, cap=cap, backward=True)
    pipeline.forward(buf, dev)
    pipeline.backward(buf, dev)
    torch.cuda.synchronize()
    return buf, dev


def check_layer(shape, inp, buf, cap):
    print(f"[parity] {shape.name} T={shape.T} H={shape.H} F={shape.F} E={shape.E} K={shape.K} "
          f"EL={shape.EL} cap={cap}", flush=True)
    ref = oracle.forward(inp, shape.e_begin, shape.EL, shape.K, cap)
    refb = oracle.backward(inp, ref, cap)
    R = min(int(ref["offsets"][-1]), cap)
    assert_equal("topk_idx", bits(buf.topk_idx), ref["topk_idx"])
    assert_close("gates", bits(buf.gates), ref["gates"])
    assert_equal("counts", bits(buf.counts)[:shape.EL], ref["counts"])
    assert_equal("offsets", bits(buf.offsets), ref["offsets"])
    assert_equal("pos", bits(buf.pos), ref["pos"])
    assert_equal("status", bits(buf.status)[0], ref["status"])
    assert_equal("src", bits(buf.src)[:R], ref["src"][:R])
    assert_equal("x_perm", bits(buf.x_perm)[:R], ref["x_perm"][:R])
    assert_close("h", bits(buf.h)[:R], ref["h"][:R])
    assert_close("ab_save", bits(buf.ab)[:R], ref["ab"][:R])
    assert_close("y", bits(buf.y)[:R], ref["y"][:R])
    assert_close("out", bits(buf.out), ref["out"])
    assert_close("dy_perm", bits(buf.dy_perm)[:R], refb["dy_perm"][:R])
    assert_close("dab", bits(buf.dab)[:R], refb["dab"][:R])
    assert_close("dx_perm", bits(buf.dx_perm)[:R], refb["dx_perm"][:R])
    assert_close("dx", bits(buf.dx), refb["dx"])
    assert_close("dw_gate", bits(buf.dw_gate), refb["dw_gate"])
    assert_close("dw_up", bits(buf.dw_up), refb["dw_up"])
    assert_close("dw_down", bits(buf.dw_down), refb["dw_down"])
    assert_close("dgates", bits(buf.dgates), refb["dgates"])
    assert_close("dlogits", bits(buf.dlogits), refb["dlogits"])
    return ref


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_forward_backward_matches_oracle(name):
    shape = SMALL[name]
    inp = synth.make_inputs(shape, seed=0, d_out=True)
    buf, _ = run_gpu(shape, inp)
    check_layer(shape, inp, buf, shape.cap)


@pytest.mark.parametrize("name", ["tiny", "skew_small"])
def test_layer_reruns_are_bitwise_identical(name):
    shape = SMALL[name]
    inp = synth.make_inputs(shape, seed=1, d_out=True)
    b1, dev = run_gpu(shape, inp)
    for _ in range(2):
        b2 = pipeline.MoeBuffers.allocate(shape, backward=True)
        pipeline.forward(b2, dev)
        pipeline.backward(b2, dev)
        torch.cuda.synchronize()
        R = int(bits(b1.offsets)[-1])
        for f in ("topk_idx", "gates", "pos", "out", "dx", "dw_gate", "dw_up", "dw_down", "dgates", "dlogits"):
            assert torch.equal(getattr(b1, f).view(torch.uint8), getattr(b2, f).view(torch.uint8)), f
        for f in ("src", "x_perm", "h", "ab", "y", "dy_perm", "dab", "dx_perm"):
            a, b = getattr(b1, f)[:R], getattr(b2, f)[:R]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f


def _inputs_with_logits(shape, logits, seed=3):
    inp = synth.make_inputs(shape, seed=seed, d_out=True)
    inp["logits"] = logits.astype(np.float32)
    return inp


def test_all_tokens_to_one_expert_and_empty_experts():
    shape = synth.MoeShape("one_hot", 90, T=300, H=128, F=128, E=8, K=2, backward=True)
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((shape.T, shape.E)).astype(np.float32)
    logits[:, 5] += 100.0   # expert 5 is everyone's first choice
    logits[:, 2] += 50.0    # expert 2 everyone's second; six experts stay empty
    inp = _inputs_with_logits(shape, logits)
    buf, _ = run_gpu(shape, inp)
    ref = check_layer(shape, inp, buf, shape.cap)
    assert sorted(ref["counts"].tolist()) == [0] * 6 + [300, 300]


def test_literal_zipf_bias_stress():
    """The skew recipe read literally (bias = ln Zipf(1.2), alpha = 1): one expert takes most of the rows
    and many get few or none; the whole layer still matches the oracle."""
    shape = SMALL["skew_small"]
    inp = synth.make_inputs(shape, seed=7, d_out=True, alpha=1.0)
    buf, _ = run_gpu(shape, inp)
    ref = check_layer(shape, inp, buf, shape.cap)
    counts = ref["counts"]
    print(f"[parity] literal skew: rows per expert {counts.min()}..{counts.max()} of {counts.sum()}", flush=True)
    assert counts.max() > 0.9 * shape.T  # a token picks an expert at most once: T rows is the most


def test_local_share_single_expert_and_nonlocal_tokens():
    shape = synth.MoeShape("single_local", 91, T=200, H=64, F=64, E=8, K=2, e_begin=3, e_local=1,
                           backward=True)
    inp = synth.make_inputs(shape, seed=0, d_out=True)
    buf, _ = run_gpu(shape, inp)
    ref = check_layer(shape, inp, buf, shape.cap)
    assert np.any(np.all(ref["pos"] < 0, axis=1))  # some tokens have no local pair -> zero rows


@pytest.mark.parametrize("T,K,E", [(1, 2, 8), (7, 3, 8), (65, 1, 16), (40, 8, 8), (33, 16, 64)])
def test_small_token_counts_and_k_extremes(T, K, E):
    shape = synth.MoeShape(f"edge_T{T}_K{K}", 92, T=T, H=128, F=64, E=E, K=K, backward=True)
    inp = synth.make_inputs(shape, seed=T, d_out=True)
    buf, _ = run_gpu(shape, inp)
    check_layer(shape, inp, buf, shape.cap)


def test_capacity_overflow_drops_tail_rows_and_sets_status():
    shape = synth.MoeShape("overflow", 93, T=256, H=128, F=128, E=8, K=2, backward=True)
    inp = synth.make_inputs(shape, seed=0, d_out=True)
    cap = 300  # R = 512 > cap
    buf, _ = run_gpu(shape, inp, cap=cap)
    ref = check_layer(shape, inp, buf, cap)
    assert ref["status"] == 1 and int(bits(buf.status)[0]) == 1


def test_zero_tokens():
    offsets = torch.full((9,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((8,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    _lib.moe_permute(idx, 0, 8, x, 0, out=dict(offsets=offsets, counts=counts, status=status))
    torch.cuda.synchronize()
    assert offsets.tolist() == [0] * 9 and counts.tolist() == [0] * 8 and status[0].item() == 0


def test_layer_at_the_largest_expert_counts():
    """The largest E (512, all local: the most groups a GroupGEMM takes) with the largest K (16): most
    experts get a handful of rows, some none, and the ranking matches 9-bit expert ids."""
    shape = synth.MoeShape("max_experts", 97, T=150, H=128, F=64, E=512, K=16, backward=True)
    inp = synth.make_inputs(shape, seed=3, d_out=True)
    buf, _ = run_gpu(shape, inp)
    ref = check_layer(shape, inp, buf, shape.cap)
    counts = ref["counts"]
    print(f"[parity] max_experts: rows per expert {counts.min()}..{counts.max()}, "
          f"{int(np.sum(counts == 0))} empty", flush=True)


def test_permute_no_local_experts():
    """Tokens but no local experts: every pair is non-local (pos -1), offsets [0], status 0."""
    idx = torch.randint(0, 8, (100, 2), dtype=torch.int32, device="cuda")
    x = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    offsets = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    out = _lib.moe_permute(idx, 0, 0, x, 0, out=dict(offsets=offsets, status=status), copy_rows=False)
    torch.cuda.synchronize()
    assert offsets.tolist() == [0] and status[0].item() == 0
    assert torch.all(out["pos"] == -1).item()


def test_wgrad_empty_expert_writes_zeros_and_grid_independence():
    """An expert with no rows gets exact zeros; a rerun (the persistent grid
    visits tiles in a different interleaving across workgroups) is identical."""
    rng = np.random.default_rng(5)
    counts = np.array([0, 130, 1, 64, 0, 257], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    M, N = 192, 128
    a = synth.f32_to_bf16_bits(rng.standard_normal((R, M)).astype(np.float32))
    b = synth.f32_to_bf16_bits(rng.standard_normal((R, N)).astype(np.float32))
    dev = pipeline.to_device(dict(a=a, b=b, offsets=offsets))
    dw = torch.full((len(counts), M, N), float("nan"), dtype=torch.float32, device="cuda")
    _lib.moe_wgrad(dev["a"], M, dev["b"], N, dev["offsets"], len(counts), M, N, R, dw=dw)
    dw2 = _lib.moe_wgrad(dev["a"], M, dev["b"], N, dev["offsets"], len(counts), M, N, R)
    torch.cuda.synchronize()
    ref = oracle.wgrad(a, M, b, N, offsets, M, N, R)
    assert_close("dw", dw.cpu().numpy(), ref)
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))
    assert np.all(dw[0].cpu().numpy() == 0) and np.all(dw[4].cpu().numpy() == 0)


@pytest.mark.parametrize("E,K", [(8, 2), (64, 8), (100, 8), (256, 8), (320, 16)])
def test_route_ties_and_signed_zeros(E, K):
    """Scores drawn from a handful of values (exact ties everywhere, -0.0 next to +0.0): the GPU's
    choice must follow (score desc, id asc) exactly."""
    rng = np.random.default_rng(E * 31 + K)
    T = 777
    logits = rng.integers(-2, 3, (T, E)).astype(np.float32)
    logits[rng.random((T, E)) < 0.2] = -0.0
    idx, g = _lib.moe_route(torch.from_numpy(logits).cuda(), K)
    torch.cuda.synchronize()
    ref_idx, ref_g = oracle.route(logits, K)
    assert_equal("topk_idx", bits(idx), ref_idx)
    assert_close("gates", bits(g), ref_g)


def _threshold_rows(E, rng):
    """Router scores that exercise both ways the route kernel selects: rows of distinct N(0,1) scores
    (a few candidates above the threshold), flat rows and rows with 64 or 65 experts tied at the top
    (64 candidates: the rank count over all ties; 65: the K rounds), 32 and 33, and a row of signed zeros."""
    rows = [rng.standard_normal(E).astype(np.float32) for _ in range(40)]
    rows.append(np.full(E, 0.5, np.float32))
    for n_top in (32, 33, 64, 65, E // 2, E - 1):
        if 0 < n_top <= E:
            r = (rng.standard_normal(E) - 5.0).astype(np.float32)
            r[rng.permutation(E)[:n_top]] = 3.0
            r2 = r.copy()
            r2[:] = -3.0
            r2[:n_top] = 3.0
            rows += [r, r2]
    z = np.zeros(E, np.float32)
    z[::2] = -0.0
    rows.append(z)
    return np.stack(rows)


@pytest.mark.parametrize("E,K", [(8, 8), (64, 8), (65, 1), (100, 3), (128, 9), (250, 8), (256, 8), (256, 16), (257, 8),
                                 (512, 8), (512, 13)])
def test_route_threshold_and_rounds(E, K):
    """Choices exactly the oracle's (score desc, id asc) on rows that take the threshold-and-rank path and
    rows that take the K rounds, interleaved so that one wave meets both; gates within tolerance; a rerun
    bitwise identical."""
    rng = np.random.default_rng(E * 7 + K)
    block = _threshold_rows(E, rng)
    logits = np.concatenate([block[rng.permutation(len(block))] for _ in range(40)])
    T = len(logits)
    print(f"[route paths] E={E} K={K} T={T}", flush=True)
    d = torch.from_numpy(logits).cuda()
    idx, g = _lib.moe_route(d, K)
    idx2, g2 = _lib.moe_route(d, K)
    torch.cuda.synchronize()
    ref_idx, ref_g = oracle.route(logits, K)
    assert_equal("topk_idx", bits(idx), ref_idx)
    assert_close("gates", bits(g), ref_g)
    assert torch.equal(idx, idx2) and torch.equal(g.view(torch.int32), g2.view(torch.int32))


# (T, K, local experts): the permute's schedules.  64-token blocks with the scan done inside the rank
# kernel (at most 256 blocks; 256 exactly for T=16384), 64-token blocks with the per-expert row scan
# (313 blocks), and 256-token blocks (blocks x local experts above 8192) with the row scan, up to
# 782 blocks per expert.
@pytest.mark.parametrize("T,K,EL", [(8192, 8, 40), (8193, 8, 40), (16384, 4, 16), (20000, 4, 16), (20000, 4, 40),
                                    (131072, 2, 32), (200000, 2, 40)])
def test_permute_local_share_and_capacity(T, K, EL):
    """A local share (experts 8.. of 64) at several thousand tokens: counts, offsets, pos, src and
    x_perm exactly as the oracle's, with the expected capacity and with half of it (rows dropped)."""
    shape = synth.MoeShape(f"paths_T{T}_K{K}", 93, T=T, H=64, F=64, E=64, K=K, e_begin=8, e_local=EL)
    inp = synth.make_inputs(shape, seed=5)
    dev = pipeline.to_device(inp)
    for cap in (shape.cap, shape.T * shape.K * EL // 64 // 2):
        buf = pipeline.MoeBuffers.allocate(shape, cap=cap, backward=False)
        pipeline.route(buf, dev["logits"])
        pipeline.permute(buf, dev["x"])
        torch.cuda.synchronize()
        idx, _ = oracle.route(inp["logits"], K)
        ref = oracle.permute(idx, shape.e_begin, shape.EL, inp["x"], cap)
        R = min(int(ref["offsets"][-1]), cap)
        assert_equal("counts", bits(buf.counts)[:shape.EL], ref["counts"])
        assert_equal("offsets", bits(buf.offsets), ref["offsets"])
        assert_equal("pos", bits(buf.pos), ref["pos"])
        assert_equal("src", bits(buf.src)[:R], ref["src"][:R])
        assert_equal("status", bits(buf.status)[0], ref["status"])
        assert_equal("x_perm", bits(buf.x_perm)[:R], ref["x_perm"][:R])


@pytest.mark.parametrize("tile", ["256", "192", "128"])
@pytest.mark.parametrize("name", ["ep_share_small", "fwdbwd_small"])
def test_layer_matches_oracle_in_every_tile_configuration(name, tile, monkeypatch):
    """The automatic choice takes the 192-row body at these sizes; pin each GroupGEMM configuration
    (MOE_GEMM_TILE, read on every call) and check the whole layer element by element."""
    monkeypatch.setenv("MOE_GEMM_TILE", tile)
    shape = SMALL[name]
    inp = synth.make_inputs(shape, seed=4, d_out=True)
    buf, _ = run_gpu(shape, inp)
    check_layer(shape, inp, buf, shape.cap)


# Row counts on each side of the 32-row MFMA blocks and of the 128/192/256-row tiles: the 128- and
# 192-row bodies run only the MFMA rows that hold valid rows, with the row blocks dealt to the two
# wave rows in turn, so a tile of up to 32 rows leaves one wave row without a valid block.
EDGE_COUNTS = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 160, 161, 191, 192, 193, 255, 256, 257,
               0, 300]


@pytest.mark.parametrize("tile", ["0", "256", "192", "128"])
def test_gemms_at_row_block_edges(tile, monkeypatch):
    """Gate/up (copy and zero-copy), down and down-dgrad GroupGEMMs on experts whose row counts sit at
    every row-block and tile edge, element by element against the oracle, in each tile configuration
    (0: the automatic choice)."""
    monkeypatch.setenv("MOE_GEMM_TILE", tile)
    counts = np.array(EDGE_COUNTS, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R, EL, H, F, K = int(offsets[-1]), len(counts), 128, 192, 1
    x_perm = synth.operand_bf16((R, H), seed=31, tag=1)
    wg = synth.operand_bf16((EL, H, F), seed=31, tag=2, std=0.05)
    wu = synth.operand_bf16((EL, H, F), seed=31, tag=3, std=0.05)
    wd = synth.operand_bf16((EL, F, H), seed=31, tag=4, std=0.05)
    hin = synth.operand_bf16((R, F), seed=31, tag=5)
    dev = pipeline.to_device(dict(x=x_perm, wg=wg, wu=wu, wd=wd, h=hin, off=offsets,
                                  src=np.arange(R, dtype=np.int32)))
    h = torch.empty((R, F), dtype=torch.bfloat16, device="cuda")
    ab = torch.empty((R, 2 * F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm_swiglu(dev["x"], dev["wg"], dev["wu"], dev["off"], R, h=h, ab_save=ab)
    # zero-copy with K = 1: row r of the grouped order is token src[r] = r
    hz = torch.empty_like(h)
    _lib.moe_grouped_gemm_swiglu_gather(dev["x"], dev["src"], K, dev["wg"], dev["wu"], dev["off"], R, h=hz)
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(dev["h"], dev["wd"], None, 0, dev["off"], F, H, R, y)
    # down dgrad with the SwiGLU-backward epilogue: W_down read transposed ([N][Kd], the layer's
    # backward) and, through the same entry point, a weight stored [Kd][N]
    dy = synth.operand_bf16((R, H), seed=31, tag=6, std=0.125)
    abin = synth.operand_bf16((R, 2 * F), seed=31, tag=7)
    wdT = np.ascontiguousarray(np.transpose(wd, (0, 2, 1)))
    d2 = pipeline.to_device(dict(dy=dy, ab=abin, wdT=wdT))
    dab = torch.empty((R, 2 * F), dtype=torch.bfloat16, device="cuda")
    dab2 = torch.empty_like(dab)
    _lib.moe_grouped_gemm(d2["dy"], dev["wd"], None, 1, dev["off"], H, F, R, dab, epilogue=_lib.MOE_EPI_SWIGLU_BWD,
                          ab=d2["ab"])
    _lib.moe_grouped_gemm(d2["dy"], d2["wdT"], None, 0, dev["off"], H, F, R, dab2,
                          epilogue=_lib.MOE_EPI_SWIGLU_BWD, ab=d2["ab"])
    torch.cuda.synchronize()
    ref_dab = oracle.bwd_down(dy, wd, abin, offsets, R)
    assert_close("dab (W_down transposed)", bits(dab), ref_dab)
    assert_close("dab (weight [Kd][N])", bits(dab2), ref_dab)
    ref_h, ref_ab = oracle.expert_up(x_perm, wg, wu, offsets, R, want_ab=True)
    assert_close("h", bits(h), ref_h)
    assert_close("ab_save", bits(ab), ref_ab)
    assert torch.equal(h.view(torch.int16), hz.view(torch.int16))
    assert_close("y", bits(y), oracle.expert_down(hin, wd, offsets, R))


def test_binding_rejects_undersized_outputs():
    """A caller buffer that is too small is refused before any kernel runs."""
    shape = SMALL["tiny"]
    inp = synth.make_inputs(shape, seed=1)
    dev = pipeline.to_device(inp)
    buf = pipeline.MoeBuffers.allocate(shape, backward=False)
    pipeline.forward(buf, dev)
    T, H, K = shape.T, shape.H, shape.K
    with pytest.raises(_lib.MoeError):
        _lib.moe_combine(buf.y, buf.pos, buf.gates, out=torch.empty((T - 1, H), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(_lib.MoeError):
        _lib.moe_route(dev["logits"], K, topk_idx=torch.empty((T, K - 1), dtype=torch.int32, device="cuda"))
    with pytest.raises(_lib.MoeError):
        _lib.moe_grouped_gemm_swiglu(buf.x_perm, dev["w_gate"], dev["w_up"], buf.offsets, buf.cap,
                                     h=torch.empty((buf.cap - 1, shape.F), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()


def _bf16_exact(x):
    """bf16 bit patterns of float32 values that bf16 represents exactly (checked)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("trans_w", [0, 1])
@pytest.mark.parametrize("tile", ["0", "256", "192", "128"])
def test_bf16_epilogue_rounds_exact_ties_to_even(trans_w, tile, monkeypatch):
    """The plain bf16 epilogue (down GEMM: weights [Kd][N]; dgrad bodies: [N][Kd]) on dot products that
    are exact in fp32 and sit on a bf16 rounding tie (both parities of the mantissa below it) or one fp32
    step to either side of one: the stored bits must equal the oracle's round-to-nearest-even exactly.
    Two non-zero terms per row make every sum exact, so the order of accumulation cannot matter."""
    monkeypatch.setenv("MOE_GEMM_TILE", tile)
    rng = np.random.default_rng(5)
    counts = np.array([300, 211], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R, EL, Kd, N = int(offsets[-1]), len(counts), 64, 320
    e = rng.integers(-20, 20, R).astype(np.float64)
    kind = rng.integers(0, 5, R)
    big = 2.0 ** e
    # relative to the bf16 ulp 2^(e-7) of big: half an ulp above an odd or an even mantissa (exact ties),
    # and just above and below a tie
    small = np.select([kind == 0, kind == 1, kind == 2, kind == 3],
                      [3 * 2.0 ** (e - 8), 2.0 ** (e - 8), 2.0 ** (e - 8) * (1 + 2.0 ** -7),
                       2.0 ** (e - 9) * (2 - 2.0 ** -7)], 2.0 ** (e - 8) * 5)
    a = rng.standard_normal((R, Kd)).astype(np.float32)
    a[:, 0] = big
    a[:, 1] = small
    # the other columns: any bf16 values (their weights are 0)
    a_bits = _bf16_exact((a.view(np.uint32) & 0xFFFF0000).view(np.float32))
    a_bits[:, 0] = _bf16_exact(big.astype(np.float32))
    a_bits[:, 1] = _bf16_exact(small.astype(np.float32))
    w = np.zeros((EL, Kd, N), np.float32)  # [Kd][N]: rows 0 and 1 scale by a power of two, the rest 0
    scale = 2.0 ** ((np.arange(N) % 4) - 1)
    w[:, 0, :] = scale
    w[:, 1, :] = scale
    w_bits = _bf16_exact(w)
    ref = oracle.expert_down(a_bits, w_bits, offsets, R)
    dev = pipeline.to_device(dict(a=a_bits, off=offsets))
    wt = np.ascontiguousarray(w_bits.transpose(0, 2, 1)) if trans_w else w_bits
    wdev = pipeline.to_device(dict(w=wt))["w"]
    y = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(dev["a"], wdev, None, trans_w, dev["off"], Kd, N, R, y)
    torch.cuda.synchronize()
    got = bits(y)
    assert_equal("y", got, ref)
    # the construction really exercises both tie directions
    exact = (big + small)[:, None] * scale[None, :]
    assert np.any((kind == 0)) and np.any(kind == 1)
    assert np.all(np.float32(exact) == exact)


@pytest.mark.parametrize("gated", [True, False])
def test_combine_rounds_exact_ties_to_even(gated):
    """The combine (gated forward and ungated combine-gradient) on tokens whose K = 3 contributions (one of
    them a row absent from the layer's share, pos < 0) sum exactly in fp32 to a bf16 tie of either mantissa
    parity, or one step beside one: the stored bits must equal the oracle's round-to-nearest-even."""
    rng = np.random.default_rng(9)
    T, K, H = 777, 3, 192
    e = rng.integers(-20, 20, (T, 1)).astype(np.float64)
    kind = rng.integers(0, 5, (T, 1))
    big = np.broadcast_to(2.0 ** e, (T, H))
    small = np.select([kind == 0, kind == 1, kind == 2, kind == 3],
                      [3 * 2.0 ** (e - 8), 2.0 ** (e - 8), 2.0 ** (e - 8) * (1 + 2.0 ** -7),
                       2.0 ** (e - 9) * (2 - 2.0 ** -7)], 2.0 ** (e - 8) * 5)
    small = np.broadcast_to(small, (T, H)) * np.where(rng.random((1, H)) < 0.5, 1.0, -1.0)
    # rows: token t's contributions at rows 2t (big) and 2t + 1 (small); the third pair is absent
    y = np.zeros((2 * T, H), np.float32)
    y[0::2] = big / 2  # the gate 2 (a power of two) makes the products exact
    y[1::2] = small
    pos = np.stack([np.arange(T) * 2, np.full(T, -1), np.arange(T) * 2 + 1], axis=1).astype(np.int32)
    g = np.stack([np.full(T, 2.0), np.full(T, 0.75), np.full(T, 1.0)], axis=1).astype(np.float32)
    if not gated:
        y[0::2] = big
    y_bits = _bf16_exact(y)
    ref = oracle.combine(y_bits, pos, g if gated else None)
    dev = pipeline.to_device(dict(y=y_bits, pos=pos, g=g))
    out = _lib.moe_combine(dev["y"], dev["pos"], dev["g"] if gated else None)
    torch.cuda.synchronize()
    assert_equal("out", bits(out), ref)
    exact = big + small
    assert np.all(np.float32(exact) == exact)


@pytest.mark.parametrize("fused", [False, True])
def test_gather_rounds_exact_ties_to_even(fused):
    """The output-gradient gather (alone and fused with the gate gradient): g * dOut with dOut a signed
    power of two and g chosen so that the fp32 product is exact and sits on a bf16 tie of either mantissa
    parity, beside one, or on a representable value; the stored rows must equal the oracle's bits."""
    rng = np.random.default_rng(13)
    T, K, H = 600, 2, 128
    d_out = (2.0 ** rng.integers(-12, 12, (T, H))) * np.where(rng.random((T, H)) < 0.5, 1.0, -1.0)
    choices = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, 0.75, 1 + 2.0 ** -8 + 2.0 ** -20],
                       np.float64)
    g = choices[rng.integers(0, len(choices), (T, K))].astype(np.float32)
    pos = (np.arange(T * K, dtype=np.int32).reshape(T, K))
    d_bits = _bf16_exact(d_out.astype(np.float32))
    offsets = np.array([0, T * K], np.int32)
    ref = oracle.bwd_gather(d_bits, np.arange(T * K, dtype=np.int32), offsets, g, K, T * K)
    dev = pipeline.to_device(dict(d=d_bits, pos=pos, g=g))
    dy = torch.empty((T * K, H), dtype=torch.bfloat16, device="cuda")
    if fused:
        y = torch.zeros((T * K, H), dtype=torch.bfloat16, device="cuda")
        _lib.moe_gather_gate_grad(dev["d"], dev["pos"], dev["g"], y, dy)
    else:
        _lib.moe_gather(dev["d"], dev["pos"], dev["g"], dy)
    torch.cuda.synchronize()
    assert_equal("dy_perm", bits(dy), ref)
    exact = d_out[:, None, :] * g.astype(np.float64)[:, :, None]
    assert np.all(np.float32(exact) == exact)


def _int_bf16(rng, shape, lo, hi):
    """bf16 bits of small integers (exact in bf16) drawn from [lo, hi]."""
    return _bf16_exact(rng.integers(lo, hi + 1, shape).astype(np.float32))


@pytest.mark.parametrize("tile", ["0", "256", "192", "128"])
def test_gemms_exact_on_integer_operands(tile, monkeypatch):
    """Every GroupGEMM data path on integer operands, whose products and sums are exact in fp32, so that
    any order of accumulation gives the same sum and the stored bits must equal the oracle's exactly: a
    row, column or k-step taken twice, skipped or taken from a neighbouring expert changes them.  Experts
    sit at every row-block and tile edge; N is not a multiple of the tile width.  Checked: the saved
    (a, b) of the gate/up GEMM (copy and zero-copy), the down GEMM, the gate/up dgrad over both
    weights, dW_gate, dW_up (one pass, copy and zero-copy) and dW_down in fp32, and the down dgrad with
    its SwiGLU-backward epilogue at a saved a of 0, where the sigmoid is exactly 1/2."""
    monkeypatch.setenv("MOE_GEMM_TILE", tile)
    rng = np.random.default_rng(17)
    counts = np.array(EDGE_COUNTS, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R, EL, H, F, K = int(offsets[-1]), len(counts), 320, 192, 1
    x = _int_bf16(rng, (R, H), -2, 2)
    wg = _int_bf16(rng, (EL, H, F), -1, 1)
    wu = _int_bf16(rng, (EL, H, F), -1, 1)
    wd = _int_bf16(rng, (EL, F, H), -1, 1)
    hin = _int_bf16(rng, (R, F), -2, 2)
    dabin = _int_bf16(rng, (R, 2 * F), -2, 2)
    dev = pipeline.to_device(dict(x=x, wg=wg, wu=wu, wd=wd, h=hin, dab=dabin, off=offsets,
                                  src=np.arange(R, dtype=np.int32)))
    h = torch.empty((R, F), dtype=torch.bfloat16, device="cuda")
    ab = torch.empty((R, 2 * F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm_swiglu(dev["x"], dev["wg"], dev["wu"], dev["off"], R, h=h, ab_save=ab)
    abz = torch.empty_like(ab)
    _lib.moe_grouped_gemm_swiglu_gather(dev["x"], dev["src"], K, dev["wg"], dev["wu"], dev["off"], R,
                                        h=torch.empty_like(h), ab_save=abz)
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(dev["h"], dev["wd"], None, 0, dev["off"], F, H, R, y)
    dx = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    # [W_gate; W_up] as stored, [H][F] each: the contraction runs over F of both segments
    _lib.moe_grouped_gemm(dev["dab"], dev["wg"], dev["wu"], 1, dev["off"], F, H, R, dx)
    dwg, dwu = _lib.moe_wgrad_gate_up(dev["x"], dev["dab"], dev["off"], EL, R)
    zwg, zwu = _lib.moe_wgrad_gate_up_gather(dev["x"], dev["src"], K, dev["dab"], dev["off"], EL, R)
    dwd = _lib.moe_wgrad(dev["h"], F, dev["x"], H, dev["off"], EL, F, H, R)
    # the down dgrad with a saved a of 0 (sigmoid 1/2 exactly): da = dh * b / 2 and db = 0, exact
    ab0 = dabin.copy()
    ab0[:, :F] = 0
    dy = _int_bf16(rng, (R, H), -2, 2)
    d3 = pipeline.to_device(dict(ab0=ab0, dy=dy))
    dab = torch.empty((R, 2 * F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(d3["dy"], dev["wd"], None, 1, dev["off"], H, F, R, dab, epilogue=_lib.MOE_EPI_SWIGLU_BWD,
                          ab=d3["ab0"])
    torch.cuda.synchronize()
    _, ref_ab = oracle.expert_up(x, wg, wu, offsets, R, want_ab=True)
    assert_equal("ab_save", bits(ab), ref_ab)
    assert_equal("ab_save (zero-copy)", bits(abz), ref_ab)
    assert_equal("y", bits(y), oracle.expert_down(hin, wd, offsets, R))
    assert_equal("dx_perm", bits(dx), oracle.bwd_up(dabin, wg, wu, offsets, R))
    ref_g = oracle.wgrad(x, H, dabin, 2 * F, offsets, H, F, R)
    ref_u = oracle.wgrad(x, H, dabin.reshape(-1)[F:], 2 * F, offsets, H, F, R)  # db: columns F.. of dab
    assert_equal("dW_gate", dwg.cpu().numpy(), ref_g)
    assert_equal("dW_up", dwu.cpu().numpy(), ref_u)
    assert_equal("dW_gate (zero-copy)", zwg.cpu().numpy(), ref_g)
    assert_equal("dW_up (zero-copy)", zwu.cpu().numpy(), ref_u)
    assert_equal("dW_down", dwd.cpu().numpy(), oracle.wgrad(hin, F, x, H, offsets, F, H, R))
    assert_equal("dab (a = 0)", bits(dab), oracle.bwd_down(dy, wd, ab0, offsets, R))


def test_gate_grad_and_route_backward_exact_on_exact_values():
    """The gate gradient (the fused gather's fp32 dot products, finished by a lane butterfly) and the
    softmax/top-k backward (a fused multiply-add chain) on values whose every product and sum is exact in
    fp32 (small integers; gates of a few bits), so that any order of the sums gives the same result: both
    must equal the oracle's bits, with exactly 0 at pairs without a local row and at unchosen experts."""
    rng = np.random.default_rng(29)
    T, K, H, E = 500, 8, 192, 64
    table = np.array([np.float32(v).view(np.uint32) >> 16 for v in range(-2, 3)], np.uint16)
    d_out = table[rng.integers(0, 5, (T, H), dtype=np.int8)]
    R = T * K
    y = table[rng.integers(0, 5, (R, H), dtype=np.int8)]
    pos = np.arange(R, dtype=np.int32).reshape(T, K)
    pos[rng.random((T, K)) < 0.2] = -1  # pairs without a local row
    gates = (rng.integers(1, 8, (T, K)) / 8.0).astype(np.float32)
    dev = pipeline.to_device(dict(d=d_out, y=y, pos=pos, g=gates))
    dy = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _, dg = _lib.moe_gather_gate_grad(dev["d"], dev["pos"], dev["g"], dev["y"], dy)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    dgi = rng.integers(-4, 5, (T, K)).astype(np.float32)
    d2 = pipeline.to_device(dict(idx=idx, dgi=dgi))
    dl = _lib.moe_route_backward(d2["idx"], dev["g"], d2["dgi"], E)
    torch.cuda.synchronize()
    assert_equal("dgates", dg.cpu().numpy(), oracle.gate_grad(d_out, y, pos))
    assert_equal("dlogits", dl.cpu().numpy(), oracle.route_backward(idx, gates, dgi, E))
