"""Pins of the CPU oracle against things other than itself (CPU only).

Every oracle function is checked here against brute force, an fp64 library
routine (numpy matmul, numpy stable argsort, scipy softmax/expit, torch
autograd), a closed form or an invariant, chosen so that a dropped term, a
wrong sign, a wrong index or a transposed operand fails at least one test.
Error bounds: an fp32 running sum of n exact products is within
gamma_n * sum|a*b| of the exact value (Higham, gamma_n = n*u/(1-n*u),
u = 2^-24); rounding to bf16 adds at most 2^-8 relative.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from routing_permute_groupgemm_amd import synth

U32 = 2.0 ** -24
U16 = 2.0 ** -8
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gamma(n):
    return n * U32 / (1 - n * U32)


def f(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def rand_bf16(rng, shape, std=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38], np.float32),
        # exact ties: 1 + 2^-8 (tie, round to even -> 1), 1 + 3*2^-8 (tie -> up)
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32),
    ])
    want = synth.f32_to_bf16_bits(vals)
    got = np.array([oracle.f32_to_bf16(v) for v in vals], np.uint16)
    assert np.array_equal(got, want)
    assert oracle.f32_to_bf16(1 + 2 ** -8) == 0x3F80
    assert oracle.f32_to_bf16(1 + 3 * 2 ** -8) == 0x3F82
    assert oracle.f32_to_bf16(float("nan")) & 0x7F80 == 0x7F80


# ---------------------------------------------------------------- route

def brute_topk(logits, K):
    T, E = logits.shape
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        idx[t] = order[:K]
    return idx


@pytest.mark.parametrize("T,E,K", [(64, 8, 2), (33, 256, 8), (40, 128, 8), (16, 5, 5), (20, 7, 1)])
def test_route_indices_brute_force(T, E, K):
    rng = np.random.default_rng(T * E + K)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # plant exact ties and signed zeros in a few tokens
    logits[0, :] = 0.0
    logits[1, ::2] = -0.0
    logits[2, 1] = logits[2, 3] = logits[2].max() + 1
    idx, _ = oracle.route(logits, K)
    assert np.array_equal(idx, brute_topk(logits, K))


def test_route_k1_is_first_argmax_and_k_eq_e_is_full_order():
    rng = np.random.default_rng(1)
    logits = np.round(rng.standard_normal((50, 16)), 1).astype(np.float32)  # many ties
    idx1, g1 = oracle.route(logits, 1)
    assert np.array_equal(idx1[:, 0], np.argmax(logits, axis=1))
    assert np.all(g1 == 1.0)
    idxE, _ = oracle.route(logits, 16)
    assert all(sorted(r) == list(range(16)) for r in idxE)


def test_route_gates_vs_fp64_softmax():
    rng = np.random.default_rng(2)
    logits = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    K = 6
    idx, g = oracle.route(logits, K)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(g - ref) / ref) < 1e-5
    assert np.all(np.abs(g.sum(axis=1, dtype=np.float64) - 1.0) <= K * 2.0 ** -23)
    assert np.all(np.diff(g, axis=1) <= 0)


def test_route_two_experts_closed_form():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((100, 2)).astype(np.float32)
    idx, g = oracle.route(logits, 2)
    s = logits.astype(np.float64)
    hi = np.maximum(s[:, 0], s[:, 1])
    lo = np.minimum(s[:, 0], s[:, 1])
    assert np.allclose(g[:, 0], 1 / (1 + np.exp(lo - hi)), rtol=4e-7, atol=0)


def test_route_golden_ties():
    with open(os.path.join(GOLDEN, "route_ties.json")) as fh:
        gold = json.load(fh)
    for case in gold["cases"]:
        logits = np.array(case["logits"], np.float32)
        idx, g = oracle.route(logits, case["K"])
        assert idx.tolist() == case["topk_idx"], case["name"]
        if "gates" in case:
            assert np.allclose(g, np.array(case["gates"]), rtol=1e-6, atol=0), case["name"]


# ---------------------------------------------------------------- permute

def reference_permute(idx, e_begin, e_local):
    flat = idx.reshape(-1).astype(np.int64)
    local = (flat >= e_begin) & (flat < e_begin + e_local)
    pairs = np.nonzero(local)[0]
    order = np.argsort(flat[pairs] - e_begin, kind="stable")
    src = pairs[order]
    counts = np.bincount(flat[pairs] - e_begin, minlength=e_local)
    pos = np.full(flat.shape, -1, np.int64)
    pos[src] = np.arange(len(src))
    return counts, src, pos.reshape(idx.shape)


@pytest.mark.parametrize("T,E,K,eb,el", [(256, 8, 2, 0, 8), (300, 64, 8, 16, 16), (97, 32, 4, 0, 32),
                                         (50, 16, 3, 10, 6), (10, 8, 2, 0, 0)])
def test_permute_equals_stable_argsort(T, E, K, eb, el):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    x = rand_bf16(rng, (T, 24))
    cap = T * K
    pm = oracle.permute(idx, eb, el, x, cap)
    counts, src, pos = reference_permute(idx, eb, el)
    R = len(src)
    assert np.array_equal(pm["counts"], counts)
    assert np.array_equal(pm["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(pm["src"][:R], src)
    assert np.array_equal(pm["pos"], pos)
    assert np.array_equal(pm["x_perm"][:R], x[src // K])
    assert pm["status"] == 0
    # invariants: stable (ascending token) within each expert; src o pos = id
    for j in range(el):
        rows = pm["src"][pm["offsets"][j]:pm["offsets"][j + 1]]
        assert np.all(np.diff(rows // K) > 0)
        assert np.all(idx.reshape(-1)[rows] == eb + j)
    loc = pm["pos"] >= 0
    assert np.array_equal(pm["src"][pm["pos"][loc]], np.nonzero(loc.reshape(-1))[0])
    if el == E:
        assert np.all(np.bincount(pm["src"][:R] // K, minlength=T) == K)


def test_permute_overflow_drops_tail_rows():
    rng = np.random.default_rng(5)
    T, E, K = 64, 4, 2
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    full = oracle.permute(idx, 0, E, None, T * K)
    cap = 50
    pm = oracle.permute(idx, 0, E, None, cap)
    assert pm["status"] == 1
    assert np.array_equal(pm["offsets"], full["offsets"])  # true totals are reported
    keep = full["pos"] < cap
    assert np.array_equal(pm["pos"][keep], full["pos"][keep])
    assert np.all(pm["pos"][~keep] == -1)
    assert np.array_equal(pm["src"][:cap], full["src"][:cap])


# ---------------------------------------------------------------- GEMMs

def grouped_setup(rng, counts, H, F):
    EL = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    x = rand_bf16(rng, (R, H))
    wg = rand_bf16(rng, (EL, H, F), 0.05)
    wu = rand_bf16(rng, (EL, H, F), 0.05)
    return offsets, R, x, wg, wu


@pytest.mark.parametrize("counts", [[37], [5, 0, 19, 1]])
def test_expert_up_vs_fp64_matmul(counts):
    rng = np.random.default_rng(sum(counts))
    H, F = 96, 40
    offsets, R, x, wg, wu = grouped_setup(rng, counts, H, F)
    h, ab = oracle.expert_up(x, wg, wu, offsets, R)
    for j in range(len(counts)):
        rs = slice(offsets[j], offsets[j + 1])
        X = f(x[rs])
        a64, b64 = X @ f(wg[j]), X @ f(wu[j])
        ba = gamma(H) * (np.abs(X) @ np.abs(f(wg[j])))
        bb = gamma(H) * (np.abs(X) @ np.abs(f(wu[j])))
        a_o, b_o = f(ab[rs, :F]), f(ab[rs, F:])
        assert np.all(np.abs(a_o - a64) <= ba + U16 * np.abs(a64) * 1.0001)
        assert np.all(np.abs(b_o - b64) <= bb + U16 * np.abs(b64) * 1.0001)
        # SwiGLU against scipy's logistic: silu(a) = a * expit(a), gate half
        h64 = a64 * scipy.special.expit(a64) * b64
        da = ba + 1e-6 * np.abs(a64)
        db = bb + 1e-6 * np.abs(b64)
        bound = 1.1 * da * np.abs(b64) + np.abs(a64) * db + U16 * np.abs(h64) * 1.01 + 1e-30
        assert np.all(np.abs(f(h[rs]) - h64) <= bound)


def test_swiglu_special_values():
    # one-hot x rows make a and b exact bf16 values; then h is a function of (a, b) alone
    vals = np.array([0.0, 20.0, -20.0, 1.0, -1.0, 3.5], np.float32)
    F = len(vals)
    H = 1
    x = synth.f32_to_bf16_bits(np.ones((1, H), np.float32))
    wg = synth.f32_to_bf16_bits(vals.reshape(1, H, F))
    wu = synth.f32_to_bf16_bits(np.full((1, H, F), 2.0, np.float32))
    h, ab = oracle.expert_up(x, wg, wu, np.array([0, 1], np.int32), 1)
    hv = f(h[0])
    assert hv[0] == 0.0                         # silu(0) = 0
    assert hv[1] == f(synth.f32_to_bf16_bits(np.array([40.0], np.float32)))[0]  # silu(20)*2 ~ 40
    assert abs(hv[2]) < 1e-7                    # silu(-20) ~ -4e-8
    ref = vals.astype(np.float64) * scipy.special.expit(vals.astype(np.float64)) * 2.0
    assert np.all(np.abs(hv - ref) <= U16 * np.abs(ref) + 1e-7)


@pytest.mark.parametrize("counts", [[23], [0, 7, 12]])
def test_expert_down_vs_fp64_matmul(counts):
    rng = np.random.default_rng(100 + sum(counts))
    F, H = 72, 48
    EL = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    h = rand_bf16(rng, (R, F))
    wd = rand_bf16(rng, (EL, F, H), 0.05)
    y = oracle.expert_down(h, wd, offsets, R)
    for j in range(EL):
        rs = slice(offsets[j], offsets[j + 1])
        ref = f(h[rs]) @ f(wd[j])
        bnd = gamma(F) * (np.abs(f(h[rs])) @ np.abs(f(wd[j]))) + U16 * np.abs(ref) * 1.0001
        assert np.all(np.abs(f(y[rs]) - ref) <= bnd)


def test_row_subset_matches_full():
    rng = np.random.default_rng(9)
    offsets, R, x, wg, wu = grouped_setup(rng, [9, 4, 11], 32, 16)
    h, ab = oracle.expert_up(x, wg, wu, offsets, R)
    rows = np.array([0, 8, 9, 23], np.int64)
    hs, abs_ = oracle.expert_up(x, wg, wu, offsets, R, rows=rows)
    assert np.array_equal(hs[rows], h[rows]) and np.array_equal(abs_[rows], ab[rows])


def test_subset_modes_match_full_results():
    """Every oracle mode that fills only some rows, tokens or groups (used at full size, where the full
    result is out of reach) writes exactly what the full call writes there, and zeros elsewhere: a
    subset path that indexed outputs by position in the subset rather than by the true row, token or
    group would fail."""
    inp, fwd, bwd, cap = _small_layer()
    offsets = fwd["offsets"]
    R = int(offsets[-1])
    rows = np.array([0, 1, R // 3, R // 2, R - 1], np.int64)
    others = np.setdiff1d(np.arange(cap), rows)
    # expert_down, bwd_down, bwd_up on a row subset
    y_s = oracle.expert_down(fwd["h"], inp["w_down"], offsets, cap, rows=rows)
    dab_s = oracle.bwd_down(bwd["dy_perm"], inp["w_down"], fwd["ab"], offsets, cap, rows=rows)
    dxp_s = oracle.bwd_up(bwd["dab"], inp["w_gate"], inp["w_up"], offsets, cap, rows=rows)
    for name, sub, full in (("y", y_s, fwd["y"]), ("dab", dab_s, bwd["dab"]), ("dx_perm", dxp_s, bwd["dx_perm"])):
        assert np.array_equal(sub[rows], full[rows]), name
        assert not sub[others].any(), name
    # combine on a token subset (gated forward and the ungated combine-gradient)
    T = fwd["pos"].shape[0]
    toks = np.array([0, 3, T // 2, T - 1], np.int64)
    rest = np.setdiff1d(np.arange(T), toks)
    out_s = oracle.combine(fwd["y"], fwd["pos"], fwd["gates"], tokens=toks)
    dx_s = oracle.combine(bwd["dx_perm"], fwd["pos"], None, tokens=toks)
    for name, sub, full in (("out", out_s, fwd["out"]), ("dx", dx_s, bwd["dx"])):
        assert np.array_equal(sub[toks], full[toks]), name
        assert not sub[rest].any(), name
    # wgrad on a group subset, also with a column subset
    H = inp["w_gate"].shape[1]
    F = inp["w_gate"].shape[2]
    EL = len(offsets) - 1
    groups = np.array([EL - 1, 0], np.int32)
    g_s = oracle.wgrad(fwd["x_perm"], H, bwd["dab"], 2 * F, offsets, H, F, cap, groups=groups)
    for j in range(EL):
        if j in groups:
            assert np.array_equal(g_s[j].view(np.uint32), bwd["dw_gate"][j].view(np.uint32)), j
        else:
            assert not g_s[j].any(), j
    cols = np.array([F - 1, 2], np.int32)
    gc = oracle.wgrad(fwd["x_perm"], H, bwd["dab"], 2 * F, offsets, H, F, cap, groups=groups, cols=cols)
    for j in groups:
        assert np.array_equal(gc[j][:, cols].view(np.uint32), bwd["dw_gate"][j][:, cols].view(np.uint32))
        assert not np.delete(gc[j], cols, axis=1).any()


# ---------------------------------------------------------------- combine

def test_combine_identity_expert_k1_is_bit_exact():
    rng = np.random.default_rng(11)
    T, E, K = 128, 8, 1
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rand_bf16(rng, (T, 64))
    idx, g = oracle.route(logits, K)
    assert np.all(g == 1.0)
    pm = oracle.permute(idx, 0, E, x, T * K)
    out = oracle.combine(pm["x_perm"], pm["pos"], g)  # y = x_perm (identity experts)
    assert np.array_equal(out, x)


def test_combine_vs_fp64_weighted_sum_and_nonlocal_tokens():
    rng = np.random.default_rng(12)
    T, E, K, H = 200, 16, 4, 40
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, g = oracle.route(logits, K)
    el = 5
    pm = oracle.permute(idx, 3, el, None, T * K)
    R = int(pm["offsets"][-1])
    y = rand_bf16(rng, (T * K, H))
    out = oracle.combine(y, pm["pos"], g)
    ref = np.zeros((T, H))
    mag = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            r = pm["pos"][t, k]
            if r >= 0:
                ref[t] += float(g[t, k]) * f(y[r])
                mag[t] += abs(float(g[t, k])) * np.abs(f(y[r]))
    bound = (K + 1) * U32 * mag * 1.01 + U16 * np.abs(ref) * 1.0001
    assert np.all(np.abs(f(out) - ref) <= bound)
    none_local = np.all(pm["pos"] < 0, axis=1)
    assert none_local.any()
    assert np.all(out[none_local] == 0)  # +0 bit pattern
    # ungated combine (combine-gradient): plain sum in k order
    out1 = oracle.combine(y, pm["pos"], None)
    ref1 = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            if pm["pos"][t, k] >= 0:
                ref1[t] += f(y[pm["pos"][t, k]])
    assert np.all(np.abs(f(out1) - ref1) <= (K * U32 * 4 + U16) * np.abs(ref1) + 1e-6 * 0 + K * U32 * 8)
    assert R > 0


# ---------------------------------------------------------------- backward

def _small_layer(seed=21, T=48, H=64, F=32, E=6, K=2, el=6, eb=0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    inp = dict(logits=logits, x=rand_bf16(rng, (T, H)),
               w_gate=rand_bf16(rng, (el, H, F), 0.1), w_up=rand_bf16(rng, (el, H, F), 0.1),
               w_down=rand_bf16(rng, (el, F, H), 0.1), d_out=rand_bf16(rng, (T, H)))
    cap = T * K
    fwd = oracle.forward(inp, eb, el, K, cap)
    bwd = oracle.backward(inp, fwd, cap)
    return inp, fwd, bwd, cap


def test_bwd_gather_scaling():
    inp, fwd, bwd, cap = _small_layer()
    R = int(fwd["offsets"][-1])
    K = fwd["topk_idx"].shape[1]
    t = fwd["src"][:R] // K
    g = fwd["gates"].reshape(-1)[fwd["src"][:R]]
    ref = g[:, None].astype(np.float64) * f(inp["d_out"][t])
    assert np.all(np.abs(f(bwd["dy_perm"][:R]) - ref) <= U16 * np.abs(ref) * 1.0001 + 1e-30)


def test_bwd_swiglu_and_down_dgrad_vs_autograd():
    """dab against torch fp64 autograd of silu(a)*b, fed the oracle's own bf16 inputs."""
    inp, fwd, bwd, cap = _small_layer()
    offsets = fwd["offsets"]
    F = inp["w_gate"].shape[2]
    H = inp["w_gate"].shape[1]
    for j in range(len(offsets) - 1):
        rs = slice(offsets[j], offsets[j + 1])
        if offsets[j] == offsets[j + 1]:
            continue
        dy = torch.tensor(f(bwd["dy_perm"][rs]))
        wd = torch.tensor(f(inp["w_down"][j]))
        a = torch.tensor(f(fwd["ab"][rs, :F]), requires_grad=True)
        b = torch.tensor(f(fwd["ab"][rs, F:]), requires_grad=True)
        dh = dy @ wd.T
        (torch.nn.functional.silu(a) * b * dh).sum().backward()
        da, db = a.grad.numpy(), b.grad.numpy()
        dh_err = gamma(H) * (np.abs(dy.numpy()) @ np.abs(wd.numpy().T))
        an, bn = a.detach().numpy(), b.detach().numpy()
        bda = dh_err * np.abs(bn) * 1.1 + U16 * np.abs(da) + 1e-5 * np.abs(dh.detach().numpy()) * (np.abs(bn) + 1)
        bdb = dh_err * np.abs(an) + U16 * np.abs(db) + 1e-5 * np.abs(dh.detach().numpy()) * (np.abs(an) + 1)
        assert np.all(np.abs(f(bwd["dab"][rs, :F]) - da) <= bda * 1.01)
        assert np.all(np.abs(f(bwd["dab"][rs, F:]) - db) <= bdb * 1.01)


def test_bwd_up_dgrad_vs_fp64_matmul():
    inp, fwd, bwd, cap = _small_layer()
    offsets = fwd["offsets"]
    F = inp["w_gate"].shape[2]
    for j in range(len(offsets) - 1):
        rs = slice(offsets[j], offsets[j + 1])
        D = f(bwd["dab"][rs])
        W = np.concatenate([f(inp["w_gate"][j]), f(inp["w_up"][j])], axis=1)  # [H, 2F]
        ref = D @ W.T
        bnd = gamma(2 * F) * (np.abs(D) @ np.abs(W.T)) + U16 * np.abs(ref) * 1.0001
        assert np.all(np.abs(f(bwd["dx_perm"][rs]) - ref) <= bnd)


def test_wgrad_vs_fp64_brute_force():
    inp, fwd, bwd, cap = _small_layer()
    offsets = fwd["offsets"]
    F = inp["w_gate"].shape[2]
    for j in range(len(offsets) - 1):
        rs = slice(offsets[j], offsets[j + 1])
        n = offsets[j + 1] - offsets[j]
        X, D, Hh, DY = f(fwd["x_perm"][rs]), f(bwd["dab"][rs]), f(fwd["h"][rs]), f(bwd["dy_perm"][rs])
        for got, A, B in ((bwd["dw_gate"][j], X, D[:, :F]), (bwd["dw_up"][j], X, D[:, F:]),
                          (bwd["dw_down"][j], Hh, DY)):
            ref = A.T @ B
            bnd = gamma(max(n, 1)) * (np.abs(A).T @ np.abs(B))
            assert np.all(np.abs(got - ref) <= bnd * 1.0001 + 1e-30)


def test_backward_chain_vs_autograd_of_unrounded_layer():
    """Whole backward against torch fp64 autograd of the layer with no intermediate rounding.

    The oracle rounds ab, h, dy_perm, dab, dx_perm to bf16, so the match is
    normwise (relative error of a few 2^-8); a sign error, a dropped SwiGLU
    term or a transposed weight gives O(1) error.
    """
    inp, fwd, bwd, cap = _small_layer(seed=33, T=64, H=64, F=48, E=8, K=3, el=5, eb=2)
    T, K = fwd["topk_idx"].shape
    x = torch.tensor(f(inp["x"]), requires_grad=True)
    wg = torch.tensor(f(inp["w_gate"]), requires_grad=True)
    wu = torch.tensor(f(inp["w_up"]), requires_grad=True)
    wd = torch.tensor(f(inp["w_down"]), requires_grad=True)
    g = torch.tensor(fwd["gates"].astype(np.float64))
    out = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(fwd["topk_idx"][t, k]) - 2
            if 0 <= e < 5:
                a = x[t] @ wg[e]
                b = x[t] @ wu[e]
                out = out.index_add(0, torch.tensor([t]), (g[t, k] * (torch.nn.functional.silu(a) * b) @ wd[e])[None])
    (out * torch.tensor(f(inp["d_out"]))).sum().backward()

    def rel(got, ref):
        return np.linalg.norm(got - ref) / np.linalg.norm(ref)

    assert rel(f(fwd["out"]), out.detach().numpy()) < 2 ** -6
    assert rel(f(bwd["dx"]), x.grad.numpy()) < 2 ** -5
    assert rel(bwd["dw_gate"], wg.grad.numpy()) < 2 ** -5
    assert rel(bwd["dw_up"], wu.grad.numpy()) < 2 ** -5
    assert rel(bwd["dw_down"], wd.grad.numpy()) < 2 ** -5


def test_backward_finite_difference_direction():
    """<dX, v> matches a central difference of <dOut, out(x + eps v)> of the fp64 layer."""
    inp, fwd, bwd, cap = _small_layer(seed=44, T=16, H=32, F=16, E=4, K=2, el=4)
    T, K = fwd["topk_idx"].shape
    X0 = f(inp["x"])
    Wg, Wu, Wd = f(inp["w_gate"]), f(inp["w_up"]), f(inp["w_down"])
    dO = f(inp["d_out"])

    def layer(X):
        out = np.zeros_like(X)
        for t in range(T):
            for k in range(K):
                e = fwd["topk_idx"][t, k]
                a, b = X[t] @ Wg[e], X[t] @ Wu[e]
                out[t] += fwd["gates"][t, k] * ((a * scipy.special.expit(a) * b) @ Wd[e])
        return out

    v = np.random.default_rng(1).standard_normal(X0.shape)
    eps = 1e-4
    fd = (np.sum(dO * layer(X0 + eps * v)) - np.sum(dO * layer(X0 - eps * v))) / (2 * eps)
    ad = np.sum(f(bwd["dx"]) * v)
    assert abs(ad - fd) <= 2 ** -5 * abs(fd)


# ---------------------------------------------------------------- router backward

def test_gate_grad_vs_fp64_dot():
    """dgates[t,k] = <dOut[t], y[pos[t,k]]> within the fp32 running-sum bound; pos < 0 gives exactly 0."""
    rng = np.random.default_rng(81)
    T, K, H, R = 24, 3, 200, 40
    d_out = rand_bf16(rng, (T, H))
    y = rand_bf16(rng, (R, H), std=0.5)
    pos = rng.integers(0, R, (T, K)).astype(np.int32)
    pos[rng.random((T, K)) < 0.3] = -1
    got = oracle.gate_grad(d_out, y, pos).astype(np.float64)
    D, Y = f(d_out), f(y)
    for t in range(T):
        for k in range(K):
            r = pos[t, k]
            if r < 0:
                assert got[t, k] == 0.0
                continue
            exact = float(np.dot(D[t], Y[r]))
            assert abs(got[t, k] - exact) <= gamma(H) * float(np.sum(np.abs(D[t] * Y[r]))) + 1e-30


def _fp64_gates(s, K):
    """Router forward in fp64 from its definition: softmax over all E, top-K, renormalise."""
    p = scipy.special.softmax(s)
    idx = np.lexsort((np.arange(len(s)), -s))[:K]
    return idx, p[idx] / np.sum(p[idx])


def test_route_backward_vs_finite_differences():
    """dlogits matches a central difference of sum_k dg_k * g_k(s) of the fp64 router forward."""
    rng = np.random.default_rng(82)
    T, E, K = 12, 9, 3
    # scores at least 0.05 apart, so a 1e-6 step never changes the top-K choice
    s = np.stack([rng.permutation(E) * 0.05 + rng.standard_normal() for _ in range(T)]).astype(np.float32)
    dg = rng.standard_normal((T, K)).astype(np.float32)
    idx, g = oracle.route(s, K)
    dl = oracle.route_backward(idx, g, dg, E).astype(np.float64)
    h = 1e-6
    for t in range(T):
        st = s[t].astype(np.float64)
        i0, _ = _fp64_gates(st, K)
        assert np.array_equal(i0, idx[t])

        def loss(v):
            i, gg = _fp64_gates(v, K)
            assert np.array_equal(i, i0)
            return float(np.dot(dg[t].astype(np.float64), gg))

        for e in range(E):
            d = np.zeros(E)
            d[e] = h
            fd = (loss(st + d) - loss(st - d)) / (2 * h)
            assert abs(dl[t, e] - fd) <= 1e-5 + 1e-4 * abs(fd), (t, e, dl[t, e], fd)


def test_route_backward_invariants():
    """Rows sum to 0; experts not chosen get exactly 0; K=1 gives exactly 0; a constant added to
    every dg_k changes nothing (the gates sum to 1); dlogits is linear in dgates."""
    rng = np.random.default_rng(83)
    T, E, K = 30, 16, 4
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, g = oracle.route(s, K)
    dg = rng.standard_normal((T, K)).astype(np.float32)
    dl = oracle.route_backward(idx, g, dg, E)
    chosen = np.zeros((T, E), bool)
    np.put_along_axis(chosen, idx, True, axis=1)
    assert np.all(dl[~chosen] == 0.0)
    scale = np.sum(np.abs(dl), axis=1) + np.sum(np.abs(g * dg), axis=1)
    assert np.all(np.abs(np.sum(dl.astype(np.float64), axis=1)) <= 1e-6 * scale)
    dl_shift = oracle.route_backward(idx, g, dg + np.float32(3.0), E)
    assert np.allclose(dl_shift, dl, atol=1e-5)
    dl2 = oracle.route_backward(idx, g, dg * np.float32(2.0), E)
    assert np.allclose(dl2, 2 * dl, rtol=1e-6, atol=1e-7)
    i1, g1 = oracle.route(s, 1)
    assert np.all(oracle.route_backward(i1, g1, dg[:, :1], E) == 0.0)


# ---------------------------------------------------------------- router projection

def test_router_logits_vs_fp64_matmul():
    """logits = fp32(x . W_r) + bias: numpy's fp64 matmul rounded to fp32 agrees to within one
    fp32 rounding (the two fp64 sums differ only in order, ~1e-16 relative)."""
    rng = np.random.default_rng(90)
    T, H, E = 37, 192, 64
    x = rand_bf16(rng, (T, H))
    w = rand_bf16(rng, (H, E), 0.02)
    bias = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, w, bias)
    dot = (f(x) @ f(w)).astype(np.float32)
    ref = dot + bias[None, :]
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 2 * U32 * (np.abs(dot) + np.abs(ref)) + 1e-30)
    # no bias: the dot product alone
    assert np.array_equal(oracle.router_logits(x, w), oracle.router_logits(x, w, np.zeros(E, np.float32)))


def test_router_logits_special_cases():
    """Identity router weight: logits = x + bias exactly.  A one-hot token picks out a row of W_r
    (a transposed W_r would give a column).  A row subset equals the same rows of the full result."""
    rng = np.random.default_rng(91)
    T, H = 9, 64
    x = rand_bf16(rng, (T, H))
    bias = rng.standard_normal(H).astype(np.float32)
    eye = synth.f32_to_bf16_bits(np.eye(H, dtype=np.float32))
    assert np.array_equal(oracle.router_logits(x, eye, bias), f(x).astype(np.float32) + bias[None, :])
    w = rand_bf16(rng, (H, 128), 0.02)
    onehot = np.zeros((3, H), np.float32)
    onehot[0, 5] = onehot[1, 0] = onehot[2, H - 1] = 1.0
    got = oracle.router_logits(synth.f32_to_bf16_bits(onehot), w)
    assert np.array_equal(got, f(w)[[5, 0, H - 1]].astype(np.float32))
    rows = np.array([0, 4, 8])
    full = oracle.router_logits(x, eye, bias)
    sub = oracle.router_logits(x, eye, bias, rows=rows)
    assert np.array_equal(sub[rows], full[rows])


def test_router_backward_vs_fp64_and_adjoint():
    """dx against numpy's fp64 matmul of bf16(dlogits) and W_r^T within the fp32-sum bound plus the
    final bf16 rounding; dW_r against fp64 x^T . bf16(dlogits) within the same kind of bound; and
    the adjoint identity <dl, v . W_r> = <dx, v> that ties the two directions together."""
    rng = np.random.default_rng(92)
    T, H, E = 23, 128, 64
    x = rand_bf16(rng, (T, H))
    w = rand_bf16(rng, (H, E), 0.02)
    dlog = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    dx, dw = oracle.router_backward(x, w, dlog)
    dl = oracle.round_bf16(dlog)
    assert np.array_equal(dl, synth.f32_to_bf16_bits(dlog))  # the rounding is RNE
    exact = f(dl) @ f(w).T
    bnd = gamma(E) * (np.abs(f(dl)) @ np.abs(f(w)).T)
    assert np.all(np.abs(f(dx) - exact) <= bnd + U16 * (np.abs(exact) + bnd) + 1e-30)
    exw = f(x).T @ f(dl)
    bndw = gamma(T) * (np.abs(f(x)).T @ np.abs(f(dl)))
    assert np.all(np.abs(dw.astype(np.float64) - exw) <= bndw + 1e-30)
    v = rng.standard_normal((T, H))
    lhs = float(np.sum(f(dl) * (v @ f(w))))
    rhs = float(np.sum(exact * v))
    assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + 1)
    # row and column subsets
    rows, cols = np.array([1, 22]), np.array([0, 63, 7])
    dx2, dw2 = oracle.router_backward(x, w, dlog, rows=rows, cols=cols)
    assert np.array_equal(dx2[rows], dx[rows])
    assert np.array_equal(dw2[:, cols], dw[:, cols])
