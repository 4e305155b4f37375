"""Buffers past 4 GiB: an expert share whose permuted rows outgrow 32-bit byte
offsets.  262400 routed rows of 8192 bf16 columns make x_perm, y and dy_perm
just over 4 GiB each, so every kernel that addresses a row of them (the row copy, both
GroupGEMMs, the combine and the output-gradient gather) must form 64-bit
offsets.  Index outputs are compared in full; floating outputs on sampled rows
and tokens, most of them past the 2 GiB and 4 GiB marks, which the oracle
computes from compact copies of just the rows they need (the oracle's groups
are given by offsets, so a sorted subset of rows with its own offsets is the
same computation).  No oracle input comes from the GPU: the down projection
and the combine take seeded synthetic operands, the latter a closed form that
both sides evaluate."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_equal
from routing_permute_groupgemm_amd import _lib, pipeline, synth

pytestmark = pytest.mark.gpu

T, K, E, H, F = 32800, 8, 64, 8192, 256
R = T * K  # every expert is local: 262400 rows, past the 2^32-byte mark of a row buffer


def bits(t):
    return pipeline.to_numpy_bits(t)


def closed_form_rows(rows):
    """y[r, c] = ((37 r + 11 c) mod 61 - 30) / 16, exact in bf16: this test's own input generator."""
    r = np.asarray(rows, np.int64)[:, None]
    c = np.arange(H, dtype=np.int64)[None, :]
    return synth.f32_to_bf16_bits(((37 * r + 11 * c) % 61 - 30).astype(np.float32) / 16.0)


def closed_form_device(rows):
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    c = torch.arange(H, dtype=torch.int64, device="cuda")[None, :]
    for lo in range(0, rows, 8192):
        r = torch.arange(lo, min(rows, lo + 8192), dtype=torch.int64, device="cuda")[:, None]
        y[lo:lo + r.shape[0]] = (((37 * r + 11 * c) % 61 - 30).to(torch.float32) / 16.0).to(torch.bfloat16)
    return y


class Big:
    pass


@pytest.fixture(scope="module")
def big():
    assert R * H * 2 > 2 ** 32
    print("\n[large] generating inputs", flush=True)
    b = Big()
    rng = np.random.default_rng(11)
    # K distinct experts per token
    b.idx = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K].astype(np.int32)
    b.gates = rng.random((T, K), dtype=np.float32)
    b.x = synth.operand_bf16((T, H), seed=11, tag=21)
    b.wg = synth.operand_bf16((E, H, F), seed=11, tag=22, std=0.02)
    b.wu = synth.operand_bf16((E, H, F), seed=11, tag=23, std=0.02)
    b.wd = synth.operand_bf16((E, F, H), seed=11, tag=24, std=0.02)
    b.dev = pipeline.to_device(dict(idx=b.idx, gates=b.gates, x=b.x, wg=b.wg, wu=b.wu, wd=b.wd))
    print("[large] permute (4 GiB of rows)", flush=True)
    b.pm = _lib.moe_permute(b.dev["idx"], 0, E, b.dev["x"], R)
    torch.cuda.synchronize()
    b.ref = oracle.permute(b.idx, 0, E, None, R)
    b.rng = np.random.default_rng(12)
    # sampled rows: both ends, around the 2 GiB and 4 GiB byte marks of a row buffer, and random
    half, full = 2 ** 31 // (2 * H), 2 ** 32 // (2 * H)
    rows = {0, 1, R // 2, half - 1, half, full - 1, full, full + 1, R - 2, R - 1}
    rows |= set(b.rng.integers(half, R, 24).tolist()) | set(b.rng.integers(0, R, 8).tolist())
    b.rows = np.array(sorted(r for r in rows if r < R), np.int64)
    yield b
    del b.pm, b.dev
    torch.cuda.empty_cache()


def compact_offsets(offsets, rows):
    """Offsets of the sorted row subset: the sampled rows of each expert, in order."""
    return np.searchsorted(rows, offsets).astype(np.int32)


def test_large_permute(big):
    pm, ref = big.pm, big.ref
    assert_equal("counts", bits(pm["counts"]), ref["counts"])
    assert_equal("offsets", bits(pm["offsets"]), ref["offsets"])
    assert_equal("pos", bits(pm["pos"]), ref["pos"])
    assert_equal("src", bits(pm["src"]), ref["src"])
    assert int(bits(pm["status"])[0]) == ref["status"] == 0
    # every row of the 4 GiB copy, on the device, in slices
    src = pm["src"].long()
    for lo in range(0, R, 32768):
        hi = min(R, lo + 32768)
        assert torch.equal(pm["x_perm"][lo:hi].view(torch.int16), big.dev["x"][src[lo:hi] // K].view(torch.int16))


def test_large_gate_up_sampled_rows(big):
    pm, rows = big.pm, big.rows
    h = torch.empty((R, F), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm_swiglu(pm["x_perm"], big.dev["wg"], big.dev["wu"], pm["offsets"], R, h=h)
    hz = torch.empty_like(h)
    _lib.moe_grouped_gemm_swiglu_gather(big.dev["x"], pm["src"], K, big.dev["wg"], big.dev["wu"], pm["offsets"], R,
                                        h=hz)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), hz.view(torch.int16))  # zero-copy reads the same rows
    xs = big.x[big.ref["src"][rows] // K]
    ref_h, _ = oracle.expert_up(xs, big.wg, big.wu, compact_offsets(big.ref["offsets"], rows), len(rows),
                                want_ab=False)
    assert_close("h", bits(h)[rows], ref_h)


def test_large_down_sampled_rows(big):
    pm, rows = big.pm, big.rows
    hin = synth.operand_bf16((R, F), seed=11, tag=25)
    hd = pipeline.to_device(dict(h=hin))["h"]
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm(hd, big.dev["wd"], None, 0, pm["offsets"], F, H, R, y)
    torch.cuda.synchronize()
    got = bits(y[torch.from_numpy(rows).cuda()])
    del y
    ref = oracle.expert_down(hin[rows], big.wd, compact_offsets(big.ref["offsets"], rows), len(rows))
    assert_close("y", got, ref)


def test_large_combine_and_gather(big):
    pm = big.pm
    y = closed_form_device(R)
    out = _lib.moe_combine(y, pm["pos"], big.dev["gates"])
    d_out = synth.operand_bf16((T, H), seed=11, tag=26)
    dd = pipeline.to_device(dict(d=d_out))["d"]
    dy = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    dg = torch.empty((T, K), dtype=torch.float32, device="cuda")
    _lib.moe_gather_gate_grad(dd, pm["pos"], big.dev["gates"], y, dy, dg)
    torch.cuda.synchronize()
    pos = big.ref["pos"]
    assert pos.min() >= 0  # every pair is local
    # tokens: both ends, random, and those whose rows lie past the 4 GiB mark
    high = np.nonzero(pos.max(axis=1) >= 2 ** 32 // (2 * H))[0]
    toks = np.unique(np.concatenate([[0, 1, T - 1], big.rng.integers(0, T, 16), high[:8], high[-8:]]))
    # compact copies: the rows these tokens use, and their positions among them
    used = np.unique(pos[toks])
    ys = closed_form_rows(used)
    pos_s = np.searchsorted(used, pos[toks]).astype(np.int32)
    ref_out = oracle.combine(ys, pos_s, big.gates[toks])
    assert_close("out", bits(out)[toks], ref_out)
    ref_dg = oracle.gate_grad(d_out[toks], ys, pos_s)
    assert_close("dgates", bits(dg)[toks], ref_dg)
    # dy_perm rows of these tokens' pairs, as one group in pair order: the compact pair index
    # i*K + k of token toks[i] is its src entry, and its row is pos[toks[i], k]
    n = len(toks) * K
    ref_dy = oracle.bwd_gather(d_out[toks], np.arange(n, dtype=np.int32), np.array([0, n], np.int32),
                               big.gates[toks], K, n)
    rows = torch.from_numpy(pos[toks].reshape(-1).astype(np.int64)).cuda()
    assert_close("dy_perm", bits(dy[rows]), ref_dy)


def test_gather_past_2gib():
    """The zero-copy gate/up GEMM addresses all tokens through one 32-bit offset range of up to 3.75 GiB:
    x of 2.87 GB (T = 200000, H = 7168), rows gathered from both ends and around the 2 GiB byte mark (tokens
    149796 and up lie past it), against the copy path bit for bit and sampled rows against the oracle."""
    Tg, Hg, Fg, Kg = 200000, 7168, 128, 1
    assert Tg * Hg * 2 > 2 ** 31
    rng = np.random.default_rng(21)
    mark = 2 ** 31 // (2 * Hg)
    toks = np.unique(np.concatenate([np.arange(0, 64), np.arange(mark - 64, mark + 64), np.arange(Tg - 64, Tg),
                                     rng.integers(0, Tg, 200)]))
    e_rows = np.array([len(toks) // 2, len(toks) - len(toks) // 2])
    offsets = np.concatenate([[0], np.cumsum(e_rows)]).astype(np.int32)
    src = toks.astype(np.int32)  # K = 1: src[r] = t
    R = len(toks)
    print(f"[large] zero-copy gate/up, x {Tg * Hg * 2 / 2 ** 30:.2f} GiB, {R} rows", flush=True)
    # x rows by a closed form that both sides evaluate: x[t, c] = ((29 t + 7 c) mod 53 - 26) / 32, exact in bf16
    x = torch.empty((Tg, Hg), dtype=torch.bfloat16, device="cuda")
    c = torch.arange(Hg, dtype=torch.int64, device="cuda")[None, :]
    for lo in range(0, Tg, 8192):
        r = torch.arange(lo, min(Tg, lo + 8192), dtype=torch.int64, device="cuda")[:, None]
        x[lo:lo + r.shape[0]] = (((29 * r + 7 * c) % 53 - 26).to(torch.float32) / 32.0).to(torch.bfloat16)
    wg = synth.operand_bf16((2, Hg, Fg), seed=21, tag=31, std=0.02)
    wu = synth.operand_bf16((2, Hg, Fg), seed=21, tag=32, std=0.02)
    dev = pipeline.to_device(dict(wg=wg, wu=wu, offsets=offsets, src=src))
    hz = torch.empty((R, Fg), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_gemm_swiglu_gather(x, dev["src"], Kg, dev["wg"], dev["wu"], dev["offsets"], R, h=hz)
    xp = x[torch.from_numpy(toks).cuda()].contiguous()
    h = torch.empty_like(hz)
    _lib.moe_grouped_gemm_swiglu(xp, dev["wg"], dev["wu"], dev["offsets"], R, h=h)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), hz.view(torch.int16))
    del x, xp
    torch.cuda.empty_cache()
    rows = np.array(sorted({0, R - 1} | set(np.searchsorted(toks, [mark - 1, mark, mark + 1]).tolist())
                           | set(rng.integers(0, R, 12).tolist())), np.int64)
    tr = toks[rows].astype(np.int64)[:, None]
    xs = synth.f32_to_bf16_bits((((29 * tr + 7 * np.arange(Hg)[None, :]) % 53 - 26).astype(np.float32)) / 32.0)
    ref_h, _ = oracle.expert_up(xs, wg, wu, compact_offsets(offsets, rows), len(rows), want_ab=False)
    assert_close("h", bits(hz)[rows], ref_h)
