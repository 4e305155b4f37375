"""CPU oracle of the MoE layer hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``moe_oracle.c`` (plain C loops, fp32
sums in a fixed order, built with ``-ffp-contract=off``) with numpy in/out and
shares no code with the HIP library.  See ``moe_oracle.c`` for the passage of
the pages each function follows.

Every function here is pinned by ``tests/test_oracle_pins.py`` against things
other than itself (brute force, numpy/torch library routines in fp64, closed
forms, invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

CFLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc into libmoe_oracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_l = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        L = _lib
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_route.argtypes = [_p, _i, _i, _i, _p, _p]
        L.oracle_permute.argtypes = [_p, _i, _i, _i, _i, _p, _i, _l, _p, _p, _p, _p, _p, _p]
        L.oracle_expert_up.argtypes = [_p, _p, _p, _p, _i, _i, _i, _l, _p, _l, _p, _p]
        L.oracle_expert_down.argtypes = [_p, _p, _p, _i, _i, _i, _l, _p, _l, _p]
        L.oracle_combine.argtypes = [_p, _p, _p, _i, _i, _i, _p, _l, _p]
        L.oracle_bwd_gather.argtypes = [_p, _p, _p, _p, _i, _i, _i, _l, _p]
        L.oracle_bwd_down.argtypes = [_p, _p, _p, _p, _i, _i, _i, _l, _p, _l, _p]
        L.oracle_bwd_up.argtypes = [_p, _p, _p, _p, _i, _i, _i, _l, _p, _l, _p]
        L.oracle_wgrad.argtypes = [_p, _l, _p, _l, _p, _i, _i, _i, _l, _p, _i, _p, _i, _p]
        L.oracle_gate_grad.argtypes = [_p, _p, _p, _i, _i, _i, _p]
        L.oracle_route_backward.argtypes = [_p, _p, _p, _i, _i, _i, _p]
        L.oracle_router_logits.argtypes = [_p, _p, _p, _i, _i, _i, _p, _i, _p]
        L.oracle_round_bf16.argtypes = [_p, _l, _p]
        L.oracle_router_dx.argtypes = [_p, _p, _i, _i, _i, _p, _i, _p]
        for name in ("oracle_route", "oracle_permute", "oracle_expert_up", "oracle_expert_down",
                     "oracle_combine", "oracle_bwd_gather", "oracle_bwd_down", "oracle_bwd_up",
                     "oracle_wgrad", "oracle_gate_grad", "oracle_route_backward", "oracle_router_logits",
                     "oracle_round_bf16", "oracle_router_dx"):
            getattr(L, name).restype = None
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def f32_to_bf16(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(v)))


def route(logits: np.ndarray, K: int):
    """-> (topk_idx int32[T,K], gates f32[T,K])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    if E > 1024 or K > 64 or K > E:
        raise ValueError("oracle route supports E<=1024, K<=min(64,E)")
    idx = np.empty((T, K), np.int32)
    g = np.empty((T, K), np.float32)
    lib().oracle_route(_ptr(logits), T, E, K, _ptr(idx), _ptr(g))
    return idx, g


def permute(topk_idx: np.ndarray, e_begin: int, e_local: int, x: np.ndarray | None, cap: int):
    """-> dict(counts, offsets, pos, src, x_perm, status). Rows >= R of src/x_perm are zero."""
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    if e_local > 1024:
        raise ValueError("oracle permute supports e_local<=1024")
    H = 0 if x is None else x.shape[1]
    counts = np.zeros(e_local, np.int32)
    offsets = np.zeros(e_local + 1, np.int32)
    pos = np.empty((T, K), np.int32)
    src = np.zeros(cap, np.int32)
    xp = None if x is None else np.zeros((cap, H), np.uint16)
    st = np.zeros(1, np.int32)
    xx = None if x is None else _c(x, np.uint16)
    lib().oracle_permute(_ptr(topk_idx), T, K, e_begin, e_local, _ptr(xx), H, cap,
                         _ptr(counts), _ptr(offsets), _ptr(pos), _ptr(src), _ptr(xp), _ptr(st))
    return dict(counts=counts, offsets=offsets, pos=pos, src=src, x_perm=xp, status=int(st[0]))


def _rows(rows):
    return None if rows is None else _c(rows, np.int64)


def expert_up(x_perm, w_gate, w_up, offsets, cap, rows=None, want_ab=True):
    """-> (h u16[cap,F], ab u16[cap,2F] or None); only `rows` are filled if given."""
    x_perm = _c(x_perm, np.uint16)
    w_gate, w_up, offsets = _c(w_gate, np.uint16), _c(w_up, np.uint16), _c(offsets, np.int32)
    EL, H, F = w_gate.shape
    h = np.zeros((cap, F), np.uint16)
    ab = np.zeros((cap, 2 * F), np.uint16) if want_ab else None
    r = _rows(rows)
    lib().oracle_expert_up(_ptr(x_perm), _ptr(w_gate), _ptr(w_up), _ptr(offsets), EL, H, F, cap,
                           _ptr(r), 0 if r is None else len(r), _ptr(h), _ptr(ab))
    return h, ab


def expert_down(h, w_down, offsets, cap, rows=None):
    h, w_down, offsets = _c(h, np.uint16), _c(w_down, np.uint16), _c(offsets, np.int32)
    EL, F, H = w_down.shape
    y = np.zeros((cap, H), np.uint16)
    r = _rows(rows)
    lib().oracle_expert_down(_ptr(h), _ptr(w_down), _ptr(offsets), EL, F, H, cap,
                             _ptr(r), 0 if r is None else len(r), _ptr(y))
    return y


def combine(y, pos, gates, tokens=None):
    """out[t] = sum_k gate*y[pos]; gates=None -> plain sum (combine-gradient)."""
    y, pos = _c(y, np.uint16), _c(pos, np.int32)
    T, K = pos.shape
    H = y.shape[1]
    g = None if gates is None else _c(gates, np.float32)
    out = np.zeros((T, H), np.uint16)
    tk = _rows(tokens)
    lib().oracle_combine(_ptr(y), _ptr(pos), _ptr(g), T, K, H, _ptr(tk),
                         0 if tk is None else len(tk), _ptr(out))
    return out


def bwd_gather(d_out, src, offsets, gates, K, cap):
    d_out, src, offsets = _c(d_out, np.uint16), _c(src, np.int32), _c(offsets, np.int32)
    H = d_out.shape[1]
    EL = len(offsets) - 1
    g = None if gates is None else _c(gates, np.float32)
    dy = np.zeros((cap, H), np.uint16)
    lib().oracle_bwd_gather(_ptr(d_out), _ptr(src), _ptr(offsets), _ptr(g), K, H, EL, cap, _ptr(dy))
    return dy


def bwd_down(dy_perm, w_down, ab_save, offsets, cap, rows=None):
    dy_perm, w_down = _c(dy_perm, np.uint16), _c(w_down, np.uint16)
    ab_save, offsets = _c(ab_save, np.uint16), _c(offsets, np.int32)
    EL, F, H = w_down.shape
    dab = np.zeros((cap, 2 * F), np.uint16)
    r = _rows(rows)
    lib().oracle_bwd_down(_ptr(dy_perm), _ptr(w_down), _ptr(ab_save), _ptr(offsets), EL, F, H, cap,
                          _ptr(r), 0 if r is None else len(r), _ptr(dab))
    return dab


def bwd_up(dab, w_gate, w_up, offsets, cap, rows=None):
    dab, w_gate, w_up = _c(dab, np.uint16), _c(w_gate, np.uint16), _c(w_up, np.uint16)
    offsets = _c(offsets, np.int32)
    EL, H, F = w_gate.shape
    dx = np.zeros((cap, H), np.uint16)
    r = _rows(rows)
    lib().oracle_bwd_up(_ptr(dab), _ptr(w_gate), _ptr(w_up), _ptr(offsets), EL, H, F, cap,
                        _ptr(r), 0 if r is None else len(r), _ptr(dx))
    return dx


def wgrad(A, lda, B, ldb, offsets, M, N, cap, groups=None, cols=None, out=None):
    """dW[j] = A_j^T B_j over each group's rows (fp32). A, B are flat/2-D u16 with row strides lda, ldb."""
    A, B, offsets = _c(A, np.uint16), _c(B, np.uint16), _c(offsets, np.int32)
    EL = len(offsets) - 1
    dw = np.zeros((EL, M, N), np.float32) if out is None else out
    g = None if groups is None else _c(groups, np.int32)
    c = None if cols is None else _c(cols, np.int32)
    lib().oracle_wgrad(_ptr(A), lda, _ptr(B), ldb, _ptr(offsets), EL, M, N, cap,
                       _ptr(g), 0 if g is None else len(g), _ptr(c), 0 if c is None else len(c), _ptr(dw))
    return dw


def gate_grad(d_out, y, pos):
    """dgates f32[T,K] = <d_out[t], y[pos[t,k]]> for local pairs, 0 for pos < 0."""
    d_out, y, pos = _c(d_out, np.uint16), _c(y, np.uint16), _c(pos, np.int32)
    T, K = pos.shape
    H = d_out.shape[1]
    dg = np.empty((T, K), np.float32)
    lib().oracle_gate_grad(_ptr(d_out), _ptr(y), _ptr(pos), T, K, H, _ptr(dg))
    return dg


def route_backward(topk_idx, gates, dgates, E):
    """dlogits f32[T,E]: the gradient of the scores through the renormalised top-K gates."""
    topk_idx, gates, dgates = _c(topk_idx, np.int32), _c(gates, np.float32), _c(dgates, np.float32)
    T, K = topk_idx.shape
    dl = np.empty((T, E), np.float32)
    lib().oracle_route_backward(_ptr(topk_idx), _ptr(gates), _ptr(dgates), T, E, K, _ptr(dl))
    return dl


def router_logits(x, w_r, bias=None, rows=None):
    """logits f32[T,E] = fp32(x . w_r in fp64) + bias; only `rows` are filled if given (others 0)."""
    x, w_r = _c(x, np.uint16), _c(w_r, np.uint16)
    T, H = x.shape
    E = w_r.shape[1]
    b = None if bias is None else _c(bias, np.float32)
    out = np.zeros((T, E), np.float32)
    r = _rows(rows)
    lib().oracle_router_logits(_ptr(x), _ptr(w_r), _ptr(b), T, H, E, _ptr(r), 0 if r is None else len(r),
                               _ptr(out))
    return out


def round_bf16(a):
    """fp32 array -> bf16 bit patterns, nearest even."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def router_backward(x, w_r, dlogits, rows=None, cols=None):
    """-> (dx u16[T,H] (only `rows` filled if given), dw_r f32[H,E] (only `cols` if given)) of the
    router projection, from bf16(dlogits)."""
    x, w_r = _c(x, np.uint16), _c(w_r, np.uint16)
    T, H = x.shape
    E = w_r.shape[1]
    dl = round_bf16(dlogits)
    dx = np.zeros((T, H), np.uint16)
    r = _rows(rows)
    lib().oracle_router_dx(_ptr(dl), _ptr(w_r), T, H, E, _ptr(r), 0 if r is None else len(r), _ptr(dx))
    dw = wgrad(x, H, dl, E, np.array([0, T], np.int32), H, E, T, cols=cols)[0]
    return dx, dw


def forward(inp: dict, e_begin: int, e_local: int, K: int, cap: int):
    """The whole oracle forward chain on one set of inputs (small sizes)."""
    idx, g = route(inp["logits"], K)
    pm = permute(idx, e_begin, e_local, inp["x"], cap)
    h, ab = expert_up(pm["x_perm"], inp["w_gate"], inp["w_up"], pm["offsets"], cap)
    y = expert_down(h, inp["w_down"], pm["offsets"], cap)
    out = combine(y, pm["pos"], g)
    return dict(topk_idx=idx, gates=g, h=h, ab=ab, y=y, out=out, **pm)


def backward(inp: dict, fwd: dict, cap: int):
    """The whole oracle backward chain given the oracle's own forward results."""
    K = fwd["topk_idx"].shape[1]
    F = inp["w_gate"].shape[2]
    H = inp["w_gate"].shape[1]
    dy = bwd_gather(inp["d_out"], fwd["src"], fwd["offsets"], fwd["gates"], K, cap)
    dab = bwd_down(dy, inp["w_down"], fwd["ab"], fwd["offsets"], cap)
    dxp = bwd_up(dab, inp["w_gate"], inp["w_up"], fwd["offsets"], cap)
    dx = combine(dxp, fwd["pos"], None)
    dwg = wgrad(fwd["x_perm"], H, dab, 2 * F, fwd["offsets"], H, F, cap)
    dwu = wgrad(fwd["x_perm"], H, dab[:, F:].copy(), F, fwd["offsets"], H, F, cap)
    dwd = wgrad(fwd["h"], F, dy, H, fwd["offsets"], F, H, cap)
    dg = gate_grad(inp["d_out"], fwd["y"], fwd["pos"])
    dl = route_backward(fwd["topk_idx"], fwd["gates"], dg, inp["logits"].shape[1])
    return dict(dy_perm=dy, dab=dab, dx_perm=dxp, dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd, dgates=dg,
                dlogits=dl)
