"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: torch tensors are checked for dtype/contiguity,
their device pointers and the current HIP stream are passed through, and a
negative status becomes a MoeError.  Every computation runs in the HIP
kernels.  There is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

_p = ctypes.c_void_p
_i = ctypes.c_int
_z = ctypes.c_size_t
_i64 = ctypes.c_int64

# every symbol declared in include/moe.h, with its ctypes signature
SIGNATURES = {
    "moe_strerror": ([_i], ctypes.c_char_p),
    "moe_abi_version": ([], _i),
    "moe_route": ([_p, _i, _i, _i, _p, _p, _p], _i),
    "moe_route_backward": ([_p, _p, _p, _i, _i, _i, _p, _p], _i),
    "moe_permute_workspace_size": ([_i, _i, _i], _z),
    "moe_permute": ([_p, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p, _z, _p], _i),
    "moe_permute_noalloc": ([_p, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p], _i),
    "moe_gather": ([_p, _p, _p, _i, _i, _i, _p, _p], _i),
    "moe_gather_gate_grad": ([_p, _p, _p, _p, _i, _i, _i, _p, _p, _p], _i),
    "moe_grouped_gemm_swiglu": ([_p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p], _i),
    "moe_grouped_gemm_swiglu_gather": ([_p, _i, _p, _i, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p], _i),
    "moe_grouped_gemm": ([_p, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p], _i),
    "moe_combine": ([_p, _p, _p, _i, _i, _i, _p, _p], _i),
    "moe_wgrad": ([_p, _i, _p, _i, _p, _i, _i, _i, _i, _p, _p], _i),
    "moe_wgrad_gate_up": ([_p, _i, _p, _i, _p, _i, _i, _p, _p, _p], _i),
    "moe_wgrad_gate_up_gather": ([_p, _i, _p, _i, _i, _p, _i, _p, _i, _i, _p, _p, _p], _i),
    "moe_wgrad_split_workspace_size": ([_i, _i, _i, _i], _z),
    "moe_wgrad_split": ([_p, _i, _p, _i, _p, _i, _i, _i, _i, _i, _p, _p, _z, _p], _i),
    "moe_router_workspace_size": ([_i, _i, _i], _z),
    "moe_router_logits": ([_p, _i, _i, _p, _i, _p, _p, _p, _z, _p], _i),
    "moe_router_backward": ([_p, _i, _i, _p, _i, _p, _p, _p, _p, _z, _p], _i),
    "moe_probe_mfma": ([_p, _i, _i, _p, _p], _i),
    "moe_probe_mfma16": ([_p, _i, _i, _p, _p], _i),
    "moe_probe_copy": ([_p, _p, _i64, _i, _i, _p], _i),
}

MOE_EPI_NONE = 0
MOE_EPI_SWIGLU_BWD = 1

_lib = None


class MoeError(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise MoeError(f"libmoe status {status}: {load().moe_strerror(status).decode()}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise MoeError(f"{name}: expected a contiguous {dtype} CUDA tensor, got {t.dtype} "
                       f"contiguous={t.is_contiguous()} device={t.device}")


def _shape(t, shape, name):
    """A caller-provided buffer must have exactly this shape (the kernels write all of it)."""
    if tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t, rows, cols, name):
    """A row buffer of the expert-grouped order: at least `rows` rows of exactly `cols` columns."""
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] != cols:
        raise MoeError(f"{name}: expected at least {rows} rows of {cols} columns, got {tuple(t.shape)}")


def moe_route(logits, K, topk_idx=None, gates=None, stream=None):
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if gates is None:
        gates = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _need(topk_idx, torch.int32, "topk_idx")
    _need(gates, torch.float32, "gates")
    _shape(topk_idx, (T, K), "topk_idx")
    _shape(gates, (T, K), "gates")
    _check(load().moe_route(_ptr(logits), T, E, K, _ptr(topk_idx), _ptr(gates), _stream(stream)))
    return topk_idx, gates


def moe_route_backward(topk_idx, gates, dgates, E, dlogits=None, stream=None):
    _need(topk_idx, torch.int32, "topk_idx")
    _need(gates, torch.float32, "gates")
    _need(dgates, torch.float32, "dgates")
    T, K = topk_idx.shape
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=gates.device)
    _need(dlogits, torch.float32, "dlogits")
    _shape(gates, (T, K), "gates")
    _shape(dgates, (T, K), "dgates")
    _shape(dlogits, (T, E), "dlogits")
    _check(load().moe_route_backward(_ptr(topk_idx), _ptr(gates), _ptr(dgates), T, E, K, _ptr(dlogits),
                                     _stream(stream)))
    return dlogits


def moe_permute_workspace_size(T, K, e_local) -> int:
    return int(load().moe_permute_workspace_size(T, K, e_local))


def moe_permute(topk_idx, e_begin, e_local, x, cap_rows, out=None, ws=None, stream=None, copy_rows=True):
    """-> dict(counts, offsets, pos, src, x_perm, status) (all device tensors).

    copy_rows=False: the index-only permutation (x_perm is None), for the
    gate/up GroupGEMM that reads x through src."""
    _need(topk_idx, torch.int32, "topk_idx")
    _need(x, torch.bfloat16, "x")
    T, K = topk_idx.shape
    H = x.shape[1]
    dev = x.device
    o = out or {}
    counts = o.get("counts")
    if counts is None:
        counts = torch.empty(max(e_local, 1), dtype=torch.int32, device=dev)
    offsets = o.get("offsets")
    if offsets is None:
        offsets = torch.empty(e_local + 1, dtype=torch.int32, device=dev)
    pos = o.get("pos")
    if pos is None:
        pos = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = o.get("src")
    if src is None:
        src = torch.empty(max(cap_rows, 1), dtype=torch.int32, device=dev)
    x_perm = o.get("x_perm")
    if x_perm is None and copy_rows:
        x_perm = torch.empty((max(cap_rows, 1), H), dtype=torch.bfloat16, device=dev)
    if not copy_rows:
        x_perm = None
    status = o.get("status")
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=dev)
    need = moe_permute_workspace_size(T, K, e_local)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for t, name, dt in ((counts, "counts", torch.int32), (offsets, "offsets", torch.int32), (pos, "pos", torch.int32),
                        (src, "src", torch.int32), (status, "status", torch.int32)):
        _need(t, dt, name)
    if counts.numel() < e_local or offsets.numel() < e_local + 1 or src.numel() < cap_rows or status.numel() < 1:
        raise MoeError("moe_permute: counts, offsets, src or status smaller than e_local, e_local+1, cap_rows, 1")
    _shape(pos, (T, K), "pos")
    if x_perm is not None:
        _need(x_perm, torch.bfloat16, "x_perm")
        _rows(x_perm, cap_rows, H, "x_perm")
    _check(load().moe_permute(_ptr(topk_idx), T, K, e_begin, e_local, _ptr(x), H, cap_rows,
                              _ptr(counts), _ptr(offsets), _ptr(pos), _ptr(src), _ptr(x_perm),
                              _ptr(status), _ptr(ws), ws.numel(), _stream(stream)))
    return dict(counts=counts[:e_local], offsets=offsets, pos=pos, src=src, x_perm=x_perm,
                status=status, ws=ws)


def moe_permute_noalloc(topk_idx, e_begin, e_local, x, cap_rows, out, stream=None, copy_rows=True):
    """moe_permute without a workspace: the library's own device array holds the count matrix.  Every
    output buffer is the caller's (out: counts, offsets, pos, src, status, and x_perm unless
    copy_rows=False); nothing is allocated here either."""
    _need(topk_idx, torch.int32, "topk_idx")
    _need(x, torch.bfloat16, "x")
    T, K = topk_idx.shape
    H = x.shape[1]
    counts, offsets, pos, src, status = (out[k] for k in ("counts", "offsets", "pos", "src", "status"))
    x_perm = out.get("x_perm") if copy_rows else None
    if copy_rows and x_perm is None:
        raise MoeError("moe_permute_noalloc: out['x_perm'] is required with copy_rows=True")
    for t, name, dt in ((counts, "counts", torch.int32), (offsets, "offsets", torch.int32), (pos, "pos", torch.int32),
                        (src, "src", torch.int32), (status, "status", torch.int32)):
        _need(t, dt, name)
    if counts.numel() < e_local or offsets.numel() < e_local + 1 or src.numel() < cap_rows or status.numel() < 1:
        raise MoeError("moe_permute_noalloc: counts, offsets, src or status smaller than e_local, e_local+1, "
                       "cap_rows, 1")
    _shape(pos, (T, K), "pos")
    if x_perm is not None:
        _need(x_perm, torch.bfloat16, "x_perm")
        _rows(x_perm, cap_rows, H, "x_perm")
    _check(load().moe_permute_noalloc(_ptr(topk_idx), T, K, e_begin, e_local, _ptr(x), H, cap_rows,
                                      _ptr(counts), _ptr(offsets), _ptr(pos), _ptr(src), _ptr(x_perm),
                                      _ptr(status), _stream(stream)))
    return dict(counts=counts[:e_local], offsets=offsets, pos=pos, src=src, x_perm=x_perm, status=status)


def moe_gather(d_out, pos, gates, dy_perm, stream=None):
    _need(d_out, torch.bfloat16, "d_out")
    _need(pos, torch.int32, "pos")
    if gates is not None:
        _need(gates, torch.float32, "gates")
    _need(dy_perm, torch.bfloat16, "dy_perm")
    T, K = pos.shape
    _shape(d_out, (T, d_out.shape[1]), "d_out")
    if dy_perm.dim() != 2 or dy_perm.shape[1] != d_out.shape[1]:
        raise MoeError(f"dy_perm: expected rows of {d_out.shape[1]} columns, got {tuple(dy_perm.shape)}")
    if gates is not None:
        _shape(gates, (T, K), "gates")
    _check(load().moe_gather(_ptr(d_out), _ptr(pos), _ptr(gates), T, K, d_out.shape[1], _ptr(dy_perm),
                             _stream(stream)))
    return dy_perm


def moe_gather_gate_grad(d_out, pos, gates, y, dy_perm, dgates=None, stream=None):
    """dy_perm as moe_gather, and dgates[t,k] = <d_out[t], y[pos[t,k]]> (0 for non-local pairs)."""
    _need(d_out, torch.bfloat16, "d_out")
    _need(pos, torch.int32, "pos")
    _need(gates, torch.float32, "gates")
    _need(y, torch.bfloat16, "y")
    _need(dy_perm, torch.bfloat16, "dy_perm")
    T, K = pos.shape
    if dgates is None:
        dgates = torch.empty((T, K), dtype=torch.float32, device=d_out.device)
    _need(dgates, torch.float32, "dgates")
    H = d_out.shape[1]
    _shape(d_out, (T, H), "d_out")
    _shape(gates, (T, K), "gates")
    _shape(dgates, (T, K), "dgates")
    for t, name in ((y, "y"), (dy_perm, "dy_perm")):
        if t.dim() != 2 or t.shape[1] != H:
            raise MoeError(f"{name}: expected rows of {H} columns, got {tuple(t.shape)}")
    _check(load().moe_gather_gate_grad(_ptr(d_out), _ptr(pos), _ptr(gates), _ptr(y), T, K, d_out.shape[1],
                                       _ptr(dy_perm), _ptr(dgates), _stream(stream)))
    return dy_perm, dgates


def _gate_up_checks(w_gate, w_up, offsets, cap_rows, h, ab_save):
    EL, H, F = w_gate.shape
    _shape(w_up, (EL, H, F), "w_up")
    if offsets.numel() < EL + 1:
        raise MoeError(f"offsets: expected {EL + 1} entries, got {offsets.numel()}")
    _need(h, torch.bfloat16, "h")
    _rows(h, cap_rows, F, "h")
    if ab_save is not None:
        _need(ab_save, torch.bfloat16, "ab_save")
        _rows(ab_save, cap_rows, 2 * F, "ab_save")


def moe_grouped_gemm_swiglu(x_perm, w_gate, w_up, offsets, cap_rows, h=None, ab_save=None, stream=None):
    _need(x_perm, torch.bfloat16, "x_perm")
    _need(w_gate, torch.bfloat16, "w_gate")
    _need(w_up, torch.bfloat16, "w_up")
    _need(offsets, torch.int32, "offsets")
    EL, H, F = w_gate.shape
    if h is None:
        h = torch.empty((x_perm.shape[0], F), dtype=torch.bfloat16, device=x_perm.device)
    _gate_up_checks(w_gate, w_up, offsets, cap_rows, h, ab_save)
    _rows(x_perm, cap_rows, H, "x_perm")
    _check(load().moe_grouped_gemm_swiglu(_ptr(x_perm), _ptr(w_gate), _ptr(w_up), _ptr(offsets), EL, H, F,
                                          cap_rows, _ptr(h), _ptr(ab_save), _stream(stream)))
    return h


def moe_grouped_gemm_swiglu_gather(x, src, K, w_gate, w_up, offsets, cap_rows, h=None, ab_save=None,
                                   stream=None):
    """Gate/up GroupGEMM + SwiGLU reading row r of the expert-grouped order
    straight from x[src[r] // K] (no x_perm)."""
    _need(x, torch.bfloat16, "x")
    _need(src, torch.int32, "src")
    _need(w_gate, torch.bfloat16, "w_gate")
    _need(w_up, torch.bfloat16, "w_up")
    _need(offsets, torch.int32, "offsets")
    EL, H, F = w_gate.shape
    T = x.shape[0]
    if h is None:
        h = torch.empty((max(cap_rows, 1), F), dtype=torch.bfloat16, device=x.device)
    _gate_up_checks(w_gate, w_up, offsets, cap_rows, h, ab_save)
    _shape(x, (T, H), "x")
    if src.numel() < cap_rows:
        raise MoeError(f"src: expected at least {cap_rows} entries, got {src.numel()}")
    _check(load().moe_grouped_gemm_swiglu_gather(_ptr(x), T, _ptr(src), int(K), _ptr(w_gate), _ptr(w_up),
                                                 _ptr(offsets), EL, H, F, cap_rows, _ptr(h), _ptr(ab_save),
                                                 _stream(stream)))
    return h


def moe_grouped_gemm(a, w0, w1, trans_w, offsets, Kd, N, cap_rows, c, epilogue=MOE_EPI_NONE, ab=None,
                     lda=None, ldc=None, stream=None):
    _need(a, torch.bfloat16, "a")
    _need(w0, torch.bfloat16, "w0")
    if w1 is not None:
        _need(w1, torch.bfloat16, "w1")
    _need(offsets, torch.int32, "offsets")
    _need(c, torch.bfloat16, "c")
    if ab is not None:
        _need(ab, torch.bfloat16, "ab")
    EL = w0.shape[0]
    lda = a.shape[1] if lda is None else lda
    ldc = c.shape[1] if ldc is None else ldc
    _shape(w0, (EL, N, Kd) if trans_w else (EL, Kd, N), "w0")
    if w1 is not None:
        _shape(w1, tuple(w0.shape), "w1")
    if offsets.numel() < EL + 1:
        raise MoeError(f"offsets: expected {EL + 1} entries, got {offsets.numel()}")
    # every row r < cap_rows of a and c may be touched, at strides lda and ldc
    for t, ld, name in ((a, lda, "a"), (c, ldc, "c")):
        if t.dim() != 2 or t.shape[0] < cap_rows or (cap_rows > 0 and t.shape[1] < ld):
            raise MoeError(f"{name}: expected at least {cap_rows} rows of {ld} columns, got {tuple(t.shape)}")
    if ab is not None:
        _rows(ab, cap_rows, 2 * N, "ab")
    _check(load().moe_grouped_gemm(_ptr(a), lda, _ptr(w0), _ptr(w1), int(trans_w), _ptr(offsets), EL, Kd, N,
                                   cap_rows, epilogue, _ptr(ab), _ptr(c), ldc, _stream(stream)))
    return c


def moe_combine(y, pos, gates, out=None, stream=None):
    _need(y, torch.bfloat16, "y")
    _need(pos, torch.int32, "pos")
    if gates is not None:
        _need(gates, torch.float32, "gates")
    T, K = pos.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(out, torch.bfloat16, "out")
    _shape(out, (T, H), "out")
    if gates is not None:
        _shape(gates, (T, K), "gates")
    _check(load().moe_combine(_ptr(y), _ptr(pos), _ptr(gates), T, K, H, _ptr(out), _stream(stream)))
    return out


def moe_wgrad(a, lda, b, ldb, offsets, e_local, M, N, cap_rows, dw=None, a_col0=0, b_col0=0, stream=None):
    """dw[j] = a_j^T b_j. a_col0/b_col0 offset the first column (e.g. b_col0=F for dW_up from dab)."""
    _need(a, torch.bfloat16, "a")
    _need(b, torch.bfloat16, "b")
    _need(offsets, torch.int32, "offsets")
    if dw is None:
        dw = torch.empty((e_local, M, N), dtype=torch.float32, device=a.device)
    _need(dw, torch.float32, "dw")
    _shape(dw, (e_local, M, N), "dw")
    if offsets.numel() < e_local + 1:
        raise MoeError(f"offsets: expected {e_local + 1} entries, got {offsets.numel()}")
    # rows r < cap_rows are read at strides lda and ldb from the column offsets
    for t, ld, c0, w, name in ((a, lda, a_col0, M, "a"), (b, ldb, b_col0, N, "b")):
        if cap_rows > 0 and t.numel() < (cap_rows - 1) * ld + c0 + w:
            raise MoeError(f"{name}: too small for {cap_rows} rows at stride {ld} from column {c0}")
    pa = a.data_ptr() + 2 * a_col0
    pb = b.data_ptr() + 2 * b_col0
    _check(load().moe_wgrad(pa, lda, pb, ldb, _ptr(offsets), e_local, M, N, cap_rows, _ptr(dw),
                            _stream(stream)))
    return dw


def moe_wgrad_gate_up(x_perm, dab, offsets, e_local, cap_rows, dw_gate=None, dw_up=None, stream=None):
    """(dw_gate, dw_up) = x_perm_j^T . [da_j | db_j] per expert, in one pass over x_perm."""
    _need(x_perm, torch.bfloat16, "x_perm")
    _need(dab, torch.bfloat16, "dab")
    _need(offsets, torch.int32, "offsets")
    H = x_perm.shape[1]
    F = dab.shape[1] // 2
    if dab.dim() != 2 or dab.shape[1] != 2 * F:
        raise MoeError(f"dab: expected [rows, 2F], got {tuple(dab.shape)}")
    _rows(x_perm, cap_rows, H, "x_perm")
    _rows(dab, cap_rows, 2 * F, "dab")
    if offsets.numel() < e_local + 1:
        raise MoeError(f"offsets: expected {e_local + 1} entries, got {offsets.numel()}")
    out = []
    for t, name in ((dw_gate, "dw_gate"), (dw_up, "dw_up")):
        if t is None:
            t = torch.empty((e_local, H, F), dtype=torch.float32, device=x_perm.device)
        _need(t, torch.float32, name)
        _shape(t, (e_local, H, F), name)
        out.append(t)
    _check(load().moe_wgrad_gate_up(_ptr(x_perm), H, _ptr(dab), F, _ptr(offsets), e_local, cap_rows, _ptr(out[0]),
                                    _ptr(out[1]), _stream(stream)))
    return out[0], out[1]


def moe_wgrad_gate_up_gather(x, src, K, dab, offsets, e_local, cap_rows, dw_gate=None, dw_up=None, stream=None):
    """moe_wgrad_gate_up reading row r of the expert-grouped order straight from x[src[r] // K] (no x_perm)."""
    _need(x, torch.bfloat16, "x")
    _need(src, torch.int32, "src")
    _need(dab, torch.bfloat16, "dab")
    _need(offsets, torch.int32, "offsets")
    if x.dim() != 2:
        raise MoeError(f"x: expected [T, H], got {tuple(x.shape)}")
    T, H = x.shape
    F = dab.shape[1] // 2
    if dab.dim() != 2 or dab.shape[1] != 2 * F:
        raise MoeError(f"dab: expected [rows, 2F], got {tuple(dab.shape)}")
    _rows(dab, cap_rows, 2 * F, "dab")
    if src.numel() < cap_rows:
        raise MoeError(f"src: expected at least {cap_rows} entries, got {src.numel()}")
    if offsets.numel() < e_local + 1:
        raise MoeError(f"offsets: expected {e_local + 1} entries, got {offsets.numel()}")
    out = []
    for t, name in ((dw_gate, "dw_gate"), (dw_up, "dw_up")):
        if t is None:
            t = torch.empty((e_local, H, F), dtype=torch.float32, device=x.device)
        _need(t, torch.float32, name)
        _shape(t, (e_local, H, F), name)
        out.append(t)
    _check(load().moe_wgrad_gate_up_gather(_ptr(x), T, _ptr(src), int(K), H, _ptr(dab), F, _ptr(offsets), e_local,
                                           cap_rows, _ptr(out[0]), _ptr(out[1]), _stream(stream)))
    return out[0], out[1]


def moe_wgrad_split_workspace_size(e_local, M, N, splits) -> int:
    return int(load().moe_wgrad_split_workspace_size(e_local, M, N, splits))


def moe_wgrad_split(a, lda, b, ldb, offsets, e_local, M, N, cap_rows, splits, dw=None, ws=None, a_col0=0,
                    b_col0=0, stream=None):
    """moe_wgrad with each expert's rows in `splits` fixed chunks whose fp32 partials are added in chunk
    order (ws: device workspace, allocated here if not given or too small)."""
    _need(a, torch.bfloat16, "a")
    _need(b, torch.bfloat16, "b")
    _need(offsets, torch.int32, "offsets")
    if dw is None:
        dw = torch.empty((e_local, M, N), dtype=torch.float32, device=a.device)
    _need(dw, torch.float32, "dw")
    _shape(dw, (e_local, M, N), "dw")
    if offsets.numel() < e_local + 1:
        raise MoeError(f"offsets: expected {e_local + 1} entries, got {offsets.numel()}")
    for t, ld, c0, w, name in ((a, lda, a_col0, M, "a"), (b, ldb, b_col0, N, "b")):
        if cap_rows > 0 and t.numel() < (cap_rows - 1) * ld + c0 + w:
            raise MoeError(f"{name}: too small for {cap_rows} rows at stride {ld} from column {c0}")
    need = moe_wgrad_split_workspace_size(e_local, M, N, splits)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=a.device)
    pa = a.data_ptr() + 2 * a_col0
    pb = b.data_ptr() + 2 * b_col0
    _check(load().moe_wgrad_split(pa, lda, pb, ldb, _ptr(offsets), e_local, M, N, cap_rows, splits, _ptr(dw),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return dw


def moe_router_workspace_size(T, H, E) -> int:
    return int(load().moe_router_workspace_size(T, H, E))


def _router_ws(T, H, E, ws, dev):
    need = moe_router_workspace_size(T, H, E)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return ws


def moe_router_logits(x, w_r, bias=None, logits=None, ws=None, stream=None):
    """logits fp32 [T,E] = x . w_r (+ bias)."""
    _need(x, torch.bfloat16, "x")
    _need(w_r, torch.bfloat16, "w_r")
    if bias is not None:
        _need(bias, torch.float32, "bias")
    T, H = x.shape
    E = w_r.shape[1]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _shape(w_r, (H, E), "w_r")
    if bias is not None:
        _shape(bias, (E,), "bias")
    _need(logits, torch.float32, "logits")
    _shape(logits, (T, E), "logits")
    ws = _router_ws(T, H, E, ws, x.device)
    _check(load().moe_router_logits(_ptr(x), T, H, _ptr(w_r), E, _ptr(bias), _ptr(logits), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return logits


def moe_router_backward(x, w_r, dlogits, dx=None, dw_r=None, ws=None, stream=None):
    """-> (dx bf16 [T,H], dw_r fp32 [H,E]) of the router projection."""
    _need(x, torch.bfloat16, "x")
    _need(w_r, torch.bfloat16, "w_r")
    _need(dlogits, torch.float32, "dlogits")
    T, H = x.shape
    E = w_r.shape[1]
    if dx is None:
        dx = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if dw_r is None:
        dw_r = torch.empty((H, E), dtype=torch.float32, device=x.device)
    _shape(w_r, (H, E), "w_r")
    _shape(dlogits, (T, E), "dlogits")
    _need(dx, torch.bfloat16, "dx")
    _shape(dx, (T, H), "dx")
    _need(dw_r, torch.float32, "dw_r")
    _shape(dw_r, (H, E), "dw_r")
    ws = _router_ws(T, H, E, ws, x.device)
    _check(load().moe_router_backward(_ptr(x), T, H, _ptr(w_r), E, _ptr(dlogits), _ptr(dx), _ptr(dw_r), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return dx, dw_r


def moe_probe_mfma(operands, iters, out=None, stream=None):
    """Measurement aid: back-to-back bf16 MFMAs on register-held operands.
    operands bf16 [blocks*4, 8, 64, 8] (per wave: 4 A then 4 B fragments) -> out fp32 [blocks*4, 64]."""
    _need(operands, torch.bfloat16, "operands")
    if operands.dim() != 4 or tuple(operands.shape[1:]) != (8, 64, 8) or operands.shape[0] % 4:
        raise MoeError(f"operands: expected shape (4*blocks, 8, 64, 8), got {tuple(operands.shape)}")
    waves = operands.shape[0]
    if out is None:
        out = torch.empty((waves, 64), dtype=torch.float32, device=operands.device)
    _need(out, torch.float32, "out")
    _shape(out, (waves, 64), "out")
    _check(load().moe_probe_mfma(_ptr(operands), waves // 4, iters, _ptr(out), _stream(stream)))
    return out


def moe_probe_mfma16(operands, iters, out=None, stream=None):
    """The probe on 16x16x32 MFMAs: operands bf16 [blocks*4, 16, 64, 8] (per wave: 8 A then 8 B fragments)
    -> out fp32 [blocks*4, 64]."""
    _need(operands, torch.bfloat16, "operands")
    if operands.dim() != 4 or tuple(operands.shape[1:]) != (16, 64, 8) or operands.shape[0] % 4:
        raise MoeError(f"operands: expected shape (4*blocks, 16, 64, 8), got {tuple(operands.shape)}")
    waves = operands.shape[0]
    if out is None:
        out = torch.empty((waves, 64), dtype=torch.float32, device=operands.device)
    _need(out, torch.float32, "out")
    _shape(out, (waves, 64), "out")
    _check(load().moe_probe_mfma16(_ptr(operands), waves // 4, iters, _ptr(out), _stream(stream)))
    return out


def moe_probe_copy(src, dst, nontemporal=0, blocks=0, stream=None):
    """Measurement aid: a plain streaming copy of src into dst (contiguous device tensors of the same
    byte size, a multiple of 16).  nontemporal: bit 0 loads, bit 1 stores; blocks 0 = 8 per CU."""
    for name, t in (("src", src), ("dst", dst)):
        if not t.is_cuda or not t.is_contiguous():
            raise MoeError(f"{name}: expected a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise MoeError("src and dst differ in byte size")
    _check(load().moe_probe_copy(_ptr(src), _ptr(dst), nbytes, nontemporal, blocks, _stream(stream)))
    return dst
