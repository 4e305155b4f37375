"""The layer's forward and backward as a sequence of libmoe calls on one stream.

Buffers are torch device tensors allocated once per shape (`MoeBuffers`);
each step is one C-ABI call, and nothing is read back to the host.
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib
from .synth import MoeShape


@dataclasses.dataclass
class MoeBuffers:
    shape: MoeShape
    cap: int
    topk_idx: torch.Tensor
    gates: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    pos: torch.Tensor
    src: torch.Tensor
    x_perm: torch.Tensor | None  # None with zero_copy
    status: torch.Tensor
    ws: torch.Tensor
    h: torch.Tensor
    ab: torch.Tensor | None
    y: torch.Tensor
    out: torch.Tensor
    # backward
    dy_perm: torch.Tensor | None = None
    dab: torch.Tensor | None = None
    dx_perm: torch.Tensor | None = None
    dx: torch.Tensor | None = None
    dw_gate: torch.Tensor | None = None
    dw_up: torch.Tensor | None = None
    dw_down: torch.Tensor | None = None
    dgates: torch.Tensor | None = None
    dlogits: torch.Tensor | None = None
    # zero-copy dispatch: the permutation is index-only, and the gate/up
    # GroupGEMM and the gate/up weight gradient read x[src[r] // K]
    zero_copy: bool = False

    @classmethod
    def allocate(cls, shape: MoeShape, cap: int | None = None, device="cuda", backward=None, zero_copy=False):
        backward = shape.backward if backward is None else backward
        T, H, F, K, EL = shape.T, shape.H, shape.F, shape.K, shape.EL
        cap = shape.cap if cap is None else cap
        capn = max(cap, 1)
        e = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        ws_bytes = max(_lib.moe_permute_workspace_size(T, K, EL), 256)
        b = cls(shape=shape, cap=cap,
                topk_idx=e((T, K), dt=torch.int32), gates=e((T, K), dt=torch.float32),
                counts=e(max(EL, 1), dt=torch.int32), offsets=e(EL + 1, dt=torch.int32),
                pos=e((T, K), dt=torch.int32), src=e(capn, dt=torch.int32),
                x_perm=None if zero_copy else e((capn, H)),
                status=e(4, dt=torch.int32), ws=e(ws_bytes, dt=torch.uint8), h=e((capn, F)),
                ab=e((capn, 2 * F)) if backward else None, y=e((capn, H)), out=e((T, H)), zero_copy=zero_copy)
        if backward:
            b.dy_perm = e((capn, H))
            b.dab = e((capn, 2 * F))
            b.dx_perm = e((capn, H))
            b.dx = e((T, H))
            b.dw_gate = e((EL, H, F), dt=torch.float32)
            b.dw_up = e((EL, H, F), dt=torch.float32)
            b.dw_down = e((EL, F, H), dt=torch.float32)
            b.dgates = e((T, K), dt=torch.float32)
            b.dlogits = e((T, shape.E), dt=torch.float32)
        return b


def route(buf: MoeBuffers, logits):
    _lib.moe_route(logits, buf.shape.K, buf.topk_idx, buf.gates)


def permute(buf: MoeBuffers, x):
    s = buf.shape
    _lib.moe_permute(buf.topk_idx, s.e_begin, s.EL, x, buf.cap,
                     out=dict(counts=buf.counts, offsets=buf.offsets, pos=buf.pos, src=buf.src,
                              x_perm=buf.x_perm, status=buf.status), ws=buf.ws, copy_rows=not buf.zero_copy)


def expert_up(buf: MoeBuffers, w_gate, w_up, x=None):
    """x (the token rows) is needed with zero_copy only."""
    if buf.zero_copy:
        _lib.moe_grouped_gemm_swiglu_gather(x, buf.src, buf.shape.K, w_gate, w_up, buf.offsets, buf.cap,
                                            h=buf.h, ab_save=buf.ab)
    else:
        _lib.moe_grouped_gemm_swiglu(buf.x_perm, w_gate, w_up, buf.offsets, buf.cap, h=buf.h, ab_save=buf.ab)


def expert_down(buf: MoeBuffers, w_down):
    s = buf.shape
    _lib.moe_grouped_gemm(buf.h, w_down, None, 0, buf.offsets, s.F, s.H, buf.cap, buf.y)


def combine(buf: MoeBuffers):
    _lib.moe_combine(buf.y, buf.pos, buf.gates, out=buf.out)


def forward(buf: MoeBuffers, inp: dict):
    """inp: device tensors logits, x, w_gate, w_up, w_down."""
    route(buf, inp["logits"])
    permute(buf, inp["x"])
    expert_up(buf, inp["w_gate"], inp["w_up"], inp["x"])
    expert_down(buf, inp["w_down"])
    combine(buf)
    return buf.out


def backward(buf: MoeBuffers, inp: dict):
    """inp additionally holds d_out (and x, read by the zero-copy weight gradient). Needs the forward's
    ab_save."""
    s = buf.shape
    H, F, EL, cap = s.H, s.F, s.EL, buf.cap
    _lib.moe_gather_gate_grad(inp["d_out"], buf.pos, buf.gates, buf.y, buf.dy_perm, buf.dgates)
    _lib.moe_route_backward(buf.topk_idx, buf.gates, buf.dgates, s.E, buf.dlogits)
    _lib.moe_grouped_gemm(buf.dy_perm, inp["w_down"], None, 1, buf.offsets, H, F, cap, buf.dab,
                          epilogue=_lib.MOE_EPI_SWIGLU_BWD, ab=buf.ab)
    _lib.moe_grouped_gemm(buf.dab, inp["w_gate"], inp["w_up"], 1, buf.offsets, F, H, cap, buf.dx_perm)
    _lib.moe_combine(buf.dx_perm, buf.pos, None, out=buf.dx)
    if buf.zero_copy:
        _lib.moe_wgrad_gate_up_gather(inp["x"], buf.src, s.K, buf.dab, buf.offsets, EL, cap, dw_gate=buf.dw_gate,
                                      dw_up=buf.dw_up)
    else:
        _lib.moe_wgrad_gate_up(buf.x_perm, buf.dab, buf.offsets, EL, cap, dw_gate=buf.dw_gate, dw_up=buf.dw_up)
    _lib.moe_wgrad(buf.h, F, buf.dy_perm, H, buf.offsets, EL, F, H, cap, dw=buf.dw_down)
    return buf.dx


def to_device(inp: dict, device="cuda") -> dict:
    """numpy inputs from synth.make_inputs -> device tensors (bf16 bit patterns viewed as bf16)."""
    import numpy as np
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.to(device)
    return out


def to_numpy_bits(t: torch.Tensor):
    """Device bf16 tensor -> numpy uint16 bit patterns (other dtypes: plain numpy)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
