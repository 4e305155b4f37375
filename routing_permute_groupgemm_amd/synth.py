"""Seeded synthetic inputs for the MoE layer hot path.

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic (no softmax, no top-k, no permutation, no GEMM) and it
imports neither the HIP binding nor the CPU oracle, so both sides can consume
the same arrays.

Workloads (sizes follow the expert-parallel MoE layer of the UniEP paper,
"MoE workflow" paragraph: tokens T, hidden H, expert intermediate F, experts
E, top-k K; the 32-of-256 expert share mirrors the DeepSeek-V3-shaped
MoonEP ``Buffer(S=4096, H=7168, K=8, E=256)`` example):

* ``tiny``          T=256    H=128  F=256  E=8   K=2  all experts local
* ``ep_share_4k``   T=4096   H=7168 F=2048 E=256 K=8  local experts 0..31
* ``skew_8k``       T=8192   H=4096 F=1536 E=128 K=8  Zipf(1.2)-skewed router
* ``fwdbwd_16k``    T=16384  H=2048 F=768  E=128 K=8  forward + backward
* ``ep_share_128k`` T=131072 H=7168 F=2048 E=256 K=8  local 0..31, Zipf(0.8)

Recipe (all bf16 values are fp32 normal samples rounded to nearest-even):
x ~ N(0,1); router weight W_r, expert weights W_gate/W_up [E_L,H,F] and
W_down [E_L,F,H] ~ N(0, 0.02); dOut ~ N(0,1).  Router logits are
``fp32(x @ W_r computed in fp64) + bias`` where the bias (fp32) is
``alpha * ln(w_rank)`` with Zipf weights ``w_j = (j+1)^-s`` assigned to
experts through a seeded random permutation.  The literal reading
(alpha = 1) saturates one expert, so the skewed workloads use alpha = 0.22,
which lands the load-imbalance metric maxvio near 2.5 (Zipf 1.2) and 1.6
(Zipf 0.8); ``alpha=1`` remains available as a stress case.

Every tensor is drawn from its own child of
``SeedSequence([1000 + workload_id, seed])`` in fixed 4 Mi-element chunks
(one grandchild stream per chunk), so the values do not depend on how many
threads fill them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np
import torch

_CHUNK = 1 << 22  # elements per independent RNG stream


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """Problem sizes in the paper's notation plus the synthetic-routing recipe."""

    name: str
    workload_id: int
    T: int
    H: int
    F: int
    E: int
    K: int
    e_begin: int = 0
    e_local: int | None = None  # None: all E experts are local
    zipf_s: float | None = None  # None: no router bias (balanced routing)
    alpha: float = 0.22  # scale of the log-Zipf bias
    backward: bool = False

    @property
    def EL(self) -> int:
        return self.E if self.e_local is None else self.e_local

    @property
    def cap(self) -> int:
        """Row capacity of the permuted buffers.

        All experts local: T*K (never overflows).  A local share of the
        experts: twice the expected routed rows T*K*E_L/E (overflow is
        detectable through the permutation's status word).
        """
        if self.EL == self.E:
            return self.T * self.K
        return min(self.T * self.K, 2 * ((self.T * self.K * self.EL + self.E - 1) // self.E))

    def scaled(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)


WORKLOADS: dict[str, MoeShape] = {
    "tiny": MoeShape("tiny", 1, T=256, H=128, F=256, E=8, K=2),
    "ep_share_4k": MoeShape("ep_share_4k", 2, T=4096, H=7168, F=2048, E=256, K=8, e_local=32),
    "skew_8k": MoeShape("skew_8k", 3, T=8192, H=4096, F=1536, E=128, K=8, zipf_s=1.2),
    "fwdbwd_16k": MoeShape("fwdbwd_16k", 4, T=16384, H=2048, F=768, E=128, K=8, backward=True),
    "ep_share_128k": MoeShape("ep_share_128k", 5, T=131072, H=7168, F=2048, E=256, K=8,
                              e_local=32, zipf_s=0.8, backward=True),
}

# Child-stream slots of each workload's SeedSequence.
_SLOTS = ("x", "w_router", "w_gate", "w_up", "w_down", "d_out", "perm")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _seedseq(shape: MoeShape, seed: int) -> dict[str, np.random.SeedSequence]:
    root = np.random.SeedSequence([1000 + shape.workload_id, seed])
    return dict(zip(_SLOTS, root.spawn(len(_SLOTS))))


def normal_f32(ss: np.random.SeedSequence, n: int, std: float = 1.0) -> np.ndarray:
    """n fp32 samples of N(0, std^2), filled chunk-by-chunk from spawned streams."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    children = ss.spawn(nchunks) if nchunks else []

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the raw 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(ss: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal_f32(ss, n, std)).reshape(shape)


def zipf_bias(shape: MoeShape, perm_ss: np.random.SeedSequence, alpha: float | None = None) -> np.ndarray:
    """Per-expert fp32 bias alpha*ln(w_rank(e)) with w_j=(j+1)^-s over a seeded permutation."""
    if shape.zipf_s is None:
        return np.zeros(shape.E, dtype=np.float32)
    a = shape.alpha if alpha is None else alpha
    perm = np.random.Generator(np.random.PCG64(perm_ss)).permutation(shape.E)
    rank_of = np.empty(shape.E, dtype=np.int64)
    rank_of[perm] = np.arange(shape.E)
    return (a * (-shape.zipf_s) * np.log(rank_of + 1.0)).astype(np.float32)


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """fp32(x @ W_r in fp64) + bias, the router scores handed to the routing step."""
    T = x_bits.shape[0]
    wr = bf16_bits_to_f32(wr_bits).astype(np.float64)
    out = np.empty((T, wr.shape[1]), dtype=np.float32)
    step = 8192
    for lo in range(0, T, step):
        xs = bf16_bits_to_f32(x_bits[lo:lo + step]).astype(np.float64)
        out[lo:lo + step] = (xs @ wr).astype(np.float32)
    out += bias[None, :]
    return out


def make_inputs(shape: MoeShape, seed: int = 0, *, weights: bool = True,
                d_out: bool | None = None, alpha: float | None = None,
                router: bool = False) -> dict[str, np.ndarray]:
    """All inputs of one layer pass as numpy arrays (bf16 as uint16 bit patterns).

    Keys: logits f32[T,E]; x u16[T,H]; w_gate, w_up u16[E_L,H,F];
    w_down u16[E_L,F,H]; d_out u16[T,H] (when the backward is wanted);
    with router=True also w_router u16[H,E] and router_bias f32[E], the
    operands the logits were made from.
    """
    ss = _seedseq(shape, seed)
    T, H, F, E, EL = shape.T, shape.H, shape.F, shape.E, shape.EL
    out: dict[str, np.ndarray] = {}
    out["x"] = normal_bf16(ss["x"], (T, H), 1.0)
    wr = normal_bf16(ss["w_router"], (H, E), 0.02)
    bias = zipf_bias(shape, ss["perm"], alpha)
    out["logits"] = router_logits(out["x"], wr, bias)
    if router:
        out["w_router"] = wr
        out["router_bias"] = bias
    if weights:
        out["w_gate"] = normal_bf16(ss["w_gate"], (EL, H, F), 0.02)
        out["w_up"] = normal_bf16(ss["w_up"], (EL, H, F), 0.02)
        out["w_down"] = normal_bf16(ss["w_down"], (EL, F, H), 0.02)
    if d_out if d_out is not None else shape.backward:
        out["d_out"] = normal_bf16(ss["d_out"], (T, H), 1.0)
    return out


def operand_bf16(shape_tuple, seed: int, tag: int, std: float = 1.0) -> np.ndarray:
    """A free-standing seeded bf16 operand (per-step tests feed these to both sides)."""
    ss = np.random.SeedSequence([2000 + tag, seed])
    return normal_bf16(ss, shape_tuple, std)


def maxvio(counts: np.ndarray, T: int, K: int, E: int) -> float:
    """Load-imbalance metric: max_e count_e / (T*K/E) - 1 (MoonEP README)."""
    return float(np.max(counts) / (T * K / E) - 1.0)
