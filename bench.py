#!/usr/bin/env python3
"""Throughput of the one-GPU MoE layer hot path on MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM: route -> permute -> gate/up GroupGEMM with
SwiGLU -> down GroupGEMM -> combine, plus (workloads with a backward) the
gate-scaled gather, both dgrad GroupGEMMs, the combine-gradient and the three
weight-gradient GroupGEMMs.  Every step is a libmoe C-ABI call on one stream.

The headline workload (default ep_share_128k: T=131072, H=7168, F=2048, the
32 local experts of E=256, K=8, forward+backward with the row-copy permute) is
timed first.  Prints one JSON line: tokens/s, the roofline of the dominant
kernel (achieved algorithmic bytes or flops per launch / its mean launch time,
from HIP events recorded on the launch stream around that kernel in the timed
steps), every GroupGEMM's fraction of the bf16 MFMA peak, the permute's and
the combine's fraction of HBM bandwidth, one summary per --also workload
(timed the same way, after the headline's buffers are freed) and the CPU
oracle's throughput on a bounded sample of the headline workload.  `step_ms`
comes from an untimed pass with events around every step: each recorded event
costs the stream a short bubble, so the timed pass records them around the
dominant step only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRCS = os.path.join(ROOT, "routing_permute_groupgemm_amd", "csrc", "gemm*")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ep_share_128k",
                    help="the headline workload (default: the largest one-GPU configuration, forward+backward)")
    ap.add_argument("--also", default="ep_share_4k,skew_8k,fwdbwd_16k",
                    help="comma-separated workloads also timed after the headline, reported under 'workloads' "
                         "(empty: none)")
    ap.add_argument("--also-steps", type=int, default=10, help="timed steps of each --also workload")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--router", action="store_true",
                    help="include the router projection x.W_r (and its backward) in the step; the pages' layer "
                         "timings exclude gating, so the default leaves it out")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of the whole step captured in a HIP graph (reported as "
                         "graph_ms_per_step; value stays the eager timed pass)")
    ap.add_argument("--dense-reference", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on a dense bf16 GEMM of each row-tiled GroupGEMM's "
                         "rows x depth x width, as a vendor-library reference on this GPU")
    ap.add_argument("--copy-rows", action="store_true",
                    help="forward-only workloads: permute with the row copy instead of zero-copy dispatch")
    ap.add_argument("--zero-copy", action="store_true",
                    help="forward+backward workloads too: no row copy, the gate/up GEMM and its weight "
                         "gradient read the tokens through src")
    ap.add_argument("--no-nb", action="store_true",
                    help="skip timing the non-bitwise (two row chunks per expert) weight gradient beside the "
                         "bitwise one on workloads with a backward")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="only time single row-tiled GroupGEMMs (128 experts x 1024 rows) over contraction "
                         "lengths, to split their time into a per-k-step and a per-tile part")
    return ap.parse_args()


def tile_sweep():
    """The down GEMM (bf16 epilogue, N = 2048) and the down dgrad (SwiGLU-backward epilogue, N = 768) on 128
    experts of 1024 rows each, at several contraction lengths; a least-squares line through
    (k-steps per tile, µs per round of 256 tiles) gives the cost per k-step and per tile."""
    import torch
    from routing_permute_groupgemm_amd import _lib
    _lib.load()
    EL, rows = 128, 1024
    cap = EL * rows
    off = torch.arange(EL + 1, dtype=torch.int32, device="cuda") * rows
    g = torch.Generator(device="cuda").manual_seed(7)
    res = {}
    for name, N, epi, kds in (("down (bf16 epilogue)", 2048, _lib.MOE_EPI_NONE, (256, 512, 768, 1536, 3072)),
                              ("down dgrad (SwiGLU-backward epilogue)", 768, _lib.MOE_EPI_SWIGLU_BWD,
                               (512, 1024, 2048, 4096))):
        pts = []
        for kd in kds:
            a = torch.randn(cap, kd, device="cuda", generator=g).to(torch.bfloat16)
            w = (torch.randn(EL, N, kd, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            ab = torch.randn(cap, 2 * N, device="cuda", generator=g).to(torch.bfloat16) if epi else None
            c = torch.empty(cap, 2 * N if epi else N, dtype=torch.bfloat16, device="cuda")
            f = lambda: _lib.moe_grouped_gemm(a, w, None, 1, off, kd, N, cap, c, epilogue=epi, ab=ab)  # noqa: E731
            for _ in range(3):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            rounds = EL * (rows // 256) * ((N + 255) // 256) / 256
            pts.append((kd // 32, ms * 1e3 / rounds))
            res.setdefault(name, {})[f"K={kd}"] = dict(ms=round(ms, 4), k_steps=kd // 32,
                                                       us_per_tile_round=round(ms * 1e3 / rounds, 2),
                                                       tflops=round(2 * cap * kd * N / ms / 1e9, 1))
            del a, w, ab, c
        n = len(pts)
        mx = sum(x for x, _ in pts) / n
        my = sum(y for _, y in pts) / n
        slope = sum((x - mx) * (y - my) for x, y in pts) / sum((x - mx) ** 2 for x, _ in pts)
        res[name]["fit"] = dict(us_per_k_step=round(slope, 3), us_per_tile=round(my - slope * mx, 2))
    print(json.dumps(res, indent=1))


def algorithmic_work(shape, R, T_act, n_active, zero_copy=False, router=False):
    """Per-launch algorithmic bytes and flops of every step (real rows only, no padding).
    With zero-copy dispatch the permutation moves indices only and the gate/up
    GroupGEMM reads the routed rows from x (the same 2*R*H bytes as from x_perm)."""
    T, H, F, E, K, EL = shape.T, shape.H, shape.F, shape.E, shape.K, shape.EL
    w = {}
    w["route"] = dict(bytes=4 * T * E + 8 * T * K, flops=0)
    rows = 0 if zero_copy else 2 * H * T_act + 2 * H * R
    w["permute"] = dict(bytes=4 * T * K * 3 + 4 * R + rows + 8 * EL, flops=0)
    ab = 2 * R * 2 * F if shape.backward else 0
    w["expert_up"] = dict(bytes=2 * n_active * H * 2 * F + 2 * R * H + 2 * R * F + ab, flops=4 * R * H * F)
    w["expert_down"] = dict(bytes=2 * n_active * F * H + 2 * R * F + 2 * R * H, flops=2 * R * F * H)
    w["combine"] = dict(bytes=2 * H * R + 8 * T * K + 2 * H * T, flops=0)
    if router:
        w["router_fwd"] = dict(bytes=2 * T * H + 2 * H * E + 4 * T * E, flops=2 * T * H * E)
        if shape.backward:
            w["router_bwd"] = dict(bytes=4 * T * E + 2 * H * E + 2 * T * H + 2 * T * H + 4 * H * E,
                                   flops=4 * T * H * E)
    if shape.backward:
        # gather + gate gradient: d_out rows read once, dy_perm written, y rows read, pos/gates in, dgates out
        w["bwd_gather"] = dict(bytes=2 * H * T_act + 2 * H * R + 2 * H * R + 12 * T * K, flops=2 * R * H)
        # router backward: topk_idx, gates, dgates in, dense dlogits out
        w["route_bwd"] = dict(bytes=12 * T * K + 4 * T * E, flops=0)
        w["bwd_down_dgrad"] = dict(bytes=2 * n_active * F * H + 2 * R * H + 4 * R * 2 * F,
                                   flops=2 * R * H * F)
        w["bwd_up_dgrad"] = dict(bytes=2 * n_active * 2 * H * F + 2 * R * 2 * F + 2 * R * H,
                                 flops=2 * R * 2 * F * H)
        w["bwd_combine"] = dict(bytes=2 * H * R + 4 * T * K + 2 * H * T, flops=0)
        for name, (m, n) in (("wgrad_gate", (H, F)), ("wgrad_up", (H, F)), ("wgrad_down", (F, H))):
            w[name] = dict(bytes=2 * R * m + 2 * R * n + 4 * EL * m * n, flops=2 * R * m * n)
        # dW_gate and dW_up in one pass over x_perm and [da | db]
        w["wgrad_gate_up"] = dict(bytes=2 * R * H + 2 * R * 2 * F + 4 * EL * H * 2 * F, flops=2 * R * H * 2 * F)
    return w


def roofline(work, ms):
    b, f = work["bytes"], work["flops"]
    t_hbm = b / (HBM_PEAK_GBS * 1e9)
    t_mfma = f / (MFMA_BF16_PEAK_TFS * 1e12)
    if f and t_mfma >= t_hbm:
        ach = f / (ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                    frac=round(ach / MFMA_BF16_PEAK_TFS, 4))
    ach = b / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4))


def src_hash():
    """Hash of the GroupGEMM sources (kernel header and its translation units)."""
    import glob
    h = hashlib.sha256()
    for path in sorted(glob.glob(GEMM_SRCS)):
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            db = json.load(fh)
        rec = db[f"{kernel}@{workload}"]
        if rec.get("gemm_src_sha") != src_hash():
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(shape, inp, budget_s):
    """The oracle as it stands, timed on the first n tokens of the same batch (the tokens are i.i.d.): one
    forward and, for workloads with a backward, one backward whose weight gradients sum over every routed
    row of the sample, as the GPU step sums over every row of the batch.  n comes from two calibration
    passes (128 and 512 tokens) that separate the per-token time from the fixed part (the fp32 weight
    gradients are written in full whatever the sample), so the timed pass takes about budget_s."""
    import oracle
    T, K, EL = shape.T, shape.K, shape.EL

    def run(n):
        sub = {k: inp[k][:n] for k in ("logits", "x")}
        sub.update({k: inp[k] for k in ("w_gate", "w_up", "w_down")})
        cap = n * K
        t0 = time.perf_counter()
        fwd = oracle.forward(sub, shape.e_begin, EL, K, cap)
        if shape.backward:
            sub["d_out"] = inp["d_out"][:n]
            oracle.backward(sub, fwd, cap)
        return time.perf_counter() - t0

    n1, n2 = min(T, 128), min(T, 512)
    t1 = run(n1)
    t2 = run(n2) if n2 > n1 else t1
    slope = max((t2 - t1) / max(n2 - n1, 1), 1e-7)
    fixed = max(t1 - slope * n1, 0.0)
    n = int(min(T, max(n2, (budget_s - fixed) / slope)))
    dt = run(n) if n > n2 else t2
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(line.split(":", 1)[1].strip() for line in fh if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    what = "forward+backward pass (weight gradients over the sample's rows)" if shape.backward else "forward pass"
    return dict(value=round(n / dt, 2), unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                cpu=cpu, host_cpus=os.cpu_count(),
                sample=f"first {n} of the {T} tokens, one {what}, {dt:.1f} s (n sized from 128- and "
                       f"512-token calibration passes: {slope * 1e3:.2f} ms/token + {fixed:.1f} s fixed)")


def calib_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}))


def measured_copy_gbps(stream):
    """Read+write GB/s of plain 1 GiB device-to-device copies on this GPU: torch's copy and the copy
    probe with each load/store hint (bit 0 non-temporal loads, bit 1 stores).  The best is the practical
    ceiling of a kernel that moves as many bytes in as out, beside the data sheet's 8 TB/s."""
    import torch
    from routing_permute_groupgemm_amd import _lib
    n = 1 << 30
    # the values do not matter to a copy's rate; the probe runs first, so that a kernel trace of the run
    # sees a probe kernel right after the timed steps
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")

    def rate(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(2 * n / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9, 1)

    rates = {}
    for nt in range(4):
        rates[f"probe_nt{nt}"] = rate(lambda: _lib.moe_probe_copy(a, b, nontemporal=nt, stream=stream))
    rates["torch"] = rate(lambda: b.copy_(a))
    del a, b
    rates["best"] = max(rates.values())
    return rates


def measured_mfma_tflops(stream, target_ms=20.0, shape=32):
    """TFLOP/s that back-to-back bf16 MFMAs reach on this GPU with N(0,1) operands held in registers
    (libmoe's probe, one workgroup of four waves per CU; shape 32: v_mfma_f32_32x32x16_bf16, 16:
    v_mfma_f32_16x16x32_bf16): the practical ceiling of an MFMA-bound kernel on real data, since the
    clock the chip holds under MFMA load depends on the operand bits."""
    import torch
    from routing_permute_groupgemm_amd import _lib
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device="cuda").manual_seed(7)
    nfrag = 8 if shape == 32 else 16
    ops = torch.randn((blocks * 4, nfrag, 64, 8), device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty((blocks * 4, 64), dtype=torch.float32, device="cuda")
    # per wave and iteration: 16 MFMAs of 32x32x16, or 64 of 16x16x32
    flop_per_iter = blocks * 4 * (16 * 2 * 32 * 32 * 16 if shape == 32 else 64 * 2 * 16 * 16 * 32)
    probe = _lib.moe_probe_mfma if shape == 32 else _lib.moe_probe_mfma16
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(iters):
        e0.record(stream)
        probe(ops, iters, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    iters = max(1, int(2000 * target_ms / max(run(2000), 1e-3)))
    rates = [flop_per_iter * iters / (run(iters) * 1e-3) / 1e12 for _ in range(3)]
    del ops, out
    return round(float(np.median(rates)), 1)


# (depth, width) of each GroupGEMM step as one dense product over all routed rows
def dense_dims(name, shape):
    H, F = shape.H, shape.F
    return {"expert_up": (H, 2 * F), "expert_down": (F, H), "bwd_down_dgrad": (H, F), "bwd_up_dgrad": (2 * F, H)}.get(name)


def dense_reference(M, Kd, N, steps):
    """TFLOP/s of torch.matmul (hipBLASLt) on a dense [M,Kd] x [Kd,N] bf16 product."""
    import torch
    a = torch.randn(M, Kd, device="cuda").to(torch.bfloat16)
    b = (torch.randn(Kd, N, device="cuda") * 0.02).to(torch.bfloat16)
    for _ in range(2):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del a, b, c
    tf = 2 * M * Kd * N / (ms * 1e-3) / 1e12
    return dict(library="torch.matmul (hipBLASLt)", shape=[M, Kd, N], ms=round(ms, 4), achieved=round(tf, 2),
                frac=round(tf / MFMA_BF16_PEAK_TFS, 4))


GEMM_STEPS = ("expert_up", "expert_down", "bwd_down_dgrad", "bwd_up_dgrad", "wgrad_gate_up", "wgrad_gate", "wgrad_up",
              "wgrad_down")
HBM_STEPS = ("route", "permute", "combine", "bwd_gather", "route_bwd", "bwd_combine")


def layer_steps(shape, dev, buf, router):
    """(name, call) of every step of one pass, in order; each call is one or more libmoe C-ABI calls."""
    import torch
    from routing_permute_groupgemm_amd import _lib, pipeline
    steps = []
    if router:
        T, H, E = shape.T, shape.H, shape.E
        r_ws = torch.empty(max(_lib.moe_router_workspace_size(T, H, E), 256), dtype=torch.uint8, device="cuda")
        r_logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        steps.append(("router_fwd", lambda: _lib.moe_router_logits(dev["x"], dev["w_router"], dev["router_bias"],
                                                                   logits=r_logits, ws=r_ws)))
        dev["logits"] = r_logits  # the route step consumes the projected scores
    steps += [("route", lambda: pipeline.route(buf, dev["logits"])),
              ("permute", lambda: pipeline.permute(buf, dev["x"])),
              ("expert_up", lambda: pipeline.expert_up(buf, dev["w_gate"], dev["w_up"], dev["x"])),
              ("expert_down", lambda: pipeline.expert_down(buf, dev["w_down"])),
              ("combine", lambda: pipeline.combine(buf))]
    if shape.backward:
        H, F, EL, cap = shape.H, shape.F, shape.EL, buf.cap
        steps += [
            ("bwd_gather", lambda: _lib.moe_gather_gate_grad(dev["d_out"], buf.pos, buf.gates, buf.y, buf.dy_perm,
                                                             buf.dgates)),
            ("route_bwd", lambda: _lib.moe_route_backward(buf.topk_idx, buf.gates, buf.dgates, shape.E,
                                                          buf.dlogits)),
            ("bwd_down_dgrad", lambda: _lib.moe_grouped_gemm(buf.dy_perm, dev["w_down"], None, 1, buf.offsets, H,
                                                             F, cap, buf.dab, epilogue=_lib.MOE_EPI_SWIGLU_BWD,
                                                             ab=buf.ab)),
            ("bwd_up_dgrad", lambda: _lib.moe_grouped_gemm(buf.dab, dev["w_gate"], dev["w_up"], 1, buf.offsets, F,
                                                           H, cap, buf.dx_perm)),
            ("bwd_combine", lambda: _lib.moe_combine(buf.dx_perm, buf.pos, None, out=buf.dx)),
            ("wgrad_gate_up",
             (lambda: _lib.moe_wgrad_gate_up_gather(dev["x"], buf.src, shape.K, buf.dab, buf.offsets, EL, cap,
                                                    dw_gate=buf.dw_gate, dw_up=buf.dw_up)) if buf.zero_copy else
             (lambda: _lib.moe_wgrad_gate_up(buf.x_perm, buf.dab, buf.offsets, EL, cap, dw_gate=buf.dw_gate,
                                             dw_up=buf.dw_up))),
            ("wgrad_down", lambda: _lib.moe_wgrad(buf.h, F, buf.dy_perm, H, buf.offsets, EL, F, H, cap,
                                                  dw=buf.dw_down)),
        ]
        if router:
            r_dx = torch.empty((shape.T, H), dtype=torch.bfloat16, device="cuda")
            r_dw = torch.empty((H, shape.E), dtype=torch.float32, device="cuda")
            steps.append(("router_bwd", lambda: _lib.moe_router_backward(dev["x"], dev["w_router"], buf.dlogits,
                                                                         dx=r_dx, dw_r=r_dw, ws=r_ws)))
    return steps


def time_steps(steps, stream, n_steps, warmup):
    """Warm-up, then an untimed breakdown pass (events around every step: each step's mean time and the
    dominant step), then the timed pass of n_steps whole steps, which records events only around the
    dominant step (every recorded event costs the stream a short bubble)."""
    import torch

    def one_step(evs=None, only=None):
        for i, (_, fn) in enumerate(steps):
            if evs is not None and (only is None or i == only):
                evs[0 if only is not None else i].record(stream)
            fn()
            if evs is not None and only is not None and i == only:
                evs[1].record(stream)
        if evs is not None and only is None:
            evs[len(steps)].record(stream)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(n_steps)]
    for k in range(n_steps):
        one_step(evs[k])
    torch.cuda.synchronize()
    per = {name: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(n_steps)]))
           for i, (name, _) in enumerate(steps)}
    dom_i = max(range(len(steps)), key=lambda i: per[steps[i][0]])
    dev_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(n_steps):
        one_step(dev_evs[k], only=dom_i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / n_steps
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_evs]))
    return dict(per=per, dom=steps[dom_i][0], dom_ms=dom_ms, ms_per_step=ms_per_step, one_step=one_step)


def time_wgrad_modes(shape, buf, reps=5):
    """The three weight-gradient GroupGEMMs of one step in the bitwise mode (one fixed-order pass over each
    expert's rows) and in the non-bitwise mode with two row chunks per expert (fp32 partials added in chunk
    order), each timed with HIP events over `reps` repetitions on the launch stream: UniEP's Table 7
    comparison.  Returns ms per step of the three calls in each mode."""
    import torch
    from routing_permute_groupgemm_amd import _lib
    H, F, EL, cap = shape.H, shape.F, shape.EL, buf.cap
    ws = torch.empty(max(_lib.moe_wgrad_split_workspace_size(EL, H, F, 2),
                         _lib.moe_wgrad_split_workspace_size(EL, F, H, 2)), dtype=torch.uint8, device="cuda")

    def bw():
        _lib.moe_wgrad(buf.x_perm, H, buf.dab, 2 * F, buf.offsets, EL, H, F, cap, dw=buf.dw_gate)
        _lib.moe_wgrad(buf.x_perm, H, buf.dab, 2 * F, buf.offsets, EL, H, F, cap, dw=buf.dw_up, b_col0=F)
        _lib.moe_wgrad(buf.h, F, buf.dy_perm, H, buf.offsets, EL, F, H, cap, dw=buf.dw_down)

    def nb():
        _lib.moe_wgrad_split(buf.x_perm, H, buf.dab, 2 * F, buf.offsets, EL, H, F, cap, 2, dw=buf.dw_gate, ws=ws)
        _lib.moe_wgrad_split(buf.x_perm, H, buf.dab, 2 * F, buf.offsets, EL, H, F, cap, 2, dw=buf.dw_up, ws=ws,
                             b_col0=F)
        _lib.moe_wgrad_split(buf.h, F, buf.dy_perm, H, buf.offsets, EL, F, H, cap, 2, dw=buf.dw_down, ws=ws)

    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in (("bw", bw), ("nb", nb), ("bw_again", bw)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / reps
    del ws
    bw_ms = (out["bw"] + out["bw_again"]) / 2
    return dict(bw_ms=round(bw_ms, 4), nb_ms=round(out["nb"], 4), nb_splits=2,
                nb_vs_bw=round(out["nb"] / bw_ms, 4), reps=reps)


def routing_stats(buf):
    offsets = buf.offsets.cpu().numpy()
    counts = np.diff(offsets)
    R = int(min(offsets[-1], buf.cap))
    pos = buf.pos.cpu().numpy()
    return dict(counts=counts, R=R, T_act=int(np.sum(np.any(pos >= 0, axis=1))), n_active=int(np.sum(counts > 0)),
                status=int(buf.status[0].item()))


def step_fracs(work, per):
    """Fraction of its roofline reached by every GroupGEMM (bf16 MFMA) and every HBM-bound step."""
    g = {n: round(work[n]["flops"] / (per[n] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4) for n in GEMM_STEPS if n in per}
    h = {n: round(work[n]["bytes"] / (per[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) for n in HBM_STEPS if n in per}
    return g, h


def run_workload(name, args, n_steps, warmup, log):
    """Generate one workload's inputs, build its buffers and time it.  Returns the summary and the state the
    headline needs afterwards (the caller drops it before the next workload)."""
    import torch
    from routing_permute_groupgemm_amd import pipeline, synth
    shape = synth.WORKLOADS[name]
    log(f"{shape.name}: generating inputs")
    inp = synth.make_inputs(shape, seed=args.seed, router=args.router)
    dev = pipeline.to_device(inp)
    zero_copy = not args.copy_rows and (not shape.backward or args.zero_copy)
    buf = pipeline.MoeBuffers.allocate(shape, zero_copy=zero_copy)
    stream = torch.cuda.current_stream()
    steps = layer_steps(shape, dev, buf, args.router)
    log(f"{shape.name}: warmup {warmup}, then {n_steps} steps with events around every step and "
        f"{n_steps} timed")
    t = time_steps(steps, stream, n_steps, warmup)
    log(f"{shape.name}: timed {n_steps} steps: {t['ms_per_step']:.3f} ms/step")
    rs = routing_stats(buf)
    work = algorithmic_work(shape, rs["R"], rs["T_act"], rs["n_active"], zero_copy, args.router)
    per = t["per"]
    gfrac, hfrac = step_fracs(work, per)
    gemm_names = [n for n in GEMM_STEPS if n in per]
    gemm_flops = sum(work[n]["flops"] for n in gemm_names)
    gemm_ms = sum(per[n] for n in gemm_names)
    summ = dict(
        ms_per_step=round(t["ms_per_step"], 4),
        tokens_per_s=round(shape.T / (t["ms_per_step"] * 1e-3), 1),
        pass_="fwd+bwd" if shape.backward else "fwd",
        dispatch="zero-copy" if zero_copy else "row copy",
        routed_rows=rs["R"],
        tokens_active=rs["T_act"],
        experts_active=rs["n_active"],
        maxvio=round(synth.maxvio(rs["counts"], shape.T, shape.K, shape.E), 3),
        dominant=t["dom"],
        dominant_frac=roofline(work[t["dom"]], t["dom_ms"])["frac"],
        groupgemm_mfma_frac=round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        gemm_mfma_frac=gfrac,
        hbm_frac=hfrac,
        step_ms={k: round(v, 4) for k, v in per.items()},
    )
    if rs["status"] != 0:
        summ["warning"] = "row capacity overflow: rows were dropped"
    if shape.backward and not args.no_nb and not zero_copy:  # the two modes are timed on x_perm
        log(f"{shape.name}: weight gradient, bitwise vs non-bitwise")
        summ["wgrad_bw_vs_nb"] = time_wgrad_modes(shape, buf)
    state = dict(shape=shape, inp=inp, dev=dev, buf=buf, steps=steps, t=t, work=work, rs=rs, zero_copy=zero_copy,
                 stream=stream)
    return summ, state


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calib_copy:
        calib_copy()
        return
    if args.tile_sweep:
        tile_sweep()
        return
    from routing_permute_groupgemm_amd import _lib, synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    _lib.load()
    summ, st = run_workload(args.workload, args, args.steps, args.warmup, log)
    shape, buf, work, t, stream = st["shape"], st["buf"], st["work"], st["t"], st["stream"]
    dom, dom_ms, per = t["dom"], t["dom_ms"], t["per"]
    rl = roofline(work[dom], dom_ms)
    rl["launch_ms"] = round(dom_ms, 4)  # the kernel's mean time between the events around it
    rl["kernel"] = dom
    rl["traffic"] = measured_traffic(dom, shape.name)
    # the rate plain copies reach on this GPU: the practical ceiling of the HBM-bound steps
    copy_rates = measured_copy_gbps(stream)
    if rl["bound"] == "hbm":
        # the spec peak above; beside it the best plain copy
        rl["measured_copy_gbps"] = copy_rates["best"]
    else:
        # likewise the rate back-to-back MFMAs on random operands reach on this GPU
        rl["measured_mfma_tflops"] = measured_mfma_tflops(stream)
        rl["measured_mfma16_tflops"] = measured_mfma_tflops(stream, shape=16)
    graph_ms = None
    if args.graph:
        one_step = t["one_step"]
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            one_step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"graph replays: {graph_ms:.3f} ms/step")
    perm_gbs = work["permute"]["bytes"] / (per["permute"] * 1e-3) / 1e9
    comb_gbs = work["combine"]["bytes"] / (per["combine"] * 1e-3) / 1e9
    result = {
        "metric": "MoE layer tokens/s on 1 GPU; GroupGEMM % bf16 MFMA peak; permute GB/s",
        "value": summ["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "H": shape.H, "F": shape.F, "E": shape.E, "K": shape.K,
                   "e_local": shape.EL, "cap_rows": buf.cap, "pass": summ["pass_"], "dispatch": summ["dispatch"],
                   "router_projection": args.router, "routed_rows": summ["routed_rows"],
                   "tokens_active": summ["tokens_active"], "experts_active": summ["experts_active"], "maxvio": summ["maxvio"],
                   "seed": args.seed, "parallelism": "single GPU"},
        "roofline": rl,
        "groupgemm_mfma_frac": summ["groupgemm_mfma_frac"],
        "gemm_mfma_frac": summ["gemm_mfma_frac"],
        # the permute step as a whole (count, scan, rank and the row copy), on its algorithmic bytes
        "permute_gbps": round(perm_gbs, 1),
        "permute_hbm_frac": round(perm_gbs / HBM_PEAK_GBS, 4),
        "permute_dispatch": summ["dispatch"],
        "combine_gbps": round(comb_gbs, 1),
        "combine_hbm_frac": round(comb_gbs / HBM_PEAK_GBS, 4),
        "hbm_frac": summ["hbm_frac"],
        # plain 1 GiB copies (torch's and the copy probe's), and each HBM-bound step against the best
        "copy_gbps": copy_rates,
        "hbm_frac_of_copy": {k: round(v * HBM_PEAK_GBS / copy_rates["best"], 4) for k, v in summ["hbm_frac"].items()},
        "step_ms": summ["step_ms"],
    }
    if "wgrad_bw_vs_nb" in summ:
        result["wgrad_bw_vs_nb"] = summ["wgrad_bw_vs_nb"]
    if graph_ms is not None:
        result["graph_ms_per_step"] = round(graph_ms, 4)
    if args.dense_reference:
        refs = {}
        for n in GEMM_STEPS:
            if n in per and dense_dims(n, shape):
                kd, nn = dense_dims(n, shape)
                refs[n] = dense_reference(summ["routed_rows"], kd, nn, max(3, args.steps // 4))
        result["dense_reference"] = refs
    if "warning" in summ:
        result["warning"] = summ["warning"]
    inp = st["inp"]
    del st, buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    others = [w for w in args.also.split(",") if w and w != args.workload]
    if others:
        result["workloads"] = {}
        for name in others:
            s2, st2 = run_workload(name, args, args.also_steps, min(args.warmup, 3), log)
            del st2
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            s2["pass"] = s2.pop("pass_")
            result["workloads"][name] = s2
    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(shape, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
