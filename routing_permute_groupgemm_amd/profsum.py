"""Turn rocprofv3 CSV output of a bench.py run into the short text summaries kept beside the code.

Three subcommands, all run on the host after the profiled bench run:

  stats     <dir>/<name>_kernel_trace.csv and _kernel_stats.csv of a `--kernel-trace --stats` run
            -> a markdown table of per-step kernel time (every dispatch is labelled with the layer
               step it belongs to) and the profiler's own per-kernel-name table
  counters  <dir>/<tag>_p<i>/p_counter_collection.csv of one `--pmc` run per counter group, and
            <dir>/calib_p3, calib_p4 of a plain device copy under FETCH_SIZE and WRITE_SIZE
            -> a markdown table of derived counter figures per GroupGEMM, and the HBM bytes per
               launch of each GroupGEMM merged into a JSON file that bench.py reads for its
               roofline's traffic figure
  kernels   <run dir>/p_counter_collection.csv of one `--pmc` run per counter group
            -> a markdown table of instruction counts and waits per kernel name

Dispatches are labelled by kernel name; the GroupGEMM template's layout / epilogue / schedule
arguments name its step.  The two weight-gradient launches of a step share one template
instance and are told apart by their order inside the step (dW_gate|dW_up first, dW_down second).
A step starts at each router top-k dispatch and at each router projection, or (in traces filtered
to the GroupGEMMs) at the second launch of the gate/up GroupGEMM since the last start.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (layout, epilogue, schedule) template arguments of the GroupGEMM -> the steps that launch that
# instance, in their order inside a layer step
GG_STEPS = {(1, 1, 0): ("expert_up",), (1, 0, 0): ("expert_down",), (0, 2, 0): ("bwd_down_dgrad",),
            (0, 0, 0): ("bwd_up_dgrad",), (1, 3, 0): ("router_fwd",), (1, 3, 1): ("wgrad_gate_up", "wgrad_down")}
# the router's backward launches the same instances once more, after the layer's own launches
GG_ROUTER = {(0, 0, 0): "router_bwd (dx)", (1, 3, 1): "router_bwd (dW_r)"}
OTHER = [("route_kernel", "route"), ("perm_count_kernel", "permute (count)"), ("perm_rowscan_kernel", "permute (scan)"),
         ("perm_empty_kernel", "permute (no pairs)"),
         ("perm_rank_kernel", "permute (rank)"), ("perm_copy_kernel", "permute (row copy)"),
         ("gather_kernel", "bwd_gather"), ("route_backward_kernel", "route_bwd"),
         ("combine_kernel<true", "combine"), ("combine_kernel<false", "bwd_combine"),
         ("copy_probe_kernel", "copy probe (after the timed steps)"),
         ("mfma16_probe_kernel", "MFMA probe 16x16x32 (after the timed steps)"),
         ("mfma_probe_kernel", "MFMA probe 32x32x16 (after the timed steps)"),
         ("split_offsets_kernel", "wgrad split (offsets)"), ("sum_split_kernel", "wgrad split (sum)"),
         ("cast_bf16_kernel", "router_bwd (cast)"), ("sum_partials_kernel", "router_bwd (dW_r sum)"),
         ("copyBuffer", "runtime copy"), ("at::native", "torch (input set-up)")]
STEP_ORDER = ["router_fwd", "route", "permute (count)", "permute (scan)", "permute (rank)", "permute (row copy)",
              "expert_up", "expert_down", "combine", "bwd_gather", "route_bwd", "bwd_down_dgrad", "bwd_up_dgrad",
              "bwd_combine", "wgrad_gate_up", "wgrad_down", "router_bwd (cast)", "router_bwd (dx)",
              "router_bwd (dW_r)", "router_bwd (dW_r sum)"]
GG_RE = re.compile(r"gg_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\w+)>")


def label_dispatches(rows):
    """rows: dicts with Dispatch_Id and Kernel_Name.  Returns {dispatch id: step label}."""
    out = {}
    seen = collections.Counter()  # GroupGEMM instances launched so far in this layer step
    has_router = router_pending = False
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        name, d = r["Kernel_Name"], int(r["Dispatch_Id"])
        if "route_kernel" in name:
            has_router, router_pending = router_pending, False
            seen.clear()
        m = GG_RE.search(name)
        if m:
            key = (int(m.group(6)), int(m.group(7)), int(m.group(8)))
            if key == (1, 3, 0):  # the router projection opens a step
                seen.clear()
                has_router = router_pending = True
            elif key == (1, 1, 0) and seen[key]:
                seen.clear()  # a new step (traces filtered to the GroupGEMMs have no route dispatch)
                has_router = False
            steps = GG_STEPS.get(key, ("GroupGEMM " + m.group(0),))
            if has_router and key in GG_ROUTER:
                steps = steps + (GG_ROUTER[key],)
            i = seen[key]
            seen[key] += 1
            step = steps[i] if i < len(steps) else steps[-1] + " (extra launch)"
            out[d] = step + (" (gathered rows)" if m.group(11) == "true" else "")
            continue
        for pat, lab in OTHER:
            if pat in name:
                out[d] = lab
                break
        else:
            out[d] = name[:60]
    return out


def bench_json(path):
    """The bench's JSON line (its last line that parses as a JSON object)."""
    res = None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{"):
                try:
                    res = json.loads(line)
                except ValueError:
                    pass
    if res is None:
        raise SystemExit(f"no bench JSON line in {path}")
    return res


def work_of(bj):
    """Algorithmic bytes and flops per launch of every step of the bench's headline workload."""
    sys.path.insert(0, REPO)
    import bench
    from routing_permute_groupgemm_amd import synth
    c = bj["config"]
    shape = synth.WORKLOADS[c["workload"]]
    return bench.algorithmic_work(shape, c["routed_rows"], c["tokens_active"], c["experts_active"],
                                  c["dispatch"] == "zero-copy", c.get("router_projection", False)), bench.src_hash()


def headline_part(trace):
    """The dispatches of the bench's headline workload: those before its first probe kernel (the bench
    measures the copy and MFMA probes' rates after the headline's steps, then runs any other workloads)."""
    trace = sorted(trace, key=lambda r: int(r["Dispatch_Id"]))
    for i, r in enumerate(trace):
        if "probe_kernel" in r["Kernel_Name"]:
            return trace[:i]
    return trace


def cmd_stats(a):
    trace = list(csv.DictReader(open(os.path.join(a.dir, f"{a.name}_kernel_trace.csv"))))
    if a.headline_only:
        trace = headline_part(trace)
    labels = label_dispatches(trace)
    dur = collections.defaultdict(list)
    kname = {}
    for r in trace:
        lab = labels[int(r["Dispatch_Id"])]
        dur[lab].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        kname.setdefault(lab, r["Kernel_Name"])
    total = sum(sum(v) for v in dur.values())
    bj = bench_json(a.bench_log)
    order = [s for s in STEP_ORDER if s in dur] + sorted(s for s in dur if s not in STEP_ORDER)
    L = [f"# Kernel time per step, {bj['config']['workload']}\n",
         "Command (MI355X, ROCm 7.2, from the repository root):\n",
         f"`{a.command}`\n",
         ("The headline workload's dispatches (those before the bench's first probe kernel), each " if a.headline_only
          else "Every dispatch of the run, ") +
         "labelled with the layer step it belongs to (the two weight-gradient launches of a step share one "
         "kernel and are told apart by their order in the step; launches after the last step, such as the "
         "bitwise-vs-non-bitwise weight-gradient timing, are marked as extra). Durations in µs.\n",
         "| step | kernel | dispatches | avg µs | min µs | max µs | share |", "|---|---|---|---|---|---|---|"]
    for s in order:
        v = dur[s]
        kn = kname[s].replace("|", "\\|")
        kn = kn if len(kn) <= 72 else kn[:72] + "…"
        L.append(f"| {s} | `{kn}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                 f"{100 * sum(v) / total:.1f}% |")
    rl = bj["roofline"]
    L.append("")
    L.append(f"Bench line of the same run: {bj['value']:.0f} {bj['unit']}, {bj['ms_per_step']} ms/step; roofline kernel "
             f"{rl['kernel']}: {rl['launch_ms']} ms per launch between HIP events, {rl['achieved']} {rl['unit']} = "
             f"{rl['frac']} of {rl['peak']}.")
    sp = os.path.join(a.dir, f"{a.name}_kernel_stats.csv")
    if os.path.exists(sp):
        L.append("\nThe profiler's own `--stats` table (per kernel name over the whole run; the weight-gradient row "
                 "mixes both launches" + (" and the other workloads' kernels share these names" if a.headline_only
                                          else "") + "):\n")
        L.append("| kernel | calls | avg µs | min µs | max µs | % |")
        L.append("|---|---|---|---|---|---|")
        for r in list(csv.DictReader(open(sp)))[:a.top]:
            kn = r["Name"].replace("|", "\\|")
            kn = kn if len(kn) <= 72 else kn[:72] + "…"
            L.append(f"| `{kn}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {r['Percentage']} |")
    open(a.out, "w").write("\n".join(L) + "\n")
    print("\n".join(L))


COUNTER_GROUPS = {
    1: "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES "
       "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS",
    2: "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_SMEM "
       "SQ_CYCLES",
    3: "FETCH_SIZE",
    4: "WRITE_SIZE",
    5: "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE GRBM_COUNT",
}


def load_pass(path):
    rows = list(csv.DictReader(open(path)))
    labels = label_dispatches(list({r["Dispatch_Id"]: r for r in rows}.values()))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, cs in per.items():
        for c, v in cs.items():
            agg[labels[d]][c].append(v)
        agg[labels[d]]["_dur"].append(dur[d])
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}, \
        {k: len(v["_dur"]) for k, v in agg.items()}


def calib_factor(path, counter):
    """Counted KiB per KiB moved by the 1 GiB device copy of `bench.py --calib-copy`."""
    vals = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    big = [v for v in vals.values() if v > 1e5]
    if not big:
        raise SystemExit(f"no copy dispatch in {path}")
    return sum(big) / len(big) / (1 << 20)


def cmd_counters(a):
    bj = bench_json(a.bench_log)
    wl = bj["config"]["workload"]
    work, sha = work_of(bj)
    ff = calib_factor(os.path.join(a.dir, "calib_p3", "p_counter_collection.csv"), "FETCH_SIZE")
    wf = calib_factor(os.path.join(a.dir, "calib_p4", "p_counter_collection.csv"), "WRITE_SIZE")
    res = collections.defaultdict(dict)
    ndisp, durs = {}, collections.defaultdict(list)
    for i in COUNTER_GROUPS:
        r, n = load_pass(os.path.join(a.dir, f"{a.tag}_p{i}", "p_counter_collection.csv"))
        for k, cs in r.items():
            durs[k].append(cs.pop("_dur"))
            res[k].update(cs)
            ndisp[k] = n[k]
    base = lambda lab: lab.replace(" (gathered rows)", "")  # noqa: E731  the step a label belongs to
    order = {n: i for i, n in enumerate(STEP_ORDER)}
    gemms = sorted((s for s in res if base(s) in work and work[base(s)]["flops"]), key=lambda s: order.get(base(s), 99))
    L = [f"# Counters of the GroupGEMMs, {wl}\n",
         f"One rocprofv3 counter run per group (MI355X, ROCm 7.2), every GroupGEMM dispatch of the run:\n",
         f"`{a.command}`\n", "with `<group>` one of:\n"]
    L += [f"{i}. `{g}`" for i, g in COUNTER_GROUPS.items()]
    L.append("\nHBM bytes: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch) divided by what the same counter reads for "
             f"a plain 1 GiB device copy (`{a.calib_command}`, once per counter): fetch factor {ff:.4f}, write "
             f"factor {wf:.4f} counted KiB per KiB moved. Values are means over the dispatches of each step.\n")
    L.append("Derived: clock = (`GRBM_GUI_ACTIVE`/8) / dispatch time; MFMA busy = `SQ_VALU_MFMA_BUSY_CYCLES` / "
             "(`GRBM_GUI_ACTIVE`/8 x 1024 SIMDs); wait shares = `SQ_WAIT_INST_ANY` (`SQ_WAIT_INST_LDS`) / "
             "`SQ_WAVE_CYCLES`; L2 hit = `TCC_HIT_sum` / (`TCC_HIT_sum` + `TCC_MISS_sum`); per-MFMA instruction "
             "ratios from `SQ_INSTS_*`; HBM read / write the scaled `FETCH_SIZE` / `WRITE_SIZE` against the step's "
             "algorithmic bytes.\n")
    L.append("| GEMM | dispatches | µs (pass 5) | clock GHz | MFMA busy | wait share | LDS-wait share | SALU/MFMA | "
             "VALU/MFMA | LDS/MFMA | L2 hit | LDS bank conflict / active | HBM read GB | HBM write GB | "
             "algorithmic GB | (read+write)/algorithmic |")
    L.append("|" + "---|" * 16)
    try:
        traffic = json.load(open(a.traffic))
    except (OSError, ValueError):
        traffic = {}
    for s in gemms:
        c = res[s]
        dur = durs[s][4]
        gui = c["GRBM_GUI_ACTIVE"] / 8
        mf = c["SQ_INSTS_MFMA"]
        rd = c["FETCH_SIZE"] * 1024 / ff / 1e9
        wr = c["WRITE_SIZE"] * 1024 / wf / 1e9
        alg = work[base(s)]["bytes"] / 1e9
        L.append(f"| {s} | {ndisp[s]} | {dur * 1e6:.0f} | {gui / dur / 1e9:.2f} | "
                 f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * 1024):.3f} | {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.3f} | "
                 f"{c['SQ_WAIT_INST_LDS'] / c['SQ_WAVE_CYCLES']:.3f} | {c['SQ_INSTS_SALU'] / mf:.2f} | "
                 f"{(c['SQ_INSTS_VALU'] - mf) / mf:.2f} | {c['SQ_INSTS_LDS'] / mf:.2f} | "
                 f"{c['TCC_HIT_sum'] / (c['TCC_HIT_sum'] + c['TCC_MISS_sum']):.3f} | "
                 f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.3f} | {rd:.2f} | {wr:.2f} | "
                 f"{alg:.2f} | {(rd + wr) / alg:.2f} |")
        traffic[f"{base(s)}@{wl}"] = dict(gemm_src_sha=sha, traffic_bytes_per_launch=int((rd + wr) * 1e9),
                                    fetch_kib=round(c["FETCH_SIZE"], 1), write_kib=round(c["WRITE_SIZE"], 1),
                                    fetch_factor=round(ff, 6), write_factor=round(wf, 6), dispatches=ndisp[s])
    L.append("\nRaw means per dispatch:\n")
    cn = sorted({c for s in gemms for c in res[s]})
    L.append("| counter | " + " | ".join(gemms) + " |")
    L.append("|---|" + "---|" * len(gemms))
    for c in cn:
        L.append(f"| `{c}` | " + " | ".join(f"{res[s].get(c, float('nan')):.4g}" for s in gemms) + " |")
    open(a.out, "w").write("\n".join(L) + "\n")
    with open(a.traffic, "w") as fh:
        json.dump(dict(sorted(traffic.items())), fh, indent=1)
        fh.write("\n")
    print("\n".join(L[:20 + len(gemms)]))


def cmd_kernels(a):
    """Counter means per dispatch of every kernel in one or more counter runs, by kernel name."""
    res = collections.defaultdict(dict)
    durs = collections.defaultdict(list)
    for d in a.runs:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        kn, dur = {}, {}
        for r in csv.DictReader(open(os.path.join(d, "p_counter_collection.csv"))):
            i = r["Dispatch_Id"]
            per[i][r["Counter_Name"]] += float(r["Counter_Value"])
            kn[i] = r["Kernel_Name"].split("(")[0].replace("void ", "")
            dur[i] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for i, cs in per.items():
            for c, v in cs.items():
                agg[kn[i]][c].append(v)
            durs[kn[i]].append(dur[i])
        for k, cs in agg.items():
            for c, v in cs.items():
                res[k][c] = sum(v) / len(v)
    L = [f"# {a.title}\n", "One rocprofv3 counter run per group (MI355X, ROCm 7.2):\n", f"`{a.command}`\n",
         "with `<group>` one of:\n"]
    L += [f"{i + 1}. `{g}`" for i, g in enumerate(a.groups)]
    L.append(f"\nMeans per dispatch; per-unit figures divide by {a.per_name} = {a.per}. VALU busy = "
             "4·`SQ_ACTIVE_INST_VALU` / (1024 SIMDs × `GRBM_GUI_ACTIVE`/8), the share of the SIMDs' cycles "
             "spent issuing VALU instructions (a wave64 VALU instruction takes 4 cycles; `GRBM_GUI_ACTIVE` also "
             "counts the cycles around a short dispatch, so this under-states it for short kernels).\n")
    L.append(f"| kernel | µs | VALU / {a.per_name} | SALU / {a.per_name} | LDS / {a.per_name} | VALU busy | "
             "wait share (`SQ_WAIT_INST_ANY` / `SQ_WAVE_CYCLES`) |")
    L.append("|---|---|---|---|---|---|---|")
    for k, c in res.items():
        gui = c.get("GRBM_GUI_ACTIVE", float("nan")) / 8
        L.append(f"| `{k}` | {sum(durs[k]) / len(durs[k]):.1f} | {c['SQ_INSTS_VALU'] / a.per:.0f} | "
                 f"{c['SQ_INSTS_SALU'] / a.per:.0f} | {c['SQ_INSTS_LDS'] / a.per:.0f} | "
                 f"{4 * c['SQ_ACTIVE_INST_VALU'] / (1024 * gui):.2f} | "
                 f"{c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.2f} |")
    L += ["", "Raw means per dispatch:", "", "| counter | " + " | ".join(f"`{k}`" for k in res) + " |",
          "|---|" + "---|" * len(res)]
    for cn in sorted({c for v in res.values() for c in v}):
        L.append(f"| `{cn}` | " + " | ".join(f"{res[k].get(cn, float('nan')):.4g}" for k in res) + " |")
    open(a.out, "w").write("\n".join(L) + "\n")
    print("\n".join(L[:12 + len(res)]))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m routing_permute_groupgemm_amd.profsum")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--name", default="kt", help="rocprofv3 -o name")
    s.add_argument("--bench-log", required=True, help="stdout of the profiled bench run")
    s.add_argument("--command", required=True, help="the profiled command, quoted in the summary")
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=20)
    s.add_argument("--headline-only", action="store_true",
                   help="summarise only the headline workload of a default bench run (dispatches before the probes)")
    c = sub.add_parser("counters")
    c.add_argument("--dir", required=True)
    c.add_argument("--tag", required=True, help="counter runs are <dir>/<tag>_p1 ... _p5")
    c.add_argument("--bench-log", required=True, help="stdout of one of the counter runs")
    c.add_argument("--command", required=True)
    c.add_argument("--calib-command", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--traffic", default=os.path.join(REPO, "profiles", "traffic.json"))
    k = sub.add_parser("kernels")
    k.add_argument("--runs", nargs="+", required=True, help="rocprofv3 -d directories, one per counter group")
    k.add_argument("--groups", nargs="+", required=True, help="the counter groups, quoted, in run order")
    k.add_argument("--per", type=float, default=1.0)
    k.add_argument("--per-name", default="dispatch")
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "kernels": cmd_kernels}[a.cmd](a)


if __name__ == "__main__":
    main()
