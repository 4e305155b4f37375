"""bench.py's host-side contract (CPU only): more than one GPU is refused
with a message, and the algorithmic work it divides by is the real-rows-only
count (no padding, each expert's weights once)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_counts_real_rows_only():
    import bench
    from routing_permute_groupgemm_amd import synth
    s = synth.WORKLOADS["ep_share_4k"]
    T, H, F, E, K, EL = s.T, s.H, s.F, s.E, s.K, s.EL
    R, T_act, n_act = 4077, 2750, 31
    w = bench.algorithmic_work(s, R, T_act, n_act)
    # the gate/up GEMM streams each active expert's two weights once, its rows and its output
    assert w["expert_up"]["bytes"] == 2 * n_act * H * 2 * F + 2 * R * H + 2 * R * F
    assert w["expert_up"]["flops"] == 4 * R * H * F
    assert w["expert_down"]["flops"] == 2 * R * F * H
    assert w["combine"]["bytes"] == 2 * H * R + 8 * T * K + 2 * H * T
    # zero-copy moves indices only in the permute step
    wz = bench.algorithmic_work(s, R, T_act, n_act, zero_copy=True)
    assert w["permute"]["bytes"] - wz["permute"]["bytes"] == 2 * H * T_act + 2 * H * R
    # the router steps appear only when asked for
    assert "router_fwd" not in w
    wr = bench.algorithmic_work(s, R, T_act, n_act, router=True)
    assert wr["router_fwd"]["flops"] == 2 * T * H * E


def _gg(lay, epi, sched, gather="false"):
    return f"void moe::gg_kernel<256, 256, 32, 2, 2, {lay}, {epi}, {sched}, 131072, 0, {gather}>(moe::GemmParams)"


def test_profile_summaries_label_every_step():
    """profsum names each dispatch of a traced bench run after its layer step: the two weight-gradient
    launches of a step share one kernel and are told apart by order, traces filtered to the GroupGEMMs
    (no route dispatch) still split into steps, and the router's extra launches get their own names."""
    from routing_permute_groupgemm_amd import profsum
    step = ["void moe::route_kernel<4, true>(float const*)", "moe::perm_count_kernel(int const*)",
            "moe::perm_rowscan_kernel(int*, int, int*)", "void moe::perm_rank_kernel<8, false>(int const*)",
            "void moe::perm_copy_kernel<4>(int)", _gg(1, 1, 0), _gg(1, 0, 0), "void moe::combine_kernel<true, true>(int)",
            "void moe::gather_kernel<true, true>(int)", "void moe::route_backward_kernel<256>(int)", _gg(0, 2, 0),
            _gg(0, 0, 0), "void moe::combine_kernel<false, true>(int)", _gg(1, 3, 1), _gg(1, 3, 1)]
    want = ["route", "permute (count)", "permute (scan)", "permute (rank)", "permute (row copy)", "expert_up",
            "expert_down", "combine", "bwd_gather", "route_bwd", "bwd_down_dgrad", "bwd_up_dgrad", "bwd_combine",
            "wgrad_gate_up", "wgrad_down"]
    rows = [dict(Dispatch_Id=str(i + 1), Kernel_Name=k) for i, k in enumerate(step * 3)]
    lab = profsum.label_dispatches(rows)
    assert [lab[i + 1] for i in range(len(rows))] == want * 3
    # only the GroupGEMMs (a counter run filtered by kernel name): the same labels, step after step
    gg = [r for r in rows if "gg_kernel" in r["Kernel_Name"]]
    lab = profsum.label_dispatches(gg)
    assert [lab[int(r["Dispatch_Id"])] for r in gg] == [w for w in want if w.startswith(("expert", "bwd_d", "bwd_u", "wgrad"))] * 3
    # with the router: its forward GEMM first, its backward's cast, dx and dW_r GEMMs and ordered sum last
    rstep = [_gg(1, 3, 0)] + step + ["moe::cast_bf16_kernel(float)", _gg(0, 0, 0), _gg(1, 3, 1),
                                     "moe::sum_partials_kernel(float)"]
    rows = [dict(Dispatch_Id=str(i + 1), Kernel_Name=k) for i, k in enumerate(rstep * 2)]
    lab = [profsum.label_dispatches(rows)[i + 1] for i in range(len(rows))]
    assert lab[:len(rstep)] == ["router_fwd"] + want + ["router_bwd (cast)", "router_bwd (dx)", "router_bwd (dW_r)",
                                                         "router_bwd (dW_r sum)"]
    assert lab[len(rstep):] == lab[:len(rstep)]
    # the zero-copy gate/up GEMM keeps its step name, marked
    assert profsum.label_dispatches([dict(Dispatch_Id="1", Kernel_Name=_gg(1, 1, 0, "true"))])[1] == \
        "expert_up (gathered rows)"


def test_profile_summaries_mark_launches_after_the_last_step():
    """Weight-gradient launches after a step without the router (the bench's bitwise-vs-non-bitwise timing)
    are marked as extra launches, not taken for the router's; a headline-only summary stops at the probes."""
    from routing_permute_groupgemm_amd import profsum
    names = ["void moe::route_kernel<4, true>(float const*)", _gg(1, 1, 0), _gg(1, 3, 1), _gg(1, 3, 1),
             _gg(1, 3, 1), "moe::split_offsets_kernel(int)", _gg(1, 3, 1), "moe::mfma_probe_kernel(int)",
             "void moe::route_kernel<2, true>(float const*)"]
    rows = [dict(Dispatch_Id=str(i + 1), Kernel_Name=k) for i, k in enumerate(names)]
    lab = profsum.label_dispatches(rows)
    assert [lab[i] for i in (3, 4, 5, 7)] == ["wgrad_gate_up", "wgrad_down", "wgrad_down (extra launch)",
                                               "wgrad_down (extra launch)"]
    assert len(profsum.headline_part(rows)) == 7
