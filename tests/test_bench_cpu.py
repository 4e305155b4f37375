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
