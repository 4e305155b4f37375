"""The layer's forward and backward replay from a HIP graph (torch.cuda.CUDAGraph).

No entry point allocates, synchronises, reads device data on the host or
records a memset, so a whole step can be captured once and replayed.  Each
replay must reproduce the eager results bit for bit (the kernels are
deterministic); the outputs are overwritten by eager work between replays so
a replay that wrote nothing would fail."""
import pytest
import torch

from routing_permute_groupgemm_amd import pipeline, synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
FWD_BWD = ("topk_idx", "gates", "offsets", "pos", "src", "x_perm", "h", "ab", "y", "out", "dy_perm", "dab",
           "dx_perm", "dx", "dw_gate", "dw_up", "dw_down", "dgates", "dlogits")
FWD_ZC = ("topk_idx", "gates", "offsets", "pos", "src", "h", "y", "out")
# row buffers of capacity cap_rows: only their first R rows are defined
ROWS = ("src", "x_perm", "h", "ab", "y", "dy_perm", "dab", "dx_perm")


def defined(buf, n, R):
    t = getattr(buf, n)
    return t[:R] if n in ROWS else t


def snapshot(buf, names, R):
    return {n: defined(buf, n, R).clone() for n in names}


def same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


@pytest.mark.parametrize("zero_copy", [False, True])
def test_layer_replays_from_a_graph(zero_copy):
    shape = W["ep_share_4k"].scaled(T=512, H=256, F=192, backward=not zero_copy)
    print(f"[graph] {shape.name} zero_copy={zero_copy}", flush=True)
    inp = synth.make_inputs(shape, seed=12, d_out=not zero_copy)
    dev = pipeline.to_device(inp)
    buf = pipeline.MoeBuffers.allocate(shape, zero_copy=zero_copy)
    names = FWD_ZC if zero_copy else FWD_BWD

    def step():
        pipeline.forward(buf, dev)
        if not zero_copy:
            pipeline.backward(buf, dev)

    step()
    torch.cuda.synchronize()
    R = min(int(buf.offsets[-1].item()), buf.cap)
    ref = snapshot(buf, names, R)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        for n in names:  # eager work between replays: clobber every output
            getattr(buf, n).fill_(-3 if getattr(buf, n).dtype in (torch.int32,) else 7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = [n for n in names if not same(defined(buf, n, R), ref[n])]
        assert not bad, f"replay {i}: {bad} differ from the eager run"
