"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before touching the GPU (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

from routing_permute_groupgemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for need in ("moe_route", "moe_permute", "moe_grouped_gemm_swiglu", "moe_grouped_gemm", "moe_combine",
                 "moe_wgrad", "moe_gather", "moe_gather_gate_grad", "moe_route_backward",
                 "moe_grouped_gemm_swiglu_gather", "moe_router_logits", "moe_router_backward"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib._LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(moe_\w+)", nm))
    for name in declared_symbols():
        assert name in exported, f"{name} declared in moe.h but not exported"
        assert hasattr(lib, name)
    assert set(_lib.SIGNATURES) == set(declared_symbols())


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("pytorch", "")
    assert "extern \"C\"" in text


def test_strerror_and_version():
    lib = _lib.load()
    assert lib.moe_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.moe_strerror(code)
    assert lib.moe_strerror(-99) == b"unknown status"


def test_workspace_size_host_only():
    lib = _lib.load()
    assert lib.moe_permute_workspace_size(131072, 8, 32) >= 512 * 32 * 4
    assert lib.moe_permute_workspace_size(0, 8, 32) > 0


# Invalid arguments are rejected before anything is enqueued (no GPU needed).
FAKE = 0x10000  # aligned, never dereferenced: validation fails first
MIS = 0x10002   # misaligned


@pytest.mark.parametrize("args,want", [
    ((FAKE, 16, 8, 9, FAKE, FAKE, None), -2),       # K > E
    ((FAKE, 16, 8, 0, FAKE, FAKE, None), -1),       # K < 1
    ((FAKE, 16, 8, 17, FAKE, FAKE, None), -1),      # K > 16
    ((FAKE, 16, 600, 8, FAKE, FAKE, None), -1),     # E > 512
    ((None, 16, 8, 2, FAKE, FAKE, None), -1),       # NULL logits
    ((MIS, 16, 8, 2, FAKE, FAKE, None), -3),        # misaligned
    ((FAKE, -1, 8, 2, FAKE, FAKE, None), -1),       # negative T
])
def test_route_rejects(args, want):
    assert _lib.load().moe_route(*args) == want


def test_route_zero_tokens_is_noop():
    assert _lib.load().moe_route(None, 0, 8, 2, None, None, None) == 0


def test_permute_rejects():
    lib = _lib.load()
    ok = dict(idx=FAKE, T=16, K=2, eb=0, el=8, x=FAKE, H=64, cap=32, counts=FAKE, offsets=FAKE, pos=FAKE,
              src=FAKE, xp=FAKE, st=FAKE, ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_permute(a["idx"], a["T"], a["K"], a["eb"], a["el"], a["x"], a["H"], a["cap"], a["counts"],
                               a["offsets"], a["pos"], a["src"], a["xp"], a["st"], a["ws"], a["wsb"], None)

    assert call(H=96) == -2            # H not a multiple of 64
    assert call(wsb=4) == -4           # workspace too small
    assert call(ws=None) == -4
    assert call(x=MIS) == -3
    assert call(cap=33) == -1          # cap > T*K
    assert call(el=513) == -1
    assert call(offsets=None) == -1
    assert call(x=None) == -1          # rows to copy but no x


def test_router_rejects():
    lib = _lib.load()
    # (x, T, H, w_r, E, bias, logits, ws, ws_bytes, stream)
    assert lib.moe_router_logits(FAKE, 64, 128, FAKE, 8, None, FAKE, FAKE, 1 << 20, None) == -2    # E % 64
    assert lib.moe_router_logits(FAKE, 64, 96, FAKE, 64, None, FAKE, FAKE, 1 << 20, None) == -2    # H % 64
    assert lib.moe_router_logits(FAKE, -1, 128, FAKE, 64, None, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.moe_router_logits(FAKE, 64, 128, None, 64, None, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.moe_router_logits(FAKE, 64, 128, FAKE, 64, MIS, FAKE, FAKE, 1 << 20, None) == -3
    # a split contraction needs the workspace
    T, H, E = 512, 7168, 256
    need = lib.moe_router_workspace_size(T, H, E)
    assert need > 0
    assert lib.moe_router_logits(FAKE, T, H, FAKE, E, None, FAKE, None, 0, None) == -4
    assert lib.moe_router_logits(FAKE, T, H, FAKE, E, None, FAKE, FAKE, 256, None) == -4
    # (x, T, H, w_r, E, dlogits, dx, dw_r, ws, ws_bytes, stream): the backward always needs it
    assert lib.moe_router_backward(FAKE, T, H, FAKE, E, FAKE, FAKE, FAKE, None, 0, None) == -4
    assert lib.moe_router_backward(FAKE, T, H, FAKE, E, FAKE, FAKE, None, FAKE, need, None) == -1
    assert lib.moe_router_backward(FAKE, T, H, FAKE, 8, FAKE, FAKE, FAKE, FAKE, need, None) == -2
    assert lib.moe_router_workspace_size(T, H, 8) == 0


def test_gather_wgrad_rejects():
    lib = _lib.load()
    g = lib.moe_wgrad_gate_up_gather
    # (x, T, src, K, H, dab, F, offsets, e_local, cap, dw_gate, dw_up, stream)
    assert g(FAKE, 64, FAKE, 2, 96, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -2   # H % 64
    assert g(FAKE, 64, FAKE, 2, 64, FAKE, 48, FAKE, 4, 16, FAKE, FAKE, None) == -2   # F % 64
    assert g(FAKE, 64, FAKE, 0, 64, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -1   # K < 1
    assert g(FAKE, 64, FAKE, 17, 64, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -1  # K > 16
    assert g(FAKE, 8, FAKE, 1, 64, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -1    # cap > T*K
    assert g(FAKE, 1966081, FAKE, 8, 1024, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -1  # x past 0xF0000000 B
    assert g(FAKE, 64, FAKE, 2, 64, FAKE, 64, None, 4, 16, FAKE, FAKE, None) == -1   # no offsets
    assert g(FAKE, 64, None, 2, 64, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -1   # no src
    assert g(FAKE, 64, FAKE, 2, 64, FAKE, 64, FAKE, 4, 16, None, FAKE, None) == -1   # no dw_gate
    assert g(MIS, 64, FAKE, 2, 64, FAKE, 64, FAKE, 4, 16, FAKE, FAKE, None) == -3    # misaligned
    assert g(None, 64, None, 2, 64, None, 64, FAKE, 0, 16, None, None, None) == 0    # no experts: nothing to do


def test_gather_gemm_rejects():
    lib = _lib.load()
    g = lib.moe_grouped_gemm_swiglu_gather
    # (x, T, src, K, w_gate, w_up, offsets, e_local, H, F, cap, h, ab, stream)
    assert g(FAKE, 64, FAKE, 2, FAKE, FAKE, FAKE, 4, 96, 64, 16, FAKE, None, None) == -2   # H % 64
    assert g(FAKE, 64, FAKE, 2, FAKE, FAKE, None, 4, 64, 64, 16, FAKE, None, None) == -1   # no offsets
    assert g(FAKE, 64, FAKE, 0, FAKE, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -1   # K < 1
    assert g(FAKE, 64, FAKE, 17, FAKE, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -1  # K > 16
    assert g(FAKE, 8, FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -1    # cap > T*K
    # x past 0xF0000000 bytes: T*H*2 = 0xF0000000 + 2048
    assert g(FAKE, 1966081, FAKE, 8, FAKE, FAKE, FAKE, 4, 1024, 64, 16, FAKE, None, None) == -1
    assert g(FAKE, 64, None, 2, FAKE, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -1   # no src
    assert g(FAKE, 64, MIS, 2, FAKE, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -3    # misaligned


def test_gemm_rejects():
    lib = _lib.load()
    # H not multiple of 64
    assert lib.moe_grouped_gemm_swiglu(FAKE, FAKE, FAKE, FAKE, 4, 96, 64, 16, FAKE, None, None) == -2
    assert lib.moe_grouped_gemm_swiglu(FAKE, FAKE, FAKE, None, 4, 64, 64, 16, FAKE, None, None) == -1
    assert lib.moe_grouped_gemm_swiglu(FAKE, MIS, FAKE, FAKE, 4, 64, 64, 16, FAKE, None, None) == -3
    # w1 only with trans_w = 1; lda too small; bad epilogue; SWIGLU_BWD needs ab
    assert lib.moe_grouped_gemm(FAKE, 64, FAKE, FAKE, 0, FAKE, 4, 64, 64, 16, 0, None, FAKE, 64, None) == -1
    assert lib.moe_grouped_gemm(FAKE, 64, FAKE, FAKE, 1, FAKE, 4, 64, 64, 16, 0, None, FAKE, 64, None) == -1
    assert lib.moe_grouped_gemm(FAKE, 64, FAKE, None, 0, FAKE, 4, 64, 64, 16, 7, None, FAKE, 64, None) == -1
    assert lib.moe_grouped_gemm(FAKE, 64, FAKE, None, 1, FAKE, 4, 64, 64, 16, 1, None, FAKE, 128, None) == -1
    # one expert's weight matrix of 2 GiB or more (32-bit load offsets)
    assert lib.moe_grouped_gemm_swiglu(FAKE, FAKE, FAKE, FAKE, 4, 16384, 65536, 16, FAKE, None, None) == -1
    assert lib.moe_grouped_gemm_swiglu_gather(FAKE, 8, FAKE, 2, FAKE, FAKE, FAKE, 4, 16384, 65536, 16, FAKE,
                                              None, None) == -1
    assert lib.moe_grouped_gemm(FAKE, 16384, FAKE, None, 0, FAKE, 4, 16384, 65536, 16, 0, None, FAKE, 65536,
                                None) == -1
    assert lib.moe_wgrad(FAKE, 64, FAKE, 64, FAKE, 4, 96, 64, 16, FAKE, None) == -2
    assert lib.moe_wgrad(FAKE, 32, FAKE, 64, FAKE, 4, 64, 64, 16, FAKE, None) == -1
    assert lib.moe_combine(FAKE, FAKE, None, 8, 2, 100, FAKE, None) == -2
    assert lib.moe_combine(FAKE, None, None, 8, 2, 64, FAKE, None) == -1
    assert lib.moe_gather(FAKE, FAKE, None, 8, 0, 64, FAKE, None) == -1


def test_router_backward_rejects():
    lib = _lib.load()
    g = lib.moe_gather_gate_grad
    assert g(FAKE, FAKE, None, FAKE, 8, 2, 64, FAKE, FAKE, None) == -1     # gates required
    assert g(FAKE, FAKE, FAKE, None, 8, 2, 64, FAKE, FAKE, None) == -1     # y required
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 2, 64, FAKE, None, None) == -1     # dgates required
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 17, 64, FAKE, FAKE, None) == -1    # K > 16
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 2, 100, FAKE, FAKE, None) == -2    # H % 64
    assert g(FAKE, FAKE, FAKE, MIS, 8, 2, 64, FAKE, FAKE, None) == -3
    assert g(None, None, None, None, 0, 2, 64, None, None, None) == 0      # no tokens: nothing to do
    r = lib.moe_route_backward
    assert r(FAKE, FAKE, FAKE, 8, 4, 5, FAKE, None) == -2                  # K > E
    assert r(FAKE, FAKE, FAKE, 8, 600, 2, FAKE, None) == -1                # E > 512
    assert r(FAKE, None, FAKE, 8, 8, 2, FAKE, None) == -1
    assert r(FAKE, FAKE, FAKE, 8, 8, 2, MIS, None) == -3
    assert r(None, None, None, 0, 8, 2, None, None) == 0


def test_pair_index_division_by_reciprocal():
    """The zero-copy GEMM turns a pair index v = t*K + k (v < 2^31) into t with the host's
    floor((2^32-1)/K), a high multiply and one correction; check that formula on edge values."""
    import numpy as np
    rng = np.random.default_rng(0)
    for K in range(1, 17):
        rcp = 0xFFFFFFFF // K
        t = np.concatenate([np.arange(0, 4096), rng.integers(0, (1 << 31) // K, 20000),
                            [(1 << 31) // K - 1]]).astype(np.uint64)
        for k in range(K):
            v = t * K + k
            v = v[v < (1 << 31)]
            q = (v * rcp) >> 32
            q = q + ((v - q * K) >= K)
            assert np.array_equal(q, v // K), K


def test_binding_rejects_wrong_buffer_shapes():
    """The shape checks the binding applies to every caller buffer before the C call (the C ABI sees
    only pointers), exercised on CPU tensors; the wrappers themselves take CUDA tensors only."""
    import torch

    with pytest.raises(_lib.MoeError):
        _lib._shape(torch.empty(3, 4), (3, 5), "t")
    with pytest.raises(_lib.MoeError):
        _lib._rows(torch.empty(7, 4), 8, 4, "t")
    with pytest.raises(_lib.MoeError):
        _lib._rows(torch.empty(9, 5), 8, 4, "t")
    _lib._rows(torch.empty(9, 4), 8, 4, "t")
    _lib._shape(torch.empty(3, 4), (3, 4), "t")


def test_probe_rejects():
    lib = _lib.load()
    p = lib.moe_probe_mfma
    assert p(FAKE, 0, 10, FAKE, None) == -1      # no blocks
    assert p(FAKE, 4, -1, FAKE, None) == -1      # negative iteration count
    assert p(None, 4, 10, FAKE, None) == -1
    assert p(FAKE, 4, 10, None, None) == -1
    assert p(MIS, 4, 10, FAKE, None) == -3
    c = lib.moe_probe_copy
    assert c(FAKE, FAKE, 24, 0, 0, None) == -1           # not a multiple of 16 bytes
    assert c(FAKE, FAKE, -16, 0, 0, None) == -1
    assert c(FAKE, FAKE, 64, 4, 0, None) == -1           # hint bits beyond 0..3
    assert c(FAKE, FAKE, 64, 0, -1, None) == -1
    assert c(None, FAKE, 64, 0, 0, None) == -1
    assert c(MIS, FAKE, 64, 0, 0, None) == -3
    assert c(None, None, 0, 3, 0, None) == 0             # nothing to copy: no launch


def test_permute_noalloc_rejects_on_the_host():
    # more count matrix than the library's 1 MiB device array holds, and a NULL status word: both are
    # refused before any device call
    lib = _lib.load()
    T, K, e_local = 1 << 20, 2, 64
    assert lib.moe_permute_workspace_size(T, K, e_local) > (1 << 20)
    assert lib.moe_permute_noalloc(FAKE, T, K, 0, e_local, FAKE, 64, T * K, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == -4
    assert lib.moe_permute_noalloc(FAKE, 64, 2, 0, 8, FAKE, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   None) == -1
    assert lib.moe_permute_noalloc(MIS, 64, 2, 0, 8, FAKE, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == -3


def test_wgrad_split_rejects_on_the_host():
    lib = _lib.load()
    assert lib.moe_wgrad_split_workspace_size(8, 128, 128, 1) == 0
    assert lib.moe_wgrad_split_workspace_size(8, 128, 128, 2) >= 16 * 128 * 128 * 4
    assert lib.moe_wgrad_split_workspace_size(300, 128, 128, 2) == 0  # more than 512 chunk groups
    # splits < 1, too many chunk groups, no workspace, a misaligned workspace
    assert lib.moe_wgrad_split(FAKE, 128, FAKE, 128, FAKE, 8, 128, 128, 64, 0, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.moe_wgrad_split(FAKE, 128, FAKE, 128, FAKE, 300, 128, 128, 64, 2, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.moe_wgrad_split(FAKE, 128, FAKE, 128, FAKE, 8, 128, 128, 64, 2, FAKE, None, 0, None) == -4
    assert lib.moe_wgrad_split(FAKE, 128, FAKE, 128, FAKE, 8, 128, 128, 64, 2, FAKE, MIS, 1 << 30, None) == -3


def test_wgrad_gate_up_rejects_on_the_host():
    lib = _lib.load()
    assert lib.moe_wgrad_gate_up(FAKE, 100, FAKE, 64, FAKE, 4, 64, FAKE, FAKE, None) == -2   # H % 64
    assert lib.moe_wgrad_gate_up(FAKE, 128, FAKE, 64, FAKE, 4, 64, FAKE, None, None) == -1   # no dw_up
    assert lib.moe_wgrad_gate_up(FAKE, 128, FAKE, 64, None, 4, 64, FAKE, FAKE, None) == -1   # no offsets
    assert lib.moe_wgrad_gate_up(FAKE, 128, FAKE, 64, FAKE, 4, 64, FAKE, MIS, None) == -3
    assert lib.moe_wgrad_gate_up(FAKE, 128, FAKE, 64, FAKE, 600, 64, FAKE, FAKE, None) == -1  # e_local > 512
