"""Comparison helpers shared by the GPU parity tests."""
import numpy as np

from routing_permute_groupgemm_amd import synth

ATOL = 1e-2
RTOL = 1e-2


def as_f32(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def assert_close(name, got, want):
    """Elementwise |got - want| <= 1e-2 + 1e-2*|want| (both fp32/bf16 arrays)."""
    g, w = as_f32(got).astype(np.float64), as_f32(want).astype(np.float64)
    assert g.shape == w.shape, f"{name}: shape {g.shape} vs {w.shape}"
    err = np.abs(g - w)
    bad = ~(err <= ATOL + RTOL * np.abs(w))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} out of tolerance; first at {tuple(i)}: "
                             f"gpu={g[tuple(i)]!r} oracle={w[tuple(i)]!r}")
    return float(err.max()) if err.size else 0.0, float(np.mean(as_bits(got) != as_bits(want)))


def as_bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_equal(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        i = np.argwhere(got != want)[0]
        raise AssertionError(f"{name}: {int((got != want).sum())} mismatches; first at {tuple(i)}: "
                             f"gpu={got[tuple(i)]} oracle={want[tuple(i)]}")
