"""Shared helpers for the GPU parity tests: comparison rules and small runners.

Comparison rules (the parity bar):
  * bf16 outputs (sum, residual): bit-exact.
  * fp32 scales: relative difference <= 1e-5.
  * fp8 e4m3fn codes: within one step in the ordered code sequence
    (sign-magnitude mapped to a signed integer, +0 == -0); NaN codes never.
"""
from __future__ import annotations

import numpy as np

SCALE_RTOL = 1e-5
FP8_MAX_STEPS = 1


def ordered_fp8(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def assert_fp8_close(got: np.ndarray, want: np.ndarray, min_exact: float = 0.999, what="fp8"):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert not np.any((got & 0x7F) == 0x7F), f"{what}: NaN code in the output"
    d = np.abs(ordered_fp8(got) - ordered_fp8(want))
    worst = int(d.max()) if d.size else 0
    assert worst <= FP8_MAX_STEPS, f"{what}: {int((d > FP8_MAX_STEPS).sum())} codes off by more than one step (max {worst})"
    if d.size:
        exact = float((d == 0).mean())
        assert exact >= min_exact, f"{what}: only {exact:.6f} of codes match exactly"
    return d


def assert_scales_close(got: np.ndarray, want: np.ndarray, what="scales"):
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    want = np.asarray(want, dtype=np.float64).reshape(-1)
    rel = np.abs(got / want - 1.0)
    assert np.all(rel <= SCALE_RTOL), f"{what}: max relative error {rel.max():.3e}"
    return rel


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what="bf16"):
    assert got.shape == want.shape, (got.shape, want.shape)
    bad = got != want
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements differ (first at {np.argwhere(bad)[0].tolist()})"
