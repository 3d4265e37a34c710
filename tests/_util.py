"""Shared helpers for the GPU parity tests: comparison rules and small runners.

Comparison rules (the parity bar):
  * bf16 outputs (sum, residual): bit-exact.
  * fp32 scales: relative difference <= 1e-5.
  * fp8 e4m3fn codes: within one step in the ordered code sequence
    (sign-magnitude mapped to a signed integer, +0 == -0); NaN codes never.
  * e5m2 codes: the same, with no inf or NaN code.
  * MXFP8: see ``check_mx``.
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


def _bf16_bits(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.bf16_bits(t)


def assert_e5m2_close(got, want, min_exact=0.999):
    assert not np.any((got & 0x7C) == 0x7C), "e5m2: inf or NaN code in the output"
    d = np.abs(ordered_fp8(got) - ordered_fp8(want))
    assert int(d.max()) <= 1, f"e5m2: {int((d > 1).sum())} codes off by more than one step"
    assert float((d == 0).mean()) >= min_exact


def oracle_rows(fn, xs, gamma, *scalars, residual_in=None, block=128, threads=None):
    """``fn(xs, gamma, *scalars, residual_in=...)`` (an oracle entry point over
    host bit arrays) evaluated on blocks of rows by a thread pool and stitched
    back together: the same result as one call over every row (rows are
    independent), in a fraction of the time.  The oracle's C calls run without
    the interpreter lock."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    rows = xs[0].shape[0]
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    spans = [(r0, min(rows, r0 + block)) for r0 in range(0, rows, block)]

    def one(span):
        r0, r1 = span
        return fn([x[r0:r1] for x in xs], gamma, *scalars,
                  residual_in=None if residual_in is None else residual_in[r0:r1])

    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(one, spans))
    return tuple(None if parts[0][k] is None else np.concatenate([p[k] for p in parts])
                 for k in range(len(parts[0])))


def check_mx(orc, xs, res, gamma, out, bscales, res_out, eps=1e-6, woff=0.0, min_exact=None,
             ref=None):
    """MXFP8 outputs against the oracle: E8M0 exponents equal except in blocks
    whose largest magnitude lies within fp32 rounding of a power of two (either
    neighbour is then correct, and the codes are checked for the GPU's
    exponent); codes within one e4m3fn step.  ``xs``, ``res`` and ``gamma``
    are tensors or host bit arrays; ``ref`` is the oracle's (codes, block
    scales, residual) when already computed."""
    as_bits = lambda t: t if isinstance(t, np.ndarray) else _bf16_bits(t)
    xs_b = [as_bits(x) for x in xs]
    res_b = None if res is None else as_bits(res)
    g_b = as_bits(gamma)
    if ref is None:
        ref = orc.arnfp8_mx(xs_b, g_b, eps, woff, residual_in=res_b)
    q, bs, h = ref
    if res_out is not None:
        assert_bits_equal(res_out if isinstance(res_out, np.ndarray) else _bf16_bits(res_out), h,
                          "residual_out")
    got_q = out if isinstance(out, np.ndarray) else out.cpu().numpy()
    got_b = bscales if isinstance(bscales, np.ndarray) else bscales.cpu().numpy()
    rows, cols = got_q.shape
    mism = np.argwhere(got_b != bs)
    if len(mism):
        q = q.copy()
        bad_rows = np.unique(mism[:, 0])
        y_rows = orc.norm_rows([x[bad_rows] for x in xs_b], g_b, eps, woff,
                               residual_in=None if res_b is None else res_b[bad_rows])
        y_of = {int(r): y_rows[k] for k, r in enumerate(bad_rows)}
        for i, b in mism:
            blk = y_of[int(i)][32 * b: 32 * b + 32]
            amax = np.max(np.abs(blk))
            frac = amax / 2.0 ** np.floor(np.log2(amax)) if amax > 0 else 1.5
            near_pow2 = min(frac - 1.0, 2.0 - frac) < 2.0 ** -20
            assert near_pow2 and abs(int(got_b[i, b]) - int(bs[i, b])) == 1, (
                f"block ({i},{b}): exponent {int(got_b[i, b]) - 127} vs oracle {int(bs[i, b]) - 127}, "
                f"amax {amax!r}")
            q[i, 32 * b: 32 * b + 32] = orc.mx_quantize_block(blk, int(got_b[i, b]) - 127)
    assert len(mism) <= max(1, got_b.size // 10000)
    if min_exact is None:
        min_exact = 0.99 if rows * cols < 4096 else 0.999
    assert_fp8_close(got_q, q, min_exact=min_exact, what="mxfp8")
