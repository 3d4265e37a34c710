"""Pins for the oracle's rank-order sum (CPU only).

What fixes the sum: each rank's bf16 value is widened exactly, the values are
added in fp32 in rank order 0..P-1, and the total is rounded to bf16 once
(b12x PR #283 "PCIeTwoShotBF16": PR description; Validation, "Precision").
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_to_f(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def f_to_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0] >> 16


def rand_bf16(rng, shape, std=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_f64(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()


# --- exact rounding by brute force (Fractions; no floating point at all) ----

def _nearest_even_fraction(q: Fraction, mbits: int) -> Fraction:
    """Round the rational q to the nearest binary float with `mbits` fraction
    bits (normal range only), ties to even, by explicit comparison."""
    if q == 0:
        return Fraction(0)
    sgn = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2); grid spacing 2^-mbits
    scaled = a * (2 ** mbits)
    lo = math.floor(scaled)
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sgn * Fraction(lo, 2 ** mbits) * Fraction(2) ** e


def brute_sum(vals_bits):
    acc = Fraction(bits_to_f(vals_bits[0]))
    for b in vals_bits[1:]:
        acc = _nearest_even_fraction(acc + Fraction(bits_to_f(b)), 23)  # fp32 add
    return _nearest_even_fraction(acc, 7)                                # bf16, once


def test_brute_force_tiny_inputs(orc):
    rng = np.random.default_rng(10)
    for P in range(1, 9):
        for rows, cols in [(1, 8), (2, 16), (3, 24), (4, 64)]:
            xs = [rand_bf16(rng, (rows, cols), std=float(rng.choice([0.01, 1.0, 300.0])))
                  for _ in range(P)]
            got = orc.sum_bf16(xs)
            for i in range(rows):
                for j in range(cols):
                    want = brute_sum([x[i, j] for x in xs])
                    g = bits_to_f(got[i, j])
                    if want == 0:
                        assert g == 0.0
                    else:
                        assert Fraction(g) == want, (P, i, j)


def test_identity_p1_bitwise_including_negative_zero(orc):
    rng = np.random.default_rng(11)
    x = rand_bf16(rng, (5, 48))
    x[0, 0] = 0x8000  # -0
    x[0, 1] = 0x0000  # +0
    x[1, 2] = 0x0001  # smallest subnormal
    x[1, 3] = 0x7F7F  # largest finite
    out = orc.sum_bf16([x])
    assert np.array_equal(out, x)


def test_one_hot_slabs_reproduce_the_value(orc):
    rng = np.random.default_rng(12)
    P, shape = 8, (6, 40)
    src = rand_bf16(rng, shape, std=50.0)
    owner = rng.integers(0, P, size=shape)
    xs = [np.where(owner == p, src, np.uint16(0)).astype(np.uint16) for p in range(P)]
    out = orc.sum_bf16(xs)
    assert np.array_equal(out, src)


def test_one_rounding_error_bound(orc):
    # |s - exact| <= half a bf16 ulp of s + (P-1) * 2^-24 * max |partial|.
    rng = np.random.default_rng(13)
    for P in (2, 4, 8):
        xs = [rand_bf16(rng, (64, 256), std=4.0) for _ in range(P)]
        f = [as_f64(x) for x in xs]
        exact = np.sum(f, axis=0)           # exact in fp64 for <= 8 such bf16 terms
        partial_max = np.max(np.abs(np.cumsum(f, axis=0)), axis=0)
        s = as_f64(orc.sum_bf16(xs))
        _, e = np.frexp(np.where(s == 0, 1.0, s))
        half_ulp = np.ldexp(1.0, e - 1 - 8)  # bf16: 8 significant bits
        bound = half_ulp + (P - 1) * 2.0 ** -24 * partial_max
        assert np.all(np.abs(s - exact) <= bound)


def test_golden_half_ulp_at_sixteen(orc):
    """The page's printed precision figure: 0.0625 max error at magnitude ~16,
    one bf16 half-ulp (b12x PR #283, Validation, "Precision")."""
    path = os.path.join(GOLDEN, "p3_half_ulp_at_16.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for r in rows:
        vals = [float(v) for v in r[:-2]]
        want_sum, want_err = float(r[-2]), float(r[-1])
        xs = [np.array([[f_to_bits(v)]], dtype=np.uint16) for v in vals]
        s = bits_to_f(orc.sum_bf16(xs)[0, 0])
        assert s == want_sum
        assert abs(s - sum(vals)) == want_err
        assert want_err <= 0.0625


def test_rank_order_matters_and_is_respected(orc):
    # (2^8 + 1) + (-2^8) in fp32 is exactly 1; summing -2^8 first gives the
    # same.  But with 2^24 scale, fp32 absorbs the small term: order decides.
    big, small = f_to_bits(2.0 ** 25), f_to_bits(1.0)
    neg = f_to_bits(-(2.0 ** 25))
    a = [np.array([[b]], dtype=np.uint16) for b in (big, small, neg)]
    b = [np.array([[x]], dtype=np.uint16) for x in (big, neg, small)]
    assert bits_to_f(orc.sum_bf16(a)[0, 0]) == 0.0   # 2^25 + 1 rounds back to 2^25
    assert bits_to_f(orc.sum_bf16(b)[0, 0]) == 1.0


def test_error_never_exceeds_per_hop_bf16_ring(orc):
    """The page claims the one-rounding sum's error never exceeds that of a
    ring that rounds to bf16 after every hop (b12x PR #283, Validation)."""
    rng = np.random.default_rng(14)
    P = 4
    xs = [rand_bf16(rng, (128, 512), std=4.0) for _ in range(P)]
    exact = np.sum([as_f64(x) for x in xs], axis=0)
    t = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) for x in xs]
    ring = t[0]
    for p in range(1, P):
        ring = ring + t[p]                   # bf16 + bf16 rounds to bf16 each hop
    err_ring = np.max(np.abs(ring.double().numpy() - exact))
    err_one = np.max(np.abs(as_f64(orc.sum_bf16(xs)) - exact))
    assert err_one <= err_ring
    assert err_one < err_ring  # strictly better on this workload


def test_bad_arguments_rejected(orc):
    x = np.zeros((2, 8), dtype=np.uint16)
    with pytest.raises((ValueError, AssertionError)):
        orc.sum_bf16([x] * 9)
