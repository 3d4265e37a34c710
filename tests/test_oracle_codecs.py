"""Pins for the oracle's number-format codecs (CPU only).

Each codec is checked two independent ways: against PyTorch's CPU conversions
(a library routine), and against a brute-force nearest-value search over the
sorted list of every finite value of the format, written here from the
definition of round-to-nearest, ties-to-even.
"""
import bisect
import math
import struct

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def f32(x: float) -> float:
    """Round a Python float to the nearest fp32 (library: struct)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_from_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


# ---------------------------------------------------------------- bf16 ----

def test_bf16_decode_all_patterns_match_torch(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([orc.bf16_to_f32(int(b)) for b in pats], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _bf16_finite_sorted():
    vals = set()
    for b in range(65536):
        e = (b >> 7) & 0xFF
        if e == 0xFF:
            continue
        vals.add(struct.unpack("<f", struct.pack("<I", b << 16))[0])
    return sorted(vals)


BF16_SORTED = None


def bf16_nearest_even(x: float) -> float:
    """Brute force: the nearest finite bf16 to x, ties to the even mantissa."""
    global BF16_SORTED
    if BF16_SORTED is None:
        BF16_SORTED = _bf16_finite_sorted()
    s = BF16_SORTED
    i = bisect.bisect_left(s, x)
    cands = [s[k] for k in (i - 1, i) if 0 <= k < len(s)]
    best = min(abs(c - x) for c in cands)
    ties = [c for c in cands if abs(c - x) == best]
    if len(ties) == 1:
        return ties[0]
    even = [c for c in ties if ((struct.unpack("<I", struct.pack("<f", c))[0] >> 16) & 1) == 0]
    assert len(even) == 1
    return even[0]


def test_bf16_encode_matches_torch_on_random_bits(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=60000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_encode_brute_force_nearest_and_ties(orc):
    rng = np.random.default_rng(2)
    xs = []
    # random fp32 in a few binades, plus exact midpoints between bf16 neighbours
    for _ in range(3000):
        xs.append(f32(float(rng.standard_normal()) * 10.0 ** rng.integers(-6, 6)))
    for b in rng.integers(0x0080, 0x7F7F, size=2000):
        lo = f32_from_bits(int(b) << 16)
        hi = f32_from_bits((int(b) + 1) << 16)
        mid = (lo + hi) / 2.0                # exact in fp32: 9 significant bits
        assert f32(mid) == mid
        xs += [mid, -mid, f32(math.nextafter(mid, math.inf)), f32(math.nextafter(mid, -math.inf))]
    for x in xs:
        got = struct.unpack("<f", struct.pack("<I", orc.f32_to_bf16(x) << 16))[0]
        assert got == bf16_nearest_even(x), x


def test_bf16_encode_special_values(orc):
    assert orc.f32_to_bf16(0.0) == 0x0000
    assert orc.f32_to_bf16(-0.0) == 0x8000
    assert orc.f32_to_bf16(math.inf) == 0x7F80
    assert orc.f32_to_bf16(-math.inf) == 0xFF80
    nan = orc.f32_to_bf16(math.nan)
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
    # the largest fp32 rounds up past the largest bf16 -> inf
    assert orc.f32_to_bf16(f32_from_bits(0x7F7FFFFF)) == 0x7F80
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1
    assert orc.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is the midpoint of 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert orc.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82


# --------------------------------------------------------- e4m3fn / e5m2 ----

def _fp8_table(decode):
    return [decode(c) for c in range(256)]


def _finite_sorted(table):
    return sorted(set(v for v in table if math.isfinite(v)))


def fp8_nearest_even(x: float, table) -> float:
    """Brute force over every finite code of the format: the nearest value,
    ties to the code with an even (zero) mantissa LSB; saturating."""
    finite = [(v, c) for c, v in enumerate(table) if math.isfinite(v)]
    vmax = max(v for v, _ in finite)
    if x >= vmax:
        return vmax
    if x <= -vmax:
        return -vmax
    best = min(abs(v - x) for v, _ in finite)
    ties = [(v, c) for v, c in finite if abs(v - x) == best]
    vals = set(v for v, _ in ties)
    if len(vals) == 1:
        return ties[0][0]
    even = set(v for v, c in ties if (c & 1) == 0)
    assert len(even) == 1, (x, ties)
    return even.pop()


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_decode_all_codes_match_torch(orc, fmt):
    dec = orc.e4m3fn_to_f64 if fmt == "e4m3fn" else orc.e5m2_to_f64
    tdt = torch.float8_e4m3fn if fmt == "e4m3fn" else torch.float8_e5m2
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(tdt).to(torch.float64).numpy()
    got = np.array(_fp8_table(dec))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_closed_form_landmarks(orc):
    assert orc.e4m3fn_to_f64(0x7E) == 448.0          # 1.75 * 2^8, largest finite
    assert orc.e4m3fn_to_f64(0x08) == 2.0 ** -6      # smallest normal
    assert orc.e4m3fn_to_f64(0x01) == 2.0 ** -9      # smallest subnormal
    assert orc.e4m3fn_to_f64(0x38) == 1.0
    assert orc.e4m3fn_to_f64(0xB8) == -1.0
    assert math.isnan(orc.e4m3fn_to_f64(0x7F)) and math.isnan(orc.e4m3fn_to_f64(0xFF))
    assert orc.e5m2_to_f64(0x7B) == 57344.0
    assert orc.e5m2_to_f64(0x7C) == math.inf
    assert orc.e5m2_to_f64(0x01) == 2.0 ** -16


def _fp8_probe_values(table, rng, n_random):
    fin = _finite_sorted(table)
    xs = []
    for a, b in zip(fin[:-1], fin[1:]):
        m = (a + b) / 2.0
        xs += [m, f32(math.nextafter(f32(m), math.inf)), f32(math.nextafter(f32(m), -math.inf)), a]
    xs += [f32(v) for v in rng.uniform(-fin[-1] * 1.2, fin[-1] * 1.2, size=n_random)]
    xs += [f32(v) for v in rng.standard_normal(n_random) * 0.01]
    return [f32(x) for x in xs]


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_encode_brute_force_nearest_even_saturating(orc, fmt):
    dec = orc.e4m3fn_to_f64 if fmt == "e4m3fn" else orc.e5m2_to_f64
    enc = orc.f32_to_e4m3fn_sat if fmt == "e4m3fn" else orc.f32_to_e5m2_sat
    table = _fp8_table(dec)
    rng = np.random.default_rng(3)
    for x in _fp8_probe_values(table, rng, 3000):
        code = enc(x)
        want = fp8_nearest_even(x, table)
        assert table[code] == want, (fmt, x, hex(code))
        if want == 0.0:
            assert (code & 0x80) == (0x80 if math.copysign(1.0, x) < 0 else 0)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_encode_matches_torch_in_range(orc, fmt):
    enc = orc.f32_to_e4m3fn_sat if fmt == "e4m3fn" else orc.f32_to_e5m2_sat
    tdt = torch.float8_e4m3fn if fmt == "e4m3fn" else torch.float8_e5m2
    vmax = 448.0 if fmt == "e4m3fn" else 57344.0
    rng = np.random.default_rng(4)
    vals = np.concatenate([rng.uniform(-vmax, vmax, 20000),
                           rng.standard_normal(20000) * 0.05]).astype(np.float32)
    ref = torch.from_numpy(vals).to(tdt).view(torch.uint8).numpy()
    got = np.array([enc(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_fp8_encode_saturates_and_nan(orc):
    assert orc.f32_to_e4m3fn_sat(1e30) == 0x7E
    assert orc.f32_to_e4m3fn_sat(-1e30) == 0xFE
    assert orc.f32_to_e4m3fn_sat(math.inf) == 0x7E
    assert orc.f32_to_e4m3fn_sat(464.0) == 0x7E      # would round to 480 (NaN code) unsaturated
    assert orc.f32_to_e4m3fn_sat(math.nan) == 0x7F
    assert orc.f32_to_e5m2_sat(1e30) == 0x7B
    assert orc.f32_to_e5m2_sat(-math.inf) == 0xFB
