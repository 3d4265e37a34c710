"""Pins for the oracle's residual add, RMSNorm, per-row scale and fp8 quant (CPU only).

Closed forms and invariants the mathematics fixes, chosen so that a dropped
term (eps, the residual, the weight offset, the floor or the clamp of the
scale), a wrong index (gamma) or a wrong order (rounding before or after the
residual add) fails at least one of them.

Sources: Modular Mojo API docs "allreduce_rmsnorm_fp8" (function summary;
Args epsilon, weight_offset, scale_ub, scale_output); TensorRT-LLM PR #19836
(RESIDUAL_RMS_NORM epilogue); tt-metal rmsnorm_2d.py (add_unit_offset).
"""
import math
import struct

import numpy as np
import pytest
import torch

E4M3_MAX = 448.0
SCALE_FLOOR = struct.unpack("<f", struct.pack("<f", 1.0 / (448.0 * 512.0)))[0]


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf(x):
    """Exact bf16 bit pattern of a value that must be representable."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, x
    return b >> 16


def bf_arr(vals, shape=None):
    a = np.array([bf(v) for v in np.ravel(vals)], dtype=np.uint16)
    return a.reshape(shape if shape is not None else np.shape(vals))


def rand_bf16(rng, shape, std=1.0, mean=0.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std + mean).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_f64(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()


def e4m3_val(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def ones_gamma(cols):
    return bf_arr([1.0] * cols)


# ------------------------------------------------------------ closed forms --

@pytest.mark.parametrize("k", [1.0, -3.5, 0.015625, 200.0])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_constant_row(orc, k, eps):
    cols = 64
    x = bf_arr([[k] * cols])
    q, s, _ = orc.arnfp8([x], ones_gamma(cols), eps, 0.0, 1200.0)
    amax = f32(abs(k) / math.sqrt(k * k + f32(eps)))
    want_scale = max(f32(min(amax, 1200.0) / 448.0), SCALE_FLOOR)
    assert s[0] == np.float32(want_scale)
    vals = e4m3_val(q)
    if amax / 448.0 >= SCALE_FLOOR:
        assert np.all(vals == math.copysign(448.0, k))
    assert np.all(np.sign(vals) == math.copysign(1.0, k))


@pytest.mark.parametrize("cols", [16, 64, 100, 256])
def test_one_hot_row_pins_gamma_index(orc, cols):
    rng = np.random.default_rng(20)
    gamma = bf_arr([f32(v) for v in np.round(rng.uniform(0.5, 1.5, cols) * 64) / 64])
    g = as_f64(gamma)
    for j0 in (0, cols // 3, cols - 1):
        for a in (2.0, -0.75):
            row = [0.0] * cols
            row[j0] = a
            q, s, _ = orc.arnfp8([bf_arr([row])], gamma, 0.0, 0.0, 1200.0)
            # y_j0 = a * sqrt(cols) / |a| * g_j0, every other y_j = 0
            want_amax = f32(math.sqrt(cols) * g[j0])
            assert s[0] == np.float32(f32(want_amax / 448.0))
            vals = e4m3_val(q[0])
            assert vals[j0] == math.copysign(448.0, a)
            assert np.all(np.delete(vals, j0) == 0.0)


def test_two_value_row_exact_codes(orc):
    # h = (k, 2k, 0, 0), g = 1, eps = 0: y proportional to (1, 2) so the codes
    # are 224 and 448 exactly (224 = 1.75 * 2^7 is an e4m3fn value).
    for k in (1.0, 0.5, -6.0):
        x = bf_arr([[k, 2 * k, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]])
        q, s, _ = orc.arnfp8([x], ones_gamma(8), 0.0, 0.0, 1200.0)
        vals = e4m3_val(q[0])
        sg = math.copysign(1.0, k)
        assert list(vals) == [224.0 * sg, 448.0 * sg, 0, 0, 0, 0, 0, 0]
        # ms = 5 k^2 / 8, amax = 2 |k| / sqrt(5 k^2 / 8) = 2 sqrt(8/5)
        assert s[0] == np.float32(f32(f32(2 * math.sqrt(8 / 5)) / 448.0))


# ---------------------------------------------------------------- residual --

def test_residual_adds_the_rounded_sum(orc):
    # ranks: 1 and 2^-9 -> fp32 1 + 2^-9 -> bf16 1 (below the midpoint).
    # residual 2^-8: bf16(1 + 2^-8) = 1 (tie, even).  Adding the unrounded
    # fp32 sum instead would give bf16(1 + 3 * 2^-9) = 1 + 2^-7.
    cols = 8
    x0 = bf_arr([[1.0] * cols])
    x1 = bf_arr([[2.0 ** -9] * cols])
    res = bf_arr([[2.0 ** -8] * cols])
    _, _, rout = orc.arnfp8([x0, x1], ones_gamma(cols), 1e-6, 0.0, 1200.0, residual_in=res)
    assert np.all(rout == bf(1.0))
    # (1 + 2^-7) + 2^-8 is a tie between odd 1 + 2^-7 and even 1 + 2^-6
    x0 = bf_arr([[1.0 + 2.0 ** -7] * cols])
    _, _, rout = orc.arnfp8([x0], ones_gamma(cols), 1e-6, 0.0, 1200.0, residual_in=res)
    assert np.all(rout == bf(1.0 + 2.0 ** -6))


def test_zero_residual_is_inert(orc):
    rng = np.random.default_rng(21)
    xs = [rand_bf16(rng, (6, 128)) for _ in range(3)]
    gamma = rand_bf16(rng, (128,), 0.2, 1.0)
    zero = np.zeros((6, 128), dtype=np.uint16)
    q0, s0, r0 = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0)
    q1, s1, r1 = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=zero)
    # s + (+0) == s except that -0 + +0 = +0
    assert np.array_equal(np.where(r0 == 0x8000, 0, r0), r1)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_residual_out_is_the_norm_input(orc):
    # Norm of the emitted residual (P = 1, no residual) reproduces the output.
    rng = np.random.default_rng(22)
    xs = [rand_bf16(rng, (5, 96)) for _ in range(4)]
    res = rand_bf16(rng, (5, 96))
    gamma = rand_bf16(rng, (96,), 0.1, 1.0)
    q, s, h = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=res)
    q2, s2, _ = orc.arnfp8([h], gamma, 1e-6, 0.0, 1200.0)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # and h is the rounded (sum, then + residual)
    srd = orc.sum_bf16(xs)
    want = orc.sum_bf16([srd, res])
    assert np.array_equal(h, want)


# ------------------------------------------------------------- invariants --

def test_unit_gain_offset_equals_gamma_one(orc):
    rng = np.random.default_rng(23)
    xs = [rand_bf16(rng, (8, 256), 0.25) for _ in range(8)]
    res = rand_bf16(rng, (8, 256))
    a = orc.arnfp8(xs, bf_arr([0.0] * 256), 1e-5, 1.0, 1200.0, residual_in=res)
    b = orc.arnfp8(xs, bf_arr([1.0] * 256), 1e-5, 0.0, 1200.0, residual_in=res)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_weight_offset_is_added_to_gamma(orc):
    # gamma = 0.5 with offset 0.25 must equal gamma = 0.75 with offset 0.
    rng = np.random.default_rng(24)
    xs = [rand_bf16(rng, (4, 64))]
    a = orc.arnfp8(xs, bf_arr([0.5] * 32 + [2.0] * 32), 1e-6, 0.25, 1200.0)
    b = orc.arnfp8(xs, bf_arr([0.75] * 32 + [2.25] * 32), 1e-6, 0.0, 1200.0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("with_res", [False, True])
def test_scale_invariance_eps_zero(orc, with_res):
    # Doubling every slab (and the residual) doubles h exactly; with eps = 0,
    # r halves exactly, so y, amax, scale and q are unchanged.
    rng = np.random.default_rng(25)
    P = 4
    xs = [rand_bf16(rng, (10, 128)) for _ in range(P)]
    res = rand_bf16(rng, (10, 128)) if with_res else None
    gamma = rand_bf16(rng, (128,), 0.2, 1.0)
    dbl = lambda a: bf_arr(as_f64(a) * 2.0, a.shape)
    q0, s0, _ = orc.arnfp8(xs, gamma, 0.0, 0.0, 1200.0, residual_in=res)
    q1, s1, _ = orc.arnfp8([dbl(x) for x in xs], gamma, 0.0, 0.0, 1200.0,
                           residual_in=None if res is None else dbl(res))
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_eps_changes_the_result(orc):
    rng = np.random.default_rng(26)
    xs = [rand_bf16(rng, (4, 64), 0.01)]
    _, s0, _ = orc.arnfp8(xs, ones_gamma(64), 0.0, 0.0, 1200.0)
    _, s1, _ = orc.arnfp8(xs, ones_gamma(64), 1e-3, 0.0, 1200.0)
    assert np.all(s1 < s0)


def test_scale_clamps_exactly_at_ub(orc):
    rng = np.random.default_rng(27)
    cols = 512
    xs = [rand_bf16(rng, (16, cols), 0.5)]
    gamma = rand_bf16(rng, (cols,), 0.1, 1.0)
    ub = 3.0
    q, s, _ = orc.arnfp8(xs, gamma, 1e-6, 0.0, ub)
    y_max = []
    h = as_f64(xs[0])
    g = as_f64(gamma)
    for i in range(16):
        y = h[i] / math.sqrt(np.mean(h[i] ** 2) + f32(1e-6)) * g
        y_max.append(np.max(np.abs(y)))
    clamped = np.array(y_max) >= ub
    assert clamped.any() and (~clamped).any()
    assert np.all(s[clamped] == np.float32(f32(ub / 448.0)))
    # clamped rows saturate at +-448 wherever |y| / scale >= 448
    vals = e4m3_val(q)
    assert np.all(np.abs(vals[clamped]).max(axis=1) == 448.0)
    assert np.all(s[~clamped] < np.float32(f32(ub / 448.0)))


def test_zero_rows_take_the_floor_scale(orc):
    x = np.zeros((3, 32), dtype=np.uint16)
    q, s, _ = orc.arnfp8([x, x], ones_gamma(32), 1e-6, 0.0, 1200.0)
    assert np.all(s == np.float32(SCALE_FLOOR))
    assert np.all(e4m3_val(q) == 0.0)


def test_tiny_rows_floor_scale_and_subnormal_codes(orc):
    # |h| constant and tiny with large eps: amax = |k| / sqrt(k^2 + eps) is
    # below 1/512, so the scale is the floor and q = y / floor < 448.
    k = 2.0 ** -12
    eps = 1.0
    x = bf_arr([[k] * 16])
    q, s, _ = orc.arnfp8([x], ones_gamma(16), eps, 0.0, 1200.0)
    assert s[0] == np.float32(SCALE_FLOOR)
    y = k / math.sqrt(k * k + f32(eps))
    vals = e4m3_val(q[0])
    assert np.all(np.abs(vals - y / SCALE_FLOOR) <= 0.5 * 2.0 ** (math.floor(math.log2(y / SCALE_FLOOR)) - 3))


def test_full_range_rows_reach_448(orc):
    rng = np.random.default_rng(28)
    xs = [rand_bf16(rng, (20, 300), 1.0) for _ in range(3)]
    q, s, _ = orc.arnfp8(xs, rand_bf16(rng, (300,), 0.2, 1.0), 1e-6, 0.0, 1200.0)
    assert np.all(np.abs(e4m3_val(q)).max(axis=1) == 448.0)
    assert np.all(s > SCALE_FLOOR)


def test_dequantised_within_half_ulp_of_normalised_row(orc):
    rng = np.random.default_rng(29)
    cols = 384
    xs = [rand_bf16(rng, (12, cols), 0.5) for _ in range(4)]
    res = rand_bf16(rng, (12, cols))
    gamma = rand_bf16(rng, (cols,), 0.1, 1.0)
    q, s, h = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=res)
    hv = as_f64(h)
    g = as_f64(gamma)
    vals = e4m3_val(q)
    for i in range(12):
        y = hv[i] / math.sqrt(np.mean(hv[i] ** 2) + f32(1e-6)) * g
        v = y / float(s[i])
        av = np.abs(v)
        # half a quantum of e4m3fn at each magnitude (subnormal quantum 2^-9),
        # plus fp32 slack for the decision value
        e = np.floor(np.log2(np.maximum(av, 2.0 ** -6)))
        half_q = 0.5 * np.exp2(e - 3)
        assert np.all(np.abs(vals[i] - v) <= half_q * (1 + 1e-6) + 1e-6 * av)


def test_library_fp8_conversion_agrees_on_decision_values(orc):
    # The decision value v = fl32(y / scale) converted by PyTorch's CPU
    # e4m3fn conversion gives the oracle's codes.
    rng = np.random.default_rng(30)
    cols = 256
    xs = [rand_bf16(rng, (16, cols)) for _ in range(2)]
    gamma = rand_bf16(rng, (cols,), 0.2, 1.0)
    q, s, h = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0)
    hv, g = as_f64(h), as_f64(gamma)
    mism = 0
    for i in range(16):
        y = hv[i] * (1.0 / math.sqrt(np.sum(hv[i] * hv[i]) / cols + f32(1e-6))) * g
        v = np.clip((y / float(s[i])).astype(np.float32), -448, 448)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        mism += int(np.sum(ref != q[i]))
    assert mism == 0


# ------------------------------------------------ eps = 0 and bad scalars --

@pytest.mark.parametrize("with_res", [False, True])
def test_eps_zero_all_zero_row_takes_floor_and_zero_codes(orc, with_res):
    # The Mojo docs put no lower bound on epsilon.  With eps = 0 an all-zero
    # row has mean(h^2) + eps = 0: the reading is y = 0, so the scale is the
    # floor and every code is a zero (never the NaN code 0x7F / 0xFF).
    # Row 1 mixes -0 and +0 (h keeps its sign, so codes may be +0 or -0);
    # row 2 is an ordinary row next to them, which must be unaffected.
    cols = 64
    x = np.zeros((3, cols), dtype=np.uint16)
    x[1, ::2] = 0x8000  # -0.0
    x[2] = bf_arr([[1.0, -2.0] * (cols // 2)])[0]
    res = np.zeros((3, cols), dtype=np.uint16) if with_res else None
    q, s, h = orc.arnfp8([x], ones_gamma(cols), 0.0, 0.0, 1200.0, residual_in=res)
    assert np.all(s[:2] == np.float32(SCALE_FLOOR))
    assert not np.any((q & 0x7F) == 0x7F)
    assert np.all((q[:2] & 0x7F) == 0)
    # row 2: ms = 2.5, y = (1, -2) / sqrt(2.5): codes 224 and -448 exactly
    vals = e4m3_val(q[2])
    assert np.all(vals[0::2] == 224.0) and np.all(vals[1::2] == -448.0)
    assert s[2] == np.float32(f32(f32(2.0 / math.sqrt(2.5)) / 448.0))


def test_eps_zero_tiny_row_still_normalises(orc):
    # Only mean + eps == 0 takes the zero branch: a row of tiny (subnormal
    # bf16) values with eps = 0 still normalises to unit RMS.
    cols = 32
    k = 2.0 ** -130  # a bf16 subnormal; k^2 is exact in fp64
    x = bf_arr([[k] * cols])
    q, s, _ = orc.arnfp8([x], ones_gamma(cols), 0.0, 0.0, 1200.0)
    assert s[0] == np.float32(f32(1.0 / 448.0))
    assert np.all(e4m3_val(q) == 448.0)


@pytest.mark.parametrize("eps,woff,ub", [(-1e-6, 0.0, 1.0), (float("nan"), 0.0, 1.0),
                                         (float("inf"), 0.0, 1.0), (1e-6, float("nan"), 1.0),
                                         (1e-6, float("inf"), 1.0), (1e-6, 0.0, 0.0),
                                         (1e-6, 0.0, -2.0), (1e-6, 0.0, float("nan"))])
def test_bad_scalars_are_rejected(orc, eps, woff, ub):
    x = bf_arr([[1.0] * 16])
    with pytest.raises(ValueError):
        orc.arnfp8([x], ones_gamma(16), eps, woff, ub)
    with pytest.raises(ValueError):
        orc.arnfp8_e5m2([x], ones_gamma(16), eps, woff, ub)


def test_infinite_scale_ub_means_no_bound(orc):
    rng = np.random.default_rng(31)
    xs = [rand_bf16(rng, (6, 128), 4.0)]
    gamma = rand_bf16(rng, (128,), 0.2, 1.0)
    a = orc.arnfp8(xs, gamma, 1e-6, 0.0, float("inf"))
    b = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1e30)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
