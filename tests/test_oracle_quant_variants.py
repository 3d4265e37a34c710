"""Pins for the oracle's quantisation variants (CPU only): e5m2 per-row output
and MXFP8 block scaling.

Sources: Huawei CANN aclnnAlltoAllQuantMatmul (x1QuantDtype: E5M2 or E4M3FN
for per-token dynamic quantisation; the mx-quantisation scale shape
(BS, ceil(H/64), 2)); the MX block rule is OCP Microscaling v1.0 (MXFP8,
E4M3 elements, E8M0 scale per 32 values).
"""
import math
import struct

import numpy as np
import pytest
import torch

E5M2_MAX = 57344.0


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf(x):
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, x
    return b >> 16


def bf_arr(vals):
    return np.array([bf(v) for v in np.ravel(vals)], dtype=np.uint16).reshape(np.shape(vals))


def rand_bf16(rng, shape, std=1.0, mean=0.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std + mean).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_f64(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()


def e5m2_val(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e5m2).double().numpy()


def e4m3_val(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


# ------------------------------------------------------------------ e5m2 ----

@pytest.mark.parametrize("k", [1.0, -3.5, 200.0])
def test_e5m2_constant_row(orc, k):
    cols = 64
    x = bf_arr([[k] * cols])
    q, s, _ = orc.arnfp8_e5m2([x], bf_arr([1.0] * cols), 1e-6, 0.0, 1e9)
    amax = f32(abs(k) / math.sqrt(k * k + f32(1e-6)))
    assert s[0] == np.float32(f32(amax / E5M2_MAX))
    assert np.all(e5m2_val(q) == math.copysign(E5M2_MAX, k))


def test_e5m2_clamp_floor_and_unit_gain(orc):
    rng = np.random.default_rng(50)
    xs = [rand_bf16(rng, (8, 256)) for _ in range(3)]
    q, s, _ = orc.arnfp8_e5m2(xs, bf_arr([1.0] * 256), 1e-6, 0.0, 1.5)
    assert np.all(s == np.float32(f32(1.5 / E5M2_MAX)))
    z = np.zeros((2, 64), dtype=np.uint16)
    _, s0, _ = orc.arnfp8_e5m2([z], bf_arr([1.0] * 64), 1e-6, 0.0, 1200.0)
    assert np.all(s0 == np.float32(f32(1.0 / (E5M2_MAX * 512.0))))
    a = orc.arnfp8_e5m2(xs, bf_arr([0.0] * 256), 1e-5, 1.0, 1200.0)
    b = orc.arnfp8_e5m2(xs, bf_arr([1.0] * 256), 1e-5, 0.0, 1200.0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_e5m2_dequantised_within_half_step_and_matches_library(orc):
    rng = np.random.default_rng(51)
    cols = 320
    xs = [rand_bf16(rng, (10, cols), 0.5) for _ in range(4)]
    res = rand_bf16(rng, (10, cols))
    gamma = rand_bf16(rng, (cols,), 0.1, 1.0)
    q, s, h = orc.arnfp8_e5m2(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=res)
    y = orc.norm_rows(xs, gamma, 1e-6, 0.0, residual_in=res)
    vals = e5m2_val(q)
    for i in range(10):
        v = y[i] / float(s[i])
        e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
        assert np.all(np.abs(vals[i] - v) <= 0.5 * np.exp2(e - 2) * (1 + 1e-6) + 1e-6 * np.abs(v))
        lib = torch.from_numpy(np.clip((v).astype(np.float32), -E5M2_MAX, E5M2_MAX)).to(
            torch.float8_e5m2).view(torch.uint8).numpy()
        assert np.array_equal(lib, q[i])
    # the residual and the e4m3 path see the same h
    _, _, h4 = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=res)
    assert np.array_equal(h, h4)


# -------------------------------------------------------------------- MX ----

def test_mx_shared_exponent_definition(orc):
    rng = np.random.default_rng(52)
    for _ in range(2000):
        v = rng.standard_normal(32) * 10.0 ** rng.integers(-8, 8)
        e = orc.mx_shared_exp(v)
        amax = np.max(np.abs(v))
        # 2^(e+8) <= amax < 2^(e+9)
        assert 2.0 ** (e + 8) <= amax < 2.0 ** (e + 9)
    assert orc.mx_shared_exp(np.zeros(32)) == -127
    assert orc.mx_shared_exp(np.full(32, 1.0)) == -8
    assert orc.mx_shared_exp(np.full(32, 448.0)) == 0
    assert orc.mx_shared_exp(np.full(32, 2.0 ** -140)) == -127  # clamped at the E8M0 floor
    assert orc.mx_shared_exp(np.full(32, 2.0 ** 200)) == 127


def test_mx_block_codes_match_library(orc):
    rng = np.random.default_rng(53)
    for _ in range(300):
        v = rng.standard_normal(32) * 10.0 ** rng.integers(-3, 3)
        e = orc.mx_shared_exp(v)
        codes = orc.mx_quantize_block(v, e)
        scaled = np.clip(np.ldexp(v, -e).astype(np.float32), -448, 448)
        lib = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, lib)


def test_mx_block_landmarks(orc):
    v = np.zeros(32)
    v[0], v[1], v[2] = 1.0, -0.5, 1.9
    e = orc.mx_shared_exp(v)
    assert e == -8
    vals = e4m3_val(orc.mx_quantize_block(v, e))
    assert vals[0] == 256.0 and vals[1] == -128.0
    assert vals[2] == 448.0            # 1.9 * 256 = 486.4 saturates
    assert np.all(vals[3:] == 0.0)


def test_mx_fused_is_norm_then_blocks(orc):
    rng = np.random.default_rng(54)
    cols = 256
    xs = [rand_bf16(rng, (6, cols)) for _ in range(3)]
    res = rand_bf16(rng, (6, cols))
    gamma = rand_bf16(rng, (cols,), 0.1, 1.0)
    q, bs, h = orc.arnfp8_mx(xs, gamma, 1e-6, 0.0, residual_in=res)
    assert bs.shape == (6, cols // 32)
    y = orc.norm_rows(xs, gamma, 1e-6, 0.0, residual_in=res)
    for i in range(6):
        for b in range(cols // 32):
            blk = y[i, 32 * b: 32 * b + 32]
            e = int(bs[i, b]) - 127
            assert 2.0 ** (e + 8) <= np.max(np.abs(blk)) < 2.0 ** (e + 9)
            codes = q[i, 32 * b: 32 * b + 32]
            # dequantised within half an E4M3 step of y (no element saturates
            # unless the block maximum lies in [448, 512) * 2^e)
            deq = e4m3_val(codes) * 2.0 ** e
            mag = np.abs(blk) * 2.0 ** -e
            step = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3) * 2.0 ** e
            sat = mag >= 448.0
            assert np.all(np.abs(deq - blk)[~sat] <= 0.5 * step[~sat] * (1 + 1e-6))
            assert np.all(np.abs(e4m3_val(codes)[sat]) == 448.0)
    _, _, h4 = orc.arnfp8(xs, gamma, 1e-6, 0.0, 1200.0, residual_in=res)
    assert np.array_equal(h, h4)


def test_norm_rows_closed_form(orc):
    # one-hot row, eps = 0: y_j0 = sqrt(cols) * g_j0, zero elsewhere
    cols = 64
    row = [0.0] * cols
    row[5] = -3.0
    gamma = bf_arr([1.0] * 5 + [1.5] + [1.0] * (cols - 6))
    y = orc.norm_rows([bf_arr([row])], gamma, 0.0, 0.0)
    assert y[0, 5] == pytest.approx(-math.sqrt(cols) * 1.5, rel=1e-15)
    assert np.all(np.delete(y[0], 5) == 0.0)


def test_eps_zero_all_zero_rows_e5m2_and_mx(orc):
    # eps = 0 on an all-zero row gives y = 0: e5m2 takes the floor scale and
    # zero codes, MX takes the smallest E8M0 scale (-127) and zero codes; an
    # ordinary row beside them is unaffected.
    cols = 64
    x = np.zeros((2, cols), dtype=np.uint16)
    x[1] = bf_arr([1.0, -2.0] * (cols // 2))
    gamma = bf_arr([1.0] * cols)
    q, s, _ = orc.arnfp8_e5m2([x], gamma, 0.0, 0.0, 1200.0)
    assert s[0] == np.float32(f32(1.0 / (E5M2_MAX * 512.0)))
    assert np.all((q[0] & 0x7F) == 0)
    assert not np.any((q & 0x7C) == 0x7C)
    assert np.all(e5m2_val(q[1])[1::2] == -E5M2_MAX)
    qm, bs, _ = orc.arnfp8_mx([x], gamma, 0.0, 0.0)
    assert np.all(bs[0] == 0) and np.all((qm[0] & 0x7F) == 0)
    # row 1: max |y| = 2 / sqrt(2.5) = 1.26..., floor(log2) = 0, e = -8
    assert np.all(bs[1] == 127 - 8)
    assert not np.any((qm & 0x7F) == 0x7F)


@pytest.mark.parametrize("eps,woff", [(-1.0, 0.0), (float("nan"), 0.0), (1e-6, float("inf"))])
def test_mx_bad_scalars_are_rejected(orc, eps, woff):
    x = bf_arr([[1.0] * 32])
    with pytest.raises(ValueError):
        orc.arnfp8_mx([x], bf_arr([1.0] * 32), eps, woff)
