"""The kernels' conversion step on gfx950 against the oracle's codecs, bit for bit.

Checks that the hardware conversions the fused kernel relies on are the OCP
formats (e4m3fn: bias 7, max 448; e5m2: bias 15, max 57344) with round to
nearest even, and that the packed bf16 conversion rounds to nearest even:
every code's value, every midpoint between neighbouring codes and the fp32
values either side of it, subnormals, out-of-range values (clamped), and
random values.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def arn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import all_reduce_rmsnorm_amd as arn

    arn.library()
    return arn


def _probe_values(decode, vmax, rng):
    vals = sorted(set(v for v in (decode(c) for c in range(256)) if math.isfinite(v)))
    xs = []
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2.0)
        xs += [a, m, np.nextafter(m, np.float32(np.inf)), np.nextafter(m, np.float32(-np.inf))]
    xs += list(rng.uniform(-vmax, vmax, 50000)) + list(rng.standard_normal(50000) * vmax * 1e-3)
    xs += [vmax * 1.01, -vmax * 1.5, 1e30, -1e30, 0.0, -0.0]
    x = np.array(xs, dtype=np.float32)
    pad = (-len(x)) % 8
    return np.concatenate([x, np.zeros(pad, np.float32)])


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_conversion_is_ocp_rne(arn, orc, fmt):
    rng = np.random.default_rng(60)
    if fmt == "e4m3fn":
        dec, enc, vmax, code = orc.e4m3fn_to_f64, orc.f32_to_e4m3fn_sat, 448.0, arn.FMT_E4M3FN
    else:
        dec, enc, vmax, code = orc.e5m2_to_f64, orc.f32_to_e5m2_sat, 57344.0, arn.FMT_E5M2
    x = _probe_values(dec, vmax, rng)
    want = np.array([enc(float(v)) for v in x], dtype=np.uint8)
    out = torch.empty(len(x), dtype=torch.uint8, device=DEV)
    arn.arnfp8_convert_f32(torch.from_numpy(x).to(DEV), out, code)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"{fmt}: {len(bad)} of {len(x)} differ, e.g. {x[bad[:5]]} -> {got[bad[:5]]} vs {want[bad[:5]]}"


def test_bf16_conversion_is_rne(arn, orc):
    rng = np.random.default_rng(61)
    bits = rng.integers(0, 2**32, 120000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    ties = ((rng.integers(0x0080, 0x7F7F, 8000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([v, ties, -ties, np.array([0.0, -0.0], np.float32)]).astype(np.float32)
    x = x[: len(x) - len(x) % 8]
    want = np.array([orc.f32_to_bf16(float(f)) for f in x], dtype=np.uint16)
    out = torch.empty(len(x), dtype=torch.int16, device=DEV)
    arn.arnfp8_convert_f32(torch.from_numpy(x).to(DEV), out, arn.CVT_BF16)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_convert_rejects_bad_arguments(arn):
    x = torch.zeros(16, dtype=torch.float32, device=DEV)
    o = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_convert_f32(x, o, arn.FMT_MXFP8)
    assert e.value.status == 9
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_convert_f32(x, o, arn.FMT_E4M3FN, n=12)
    assert e.value.status == 3
