"""GPU parity of the quantisation variants (arnfp8_run_fmt) against the CPU oracle.

e5m2 per-row output: scales within 1e-5 relative, codes within one e5m2 step.
MXFP8: the E8M0 block exponents equal the oracle's, except in blocks whose
largest magnitude lies within fp32 rounding of a power of two (there the
exponent is decided by an fp32 value whose last bits depend on the order of
the row's sum of squares: either neighbour is a correct result, and the codes
are then checked against the oracle's codes for the GPU's exponent); codes
within one e4m3fn step.  bf16 residual outputs bit-exact throughout.
"""
import numpy as np
import pytest
import torch

from tests._util import assert_bits_equal, assert_e5m2_close, assert_fp8_close, assert_scales_close, check_mx

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def arn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import all_reduce_rmsnorm_amd as arn

    arn.library()
    return arn


def _bits(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.bf16_bits(t)


def _case(seed, rows, cols, P, std=0.5):
    g = torch.Generator().manual_seed(seed)
    xs = [(torch.randn((rows, cols), generator=g) * std).to(torch.bfloat16) for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    return xs, res, gamma


@pytest.mark.parametrize("rows,cols,P", [(4, 256, 2), (32, 7168, 4), (37, 7176, 8), (3, 65536, 3)])
def test_e5m2_matches_oracle(arn, orc, rows, cols, P):
    print(f"[e5m2] rows={rows} cols={cols} P={P}", flush=True)
    xs, res, gamma = _case(rows + cols + P, rows, cols, P)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run_fmt([x.to(DEV) for x in xs], res.to(DEV), res_out, out, scales, gamma.to(DEV),
                       1e-6, 0.0, 1200.0, out_format=arn.FMT_E5M2)
    torch.cuda.synchronize()
    q, s, h = orc.arnfp8_e5m2([_bits(x) for x in xs], _bits(gamma), 1e-6, 0.0, 1200.0,
                              residual_in=_bits(res))
    assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    assert_e5m2_close(out.cpu().numpy(), q, min_exact=0.99 if rows * cols < 4096 else 0.999)


def test_e5m2_clamp_and_floor(arn, orc):
    xs, res, gamma = _case(5, 8, 1024, 2, std=1.0)
    xs[0][7] = 0.0
    xs[1][7] = 0.0
    out = torch.empty((8, 1024), dtype=torch.uint8, device=DEV)
    scales = torch.empty((8,), dtype=torch.float32, device=DEV)
    arn.arnfp8_run_fmt([x.to(DEV) for x in xs], None, None, out, scales, gamma.to(DEV), 1e-6, 0.0,
                       2.0, out_format=arn.FMT_E5M2)
    torch.cuda.synchronize()
    q, s, _ = orc.arnfp8_e5m2([_bits(x) for x in xs], _bits(gamma), 1e-6, 0.0, 2.0)
    sg = scales.cpu().numpy()
    assert np.all(sg[:7] == np.float32(2.0 / 57344.0)) and np.all(s[:7] == sg[:7])
    assert sg[7] == np.float32(1.0 / (57344.0 * 512.0)) == s[7]
    assert_e5m2_close(out.cpu().numpy(), q, min_exact=0.99)


@pytest.mark.parametrize("rows,cols,P", [(4, 256, 2), (32, 7168, 4), (37, 2880, 8), (128, 8192, 8),
                                         (2, 65536, 2)])
def test_mxfp8_matches_oracle(arn, orc, rows, cols, P):
    print(f"[mxfp8] rows={rows} cols={cols} P={P}", flush=True)
    xs, res, gamma = _case(3 * rows + cols + P, rows, cols, P)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    bscales = torch.full((rows, cols // 32), 0xFF, dtype=torch.uint8, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run_fmt([x.to(DEV) for x in xs], res.to(DEV), res_out, out, bscales, gamma.to(DEV),
                       1e-6, 0.0, 0.0, out_format=arn.FMT_MXFP8)
    torch.cuda.synchronize()
    check_mx(orc, xs, res, gamma, out, bscales, res_out)


def test_mxfp8_zero_and_wide_range_blocks(arn, orc):
    rows, cols = 3, 512
    xs, res, gamma = _case(77, rows, cols, 1, std=1.0)
    x = xs[0].float()
    x[0, :64] = 0.0                      # two all-zero blocks -> exponent -127
    x[1, 32:64] *= 1e-6                  # a tiny block next to normal ones
    x[2, :32] *= 1e4                     # a dominant block
    xs = [x.to(torch.bfloat16)]
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    bscales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    arn.arnfp8_run_fmt([xs[0].to(DEV)], None, None, out, bscales, gamma.to(DEV), 1e-6, 0.0, 0.0,
                       out_format=arn.FMT_MXFP8)
    torch.cuda.synchronize()
    b = bscales.cpu().numpy()
    assert b[0, 0] == 0 and b[0, 1] == 0
    assert np.all(out.cpu().numpy()[0, :64] & 0x7F == 0)
    check_mx(orc, xs, None, gamma, out, bscales, None)


def test_format_errors(arn):
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 48), dtype=torch.uint8, device=DEV)
    s = torch.empty((4, 2), dtype=torch.uint8, device=DEV)
    g = torch.ones((48,), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_run_fmt([x], None, None, out, s, g, 1e-6, 0.0, 1.0, out_format=arn.FMT_MXFP8)
    assert e.value.status == 3  # cols % 32 != 0
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_run_fmt([x], None, None, out, s, g, 1e-6, 0.0, 1.0, out_format=7)
    assert e.value.status == 9


@pytest.mark.parametrize("stores", [1, 2])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2", "mxfp8"])
def test_every_format_under_both_store_policies(arn, orc, fmt, stores):
    """Each output format with nt (1) and sc1 (2) row stores on a ragged shape."""
    rows, cols, P = 21, 7168 + 64 * 3, 4
    print(f"[{fmt}] stores={stores}", flush=True)
    xs, res, gamma = _case(11 * stores + len(fmt), rows, cols, P)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    code = {"e4m3fn": arn.FMT_E4M3FN, "e5m2": arn.FMT_E5M2, "mxfp8": arn.FMT_MXFP8}[fmt]
    if fmt == "mxfp8":
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    else:
        scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    arn.arnfp8_run_fmt([x.to(DEV) for x in xs], res.to(DEV), res_out, out, scales, gamma.to(DEV),
                       1e-6, 0.0, 1200.0, out_format=code, launch=dict(stores=stores))
    torch.cuda.synchronize()
    if fmt == "mxfp8":
        check_mx(orc, xs, res, gamma, out, scales, res_out)
        return
    fn = orc.arnfp8 if fmt == "e4m3fn" else orc.arnfp8_e5m2
    q, s, h = fn([_bits(x) for x in xs], _bits(gamma), 1e-6, 0.0, 1200.0, residual_in=_bits(res))
    assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    if fmt == "e4m3fn":
        assert_fp8_close(out.cpu().numpy(), q)
    else:
        assert_e5m2_close(out.cpu().numpy(), q)
