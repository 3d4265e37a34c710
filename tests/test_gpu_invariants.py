"""Device-side invariants and the eps = 0 cases, each also against the oracle.

* eps = 0 on all-zero rows (+0 and -0): the floor scale and zero codes in
  every output format, never a NaN code (the Mojo docs "allreduce_rmsnorm_fp8",
  Args, put no lower bound on epsilon); ordinary and tiny (normal-range) rows
  beside them are unaffected.
* One-hot slabs (every element nonzero on exactly one rank, +0 elsewhere):
  the rank-order sum reproduces the gathered input bit for bit (b12x PR #283,
  PR description: one rounding of the exact sum).
* Scale invariance with eps = 0: doubling every slab and the residual doubles
  the bf16 residual exactly and leaves the scales and codes unchanged, within
  the parity tolerance (RMSNorm's output does not depend on the input's
  scale when eps = 0).
"""
import numpy as np
import pytest
import torch

from tests._util import (assert_bits_equal, assert_e5m2_close, assert_fp8_close,
                         assert_scales_close, check_mx, ordered_fp8)

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


def _run(arn, fmt, xs, res, gamma, eps, woff, ub, in_place=False):
    rows, cols = xs[0].shape
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    if fmt == "mxfp8":
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    else:
        scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_d = None if res is None else res.to(DEV)
    res_out = res_d if (in_place and res_d is not None) else torch.empty(
        (rows, cols), dtype=torch.bfloat16, device=DEV)
    code = {"e4m3fn": arn.FMT_E4M3FN, "e5m2": arn.FMT_E5M2, "mxfp8": arn.FMT_MXFP8}[fmt]
    arn.arnfp8_run_fmt([x.to(DEV) for x in xs], res_d, res_out, out, scales, gamma.to(DEV), eps,
                       woff, ub, out_format=code)
    torch.cuda.synchronize()
    return out, scales, res_out


def _check(orc, fmt, xs, res, gamma, eps, woff, ub, out, scales, res_out, min_exact=0.99):
    if fmt == "mxfp8":
        check_mx(orc, xs, res, gamma, out, scales, res_out, eps=eps, woff=woff,
                 min_exact=min_exact)
        return None
    fn = orc.arnfp8 if fmt == "e4m3fn" else orc.arnfp8_e5m2
    q, s, h = fn([_bits(x) for x in xs], _bits(gamma), eps, woff, ub,
                 residual_in=None if res is None else _bits(res))
    assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    if fmt == "e4m3fn":
        assert_fp8_close(out.cpu().numpy(), q, min_exact=min_exact)
    else:
        assert_e5m2_close(out.cpu().numpy(), q, min_exact=min_exact)
    return q, s


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2", "mxfp8"])
@pytest.mark.parametrize("cols", [256, 7168])
def test_eps_zero_zero_rows(arn, orc, fmt, cols):
    """Rows 0-1 all zero (+0; -0 mixed in), row 2 ordinary, row 3 tiny but of
    normal fp32 mean square (RMS ~1e-10), rows 4.. random; P = 3 with a
    residual that is zero on the zero rows."""
    print(f"[eps=0] fmt={fmt} cols={cols}", flush=True)
    rows, P = 9, 3
    g = torch.Generator().manual_seed(cols + len(fmt))
    xs = [torch.randn((rows, cols), generator=g) * 0.5 for _ in range(P)]
    res = torch.randn((rows, cols), generator=g)
    for x in xs:
        x[0:2] = 0.0
        x[1, ::3] = -0.0
        x[3] *= 1e-10
    res[0:2] = 0.0
    res[1, ::3] = -0.0  # h = -0 + -0 = -0 there: codes may be -0, never NaN
    res[3] *= 1e-10
    xs = [x.to(torch.bfloat16) for x in xs]
    res = res.to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    out, scales, res_out = _run(arn, fmt, xs, res, gamma, 0.0, 0.0, 1200.0)
    _check(orc, fmt, xs, res, gamma, 0.0, 0.0, 1200.0, out, scales, res_out, min_exact=0.99)
    codes = out.cpu().numpy()
    assert np.all((codes[0:2] & 0x7F) == 0), "zero rows must give zero codes"
    sc = scales.cpu().numpy()
    if fmt == "e4m3fn":
        assert np.all(sc[0:2] == np.float32(1.0 / (448.0 * 512.0)))
        assert np.all(sc[2:] > np.float32(1.0 / (448.0 * 512.0)))
    elif fmt == "e5m2":
        assert np.all(sc[0:2] == np.float32(1.0 / (57344.0 * 512.0)))
    else:
        assert np.all(sc[0:2] == 0)  # E8M0 byte 0: 2^-127
    # the tiny row still normalises to full range
    assert np.max(np.abs(ordered_fp8(codes[3]))) >= (0x7E if fmt != "e5m2" else 0x7B) - 8


def test_eps_zero_in_place_all_zero_workload(arn, orc):
    """The decode workload's shape with every input zero and eps = 0, the
    residual updated in place: floor scales and zero codes on every row."""
    rows, cols, P = 32, 7168, 4
    xs = [torch.zeros((rows, cols), dtype=torch.bfloat16) for _ in range(P)]
    res = torch.zeros((rows, cols), dtype=torch.bfloat16)
    gamma = torch.ones((cols,), dtype=torch.bfloat16)
    out, scales, res_out = _run(arn, "e4m3fn", xs, res, gamma, 0.0, 0.0, 1200.0, in_place=True)
    assert torch.all(out == 0)
    assert torch.all(scales == float(np.float32(1.0 / 229376.0)))
    assert torch.all(res_out.view(torch.int16) == 0)


@pytest.mark.parametrize("P", [2, 5, 8])
def test_one_hot_slabs_reproduce_the_input(arn, orc, P):
    """Every element is nonzero on exactly one rank (+0 on the others): the sum
    is that value exactly, on the sum-only path and as the fused path's
    residual output; the fused outputs also match the oracle."""
    rows, cols = 37, 7176
    print(f"[one-hot] P={P}", flush=True)
    g = torch.Generator().manual_seed(40 + P)
    full = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    owner = torch.randint(0, P, (rows, cols), generator=g)
    xs = [torch.where(owner == p, full, torch.zeros_like(full)) for p in range(P)]
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arn_sum_bf16([x.to(DEV) for x in xs], out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out), _bits(full), "one-hot sum")
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    q, scales, res_out = _run(arn, "e4m3fn", xs, None, gamma, 1e-6, 0.0, 1200.0)
    assert_bits_equal(_bits(res_out), _bits(full), "one-hot residual_out (the sum)")
    _check(orc, "e4m3fn", xs, None, gamma, 1e-6, 0.0, 1200.0, q, scales, res_out,
           min_exact=0.999)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2", "mxfp8"])
@pytest.mark.parametrize("with_res", [False, True])
def test_doubling_with_eps_zero_changes_nothing(arn, orc, fmt, with_res):
    """eps = 0: doubling every slab (and the residual) doubles h exactly; the
    scales and codes stay the same within the parity tolerance, and each run
    matches the oracle."""
    rows, cols, P = 24, 8192, 4
    print(f"[doubling] fmt={fmt} residual={with_res}", flush=True)
    g = torch.Generator().manual_seed(50 + with_res + len(fmt))
    xs = [(torch.randn((rows, cols), generator=g) * 0.5).to(torch.bfloat16) for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16) if with_res else None
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    a = _run(arn, fmt, xs, res, gamma, 0.0, 0.0, 1200.0)
    xs2 = [x * 2 for x in xs]  # exact in bf16
    res2 = None if res is None else res * 2
    b = _run(arn, fmt, xs2, res2, gamma, 0.0, 0.0, 1200.0)
    assert torch.equal(b[2].view(torch.int16), (a[2] * 2).view(torch.int16)), "h must double"
    if fmt == "mxfp8":
        ga, gb = a[1].cpu().numpy().astype(np.int32), b[1].cpu().numpy().astype(np.int32)
        assert np.all(np.abs(ga - gb) <= 1)
        same = ga == gb
        assert same.mean() >= 0.999
    else:
        assert_scales_close(b[1].cpu().numpy(), a[1].cpu().numpy(), "doubled scales")
        assert np.max(np.abs(ordered_fp8(b[0].cpu().numpy()) - ordered_fp8(a[0].cpu().numpy()))) <= 1
    _check(orc, fmt, xs, res, gamma, 0.0, 0.0, 1200.0, *a, min_exact=0.999)
    _check(orc, fmt, xs2, res2, gamma, 0.0, 0.0, 1200.0, *b, min_exact=0.999)


def test_bad_scalars_raise_before_launch(arn):
    x = torch.ones((4, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.full((4, 64), 0x11, dtype=torch.uint8, device=DEV)
    s = torch.full((4,), -1.0, dtype=torch.float32, device=DEV)
    gm = torch.ones((64,), dtype=torch.bfloat16, device=DEV)
    for eps, woff, ub in ((-1e-6, 0.0, 1.0), (float("nan"), 0.0, 1.0), (1e-6, 0.0, 0.0)):
        with pytest.raises(arn.ArnFp8Error) as e:
            arn.arnfp8_run([x], None, None, out, s, gm, eps, woff, ub)
        assert e.value.status == 10
    torch.cuda.synchronize()
    assert torch.all(out == 0x11) and torch.all(s == -1.0), "a rejected call wrote an output"
