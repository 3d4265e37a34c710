"""Seeded random cases of the fused op against the CPU oracle.

Each case draws its own shape (ragged columns, 1 to a few hundred rows), P,
residual mode (none, read only, written only, read and written, in place),
output format, launch shape (lanes, chunks per lane, grid, store policy),
value scale, zero rows, shared outliers, eps (0 included: zero rows then take
the all-zero result), weight offset and scale_ub, all
from one seed, so a failure names a case that can be rerun alone.  The bar is
the parity bar of the other GPU tests; the share of exactly equal codes is
only checked on cases large enough for it to mean something.
"""
import numpy as np
import pytest
import torch

from tests._util import (assert_bits_equal, assert_e5m2_close, assert_fp8_close,
                         assert_scales_close, check_mx)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 160
MAX_ELEMS = 400_000


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


def _launch(rng, c16):
    """A valid launch shape for rows of c16 16-byte chunks, or None (automatic)."""
    if rng.random() < 0.25:
        return None
    vpts = [v for v in (1, 2, 4, 8, 16) if -(-c16 // v) <= (1024 if v == 1 else 512)]
    vpt = int(rng.choice(vpts))
    limit = 1024 if vpt == 1 else 512
    lanes = -(-c16 // vpt)
    lo = max(64, -(-lanes // 64) * 64)
    threads = int(rng.choice(np.arange(lo, limit + 1, 64)))
    return dict(threads=threads, vpt=vpt, stores=int(rng.integers(0, 3)))


def _case(i):
    rng = np.random.default_rng(7000 + i)
    fmt = ["e4m3fn", "e5m2", "mxfp8"][i % 3]
    unit = 32 if fmt == "mxfp8" else 8
    cols = int(rng.integers(1, 12000 // unit + 1)) * unit
    rows = int(rng.integers(1, max(2, min(300, MAX_ELEMS // cols)) + 1))
    P = int(rng.integers(1, 9))
    res_mode = ["none", "in_only", "out_only", "in_out", "in_place"][int(rng.integers(0, 5))]
    std = float(rng.choice([1e-3, 0.5, 30.0]))
    woff = float(rng.choice([0.0, 1.0]))
    return dict(fmt=fmt, rows=rows, cols=cols, P=P, res_mode=res_mode, std=std, woff=woff,
                eps=float(rng.choice([0.0, 1e-6, 1e-5, 1e-3])),
                ub=float(rng.choice([1.0, 64.0, 1200.0])),
                zero_rows=bool(rng.random() < 0.3), outliers=bool(rng.random() < 0.3),
                launch=_launch(rng, cols // 8), grid=int(rng.integers(1, rows + 4)),
                seed=int(rng.integers(0, 2**31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(arn, orc, i):
    c = _case(i)
    print(f"[fuzz {i}] {c}", flush=True)
    rows, cols, P = c["rows"], c["cols"], c["P"]
    g = torch.Generator().manual_seed(c["seed"])
    xs = [torch.randn((rows, cols), generator=g) * c["std"] for _ in range(P)]
    res = None
    if c["res_mode"] in ("in_only", "in_out", "in_place"):
        res = torch.randn((rows, cols), generator=g) * c["std"]
    if c["outliers"]:
        mask = torch.rand((rows, cols), generator=g) < 0.002
        xs = [torch.where(mask, x * 100.0, x) for x in xs]
    if c["zero_rows"]:
        z = torch.randint(0, rows, (max(1, rows // 8),), generator=g)
        for x in xs:
            x[z] = 0.0
        if res is not None:
            res[z] = 0.0
    xs = [x.to(torch.bfloat16) for x in xs]
    res = None if res is None else res.to(torch.bfloat16)
    if c["woff"] == 1.0:
        gamma = (torch.randn((cols,), generator=g) * 0.02).to(torch.bfloat16)
    else:
        gamma = (torch.rand((cols,), generator=g) + 0.5).to(torch.bfloat16)

    xs_d = [x.to(DEV) for x in xs]
    res_d = None if res is None else res.to(DEV)
    if c["res_mode"] == "in_place":
        res_out = res_d
    elif c["res_mode"] in ("out_only", "in_out"):
        res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    else:
        res_out = None
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    code = {"e4m3fn": arn.FMT_E4M3FN, "e5m2": arn.FMT_E5M2, "mxfp8": arn.FMT_MXFP8}[c["fmt"]]
    if c["fmt"] == "mxfp8":
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    else:
        scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    launch = None if c["launch"] is None else dict(c["launch"], grid=c["grid"])
    arn.arnfp8_run_fmt(xs_d, res_d, res_out, out, scales, gamma.to(DEV), c["eps"], c["woff"],
                       c["ub"], out_format=code, launch=launch)
    torch.cuda.synchronize()

    min_exact = 0.99 if rows * cols >= 8192 else 0.0
    if c["fmt"] == "mxfp8":
        check_mx(orc, xs, res, gamma, out, scales, res_out, eps=c["eps"], woff=c["woff"],
                 min_exact=min_exact)
        return
    fn = orc.arnfp8 if c["fmt"] == "e4m3fn" else orc.arnfp8_e5m2
    q, s, h = fn([_bits(x) for x in xs], _bits(gamma), c["eps"], c["woff"], c["ub"],
                 residual_in=None if res is None else _bits(res))
    if res_out is not None:
        assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    if c["fmt"] == "e4m3fn":
        assert_fp8_close(out.cpu().numpy(), q, min_exact=min_exact)
    else:
        assert_e5m2_close(out.cpu().numpy(), q, min_exact=min_exact)
