"""Seeded random cases of the split-row path (arnfp8_run_split) against the
CPU oracle, and the workloads the benchmark times through it at full size.

Each random case draws its own shape (ragged columns up to 65536, 1 to 300
rows), P, residual mode (none, read only, written only, read and written;
the split path refuses an in-place residual), part count (automatic or 1 to
8, within the 1024 chunks a part may hold), spin bound (the default, or none
at all so that every part recomputes its partners), value scale, zero rows,
shared outliers, eps (0 included), weight offset and scale_ub, all from one
seed, so a failure names a case that can be rerun alone.  One workspace
serves every case, as it would a caller's stream.  The bar is the parity bar
of the other GPU tests.
"""
import numpy as np
import pytest
import torch

from tests._util import assert_bits_equal, assert_fp8_close, assert_scales_close, oracle_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 60
MAX_ELEMS = 400_000
WS_ROWS = 300


@pytest.fixture(scope="module")
def arn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import all_reduce_rmsnorm_amd as arn

    arn.library()
    return arn


@pytest.fixture(scope="module")
def workspace(arn):
    return torch.zeros((arn.arnfp8_split_workspace_bytes(WS_ROWS) // 8,), dtype=torch.int64,
                       device=DEV)


def _bits(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.bf16_bits(t)


def _case(i):
    rng = np.random.default_rng(9100 + i)
    cols = int(rng.integers(1, 65536 // 8 + 1)) * 8 if rng.random() < 0.15 else \
        int(rng.integers(1, 12000 // 8 + 1)) * 8
    rows = int(rng.integers(1, max(2, min(WS_ROWS, MAX_ELEMS // cols)) + 1))
    c16 = cols // 8
    min_parts = -(-c16 // 1024)
    parts = 0 if rng.random() < 0.3 else int(rng.integers(min_parts, 9))
    return dict(rows=rows, cols=cols, P=int(rng.integers(1, 9)),
                res_mode=["none", "in_only", "out_only", "in_out"][int(rng.integers(0, 4))],
                parts=parts, spin=-1 if rng.random() < 0.2 else 0,
                std=float(rng.choice([1e-3, 0.5, 30.0])), woff=float(rng.choice([0.0, 1.0])),
                eps=float(rng.choice([0.0, 1e-6, 1e-5, 1e-3])),
                ub=float(rng.choice([1.0, 64.0, 1200.0])),
                zero_rows=bool(rng.random() < 0.3), outliers=bool(rng.random() < 0.3),
                seed=int(rng.integers(0, 2**31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_split_case_matches_oracle(arn, orc, workspace, i):
    c = _case(i)
    print(f"[split fuzz {i}] {c}", flush=True)
    rows, cols, P = c["rows"], c["cols"], c["P"]
    g = torch.Generator().manual_seed(c["seed"])
    xs = [torch.randn((rows, cols), generator=g) * c["std"] for _ in range(P)]
    res = None
    if c["res_mode"] in ("in_only", "in_out"):
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

    res_out = (torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
               if c["res_mode"] in ("out_only", "in_out") else None)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    arn.arnfp8_run_split([x.to(DEV) for x in xs], None if res is None else res.to(DEV), res_out,
                         out, scales, gamma.to(DEV), c["eps"], c["woff"], c["ub"],
                         workspace=workspace, opts=dict(parts=c["parts"], spin_polls=c["spin"]))
    torch.cuda.synchronize()

    q, s, h = orc.arnfp8([_bits(x) for x in xs], _bits(gamma), c["eps"], c["woff"], c["ub"],
                         residual_in=None if res is None else _bits(res))
    if res_out is not None:
        assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    assert_fp8_close(out.cpu().numpy(), q, min_exact=0.99 if rows * cols >= 8192 else 0.0)


@pytest.mark.parametrize("name", ["token_p8_1x8192", "unit_offset_p8_128x8192"])
def test_benchmarked_split_workload_every_row(arn, orc, name):
    """The workloads the benchmark times through arnfp8_run_split, at full size
    with their own value laws and scalars and the automatic part count the
    benchmark uses: every element against the oracle."""
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[name]
    print(f"[split workload] {name} parts {arn.arnfp8_split_parts(w.rows, w.cols)}", flush=True)
    host = synth.make_inputs(w, device="cpu")
    ws = torch.zeros((arn.arnfp8_split_workspace_bytes(w.rows) // 8,), dtype=torch.int64,
                     device=DEV)
    res_out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((w.rows, w.cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.rows,), dtype=torch.float32, device=DEV)
    arn.arnfp8_run_split([x.to(DEV) for x in host["inputs"]], host["residual"].to(DEV), res_out,
                         out, scales, host["gamma"].to(DEV), w.eps, w.weight_offset, w.scale_ub,
                         workspace=ws)
    torch.cuda.synchronize()
    q, s, h = oracle_rows(orc.arnfp8, [_bits(x) for x in host["inputs"]], _bits(host["gamma"]),
                          w.eps, w.weight_offset, w.scale_ub,
                          residual_in=_bits(host["residual"]), block=16)
    assert_bits_equal(_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    assert_fp8_close(out.cpu().numpy(), q)
