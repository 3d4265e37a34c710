"""Every row of the full prefill workload against the CPU oracle.

P = 8 bf16 slabs [8192, 7168] ~ N(0, 0.5) with 0.1 % shared outliers x100, a
bf16 residual ~ N(0, 1), gamma ~ U(0.8, 1.2), eps 1e-6, scale_ub 64: the
workload the benchmark times, in the launch it times (automatic shape,
residual out of place).  The oracle runs on blocks of rows in a thread pool
(rows are independent), so every element of every output is compared:
residual bit-exact, scales within 1e-5 relative, codes within one step.  The
criterion is the one TensorRT-LLM PR #19836 (Description, test results) and
b12x PR #283 (Validation) state over the whole output, not a sample.
"""
import numpy as np
import pytest
import torch

from tests._util import (assert_bits_equal, assert_e5m2_close, assert_fp8_close,
                         assert_scales_close, check_mx, oracle_rows)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def arn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import all_reduce_rmsnorm_amd as arn

    arn.library()
    return arn


@pytest.fixture(scope="module")
def prefill(arn):
    """The workload on the device, and its host bit patterns for the oracle."""
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS["prefill_p8_8192x7168"]
    print(f"[prefill every row] generating {w.name}", flush=True)
    d = synth.make_inputs(w, device=DEV)
    host = {"xs": [synth.bf16_bits(x) for x in d["inputs"]],
            "res": synth.bf16_bits(d["residual"]), "gamma": synth.bf16_bits(d["gamma"])}
    yield w, d, host
    del d
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def e4m3_ref(orc, prefill):
    w, _, host = prefill
    print("[prefill every row] oracle, e4m3fn", flush=True)
    return oracle_rows(orc.arnfp8, host["xs"], host["gamma"], w.eps, w.weight_offset, w.scale_ub,
                       residual_in=host["res"])


def _fp8(t):
    return t.view(torch.uint8).cpu().numpy()


def test_every_row_e4m3fn(arn, prefill, e4m3_ref):
    from all_reduce_rmsnorm_amd import synth

    w, d, _ = prefill
    print("[prefill every row] e4m3fn", flush=True)
    out = torch.empty((w.rows, w.cols), dtype=torch.float8_e4m3fn, device=DEV)
    scales = torch.empty((w.rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run(d["inputs"], d["residual"], res_out, out, scales, d["gamma"], w.eps,
                   w.weight_offset, w.scale_ub)
    torch.cuda.synchronize()
    q, s, h = e4m3_ref
    assert_bits_equal(synth.bf16_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    assert_fp8_close(_fp8(out), q)
    clamped = s == np.float32(w.scale_ub / 448.0)
    print(f"[prefill every row] rows where scale_ub clamps: {int(clamped.sum())} of {w.rows}",
          flush=True)
    assert clamped.any() and (~clamped).any()


def test_every_row_e5m2(arn, orc, prefill):
    from all_reduce_rmsnorm_amd import synth

    w, d, host = prefill
    print("[prefill every row] e5m2", flush=True)
    out = torch.empty((w.rows, w.cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run_fmt(d["inputs"], d["residual"], res_out, out, scales, d["gamma"], w.eps,
                       w.weight_offset, w.scale_ub, out_format=arn.FMT_E5M2)
    torch.cuda.synchronize()
    q, s, h = oracle_rows(orc.arnfp8_e5m2, host["xs"], host["gamma"], w.eps, w.weight_offset,
                          w.scale_ub, residual_in=host["res"])
    assert_bits_equal(synth.bf16_bits(res_out), h, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s)
    assert_e5m2_close(out.cpu().numpy(), q)


def test_every_row_mxfp8(arn, orc, prefill):
    w, d, host = prefill
    print("[prefill every row] mxfp8", flush=True)
    out = torch.empty((w.rows, w.cols), dtype=torch.uint8, device=DEV)
    bscales = torch.empty((w.rows, w.cols // 32), dtype=torch.uint8, device=DEV)
    res_out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run_fmt(d["inputs"], d["residual"], res_out, out, bscales, d["gamma"], w.eps,
                       w.weight_offset, w.scale_ub, out_format=arn.FMT_MXFP8)
    torch.cuda.synchronize()
    ref = oracle_rows(orc.arnfp8_mx, host["xs"], host["gamma"], w.eps, w.weight_offset,
                      residual_in=host["res"])
    check_mx(orc, host["xs"], host["res"], host["gamma"], out, bscales, res_out, eps=w.eps,
             woff=w.weight_offset, ref=ref)


def test_every_rank_of_the_two_stage_share(arn, prefill, e4m3_ref):
    """All 8 ranks' shares (1024 rows each), as the benchmark times them: every
    slot byte against the oracle's rows of that share, every residual row, and
    the shares together equal a full call's residual."""
    import oracle as orc_mod
    from all_reduce_rmsnorm_amd import synth

    w, d, _ = prefill
    ngpus = 8
    q, s, h = e4m3_ref
    nbytes = arn.arnfp8_stage_bytes(w.rows, w.cols, ngpus)
    S = -(-w.rows // ngpus)
    res_out = torch.full((w.rows, w.cols), 7.0, dtype=torch.bfloat16, device=DEV)
    for rank in range(ngpus):
        print(f"[prefill every row] share rank {rank} of {ngpus}", flush=True)
        staging = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        arn.arnfp8_run_share(d["inputs"], d["residual"], res_out, staging, d["gamma"], w.eps,
                             w.weight_offset, w.scale_ub, ngpus=ngpus, rank=rank)
        torch.cuda.synchronize()
        first, count = orc_mod.share_rows(w.rows, ngpus, rank)
        got = staging.cpu().numpy()
        data = got[: S * w.cols].reshape(S, w.cols)
        assert_fp8_close(data[:count], q[first:first + count])
        assert_scales_close(got[S * w.cols: S * w.cols + 4 * count].view(np.float32),
                            s[first:first + count])
        assert np.all(got[S * w.cols + 4 * count:] == 0xA5)
    assert_bits_equal(synth.bf16_bits(res_out), h, "residual of all shares")
