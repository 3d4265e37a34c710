"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generators in ``all_reduce_rmsnorm_amd.synth``;
the oracle sees the very same bytes.  Bar: bf16 bit-exact, scales within
1e-5 relative, fp8 within one e4m3 step (see ``tests/_util.py``).
"""
import numpy as np
import pytest
import torch

from tests._util import assert_bits_equal, assert_fp8_close, assert_scales_close

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
def synth():
    from all_reduce_rmsnorm_amd import synth

    return synth


def _bits(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.bf16_bits(t)


def _fp8(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.fp8_bits(t)


def run_fused(arn, inputs, gamma, eps, woff, ub, residual=None, in_place=True, want_res_out=True):
    rows, cols = inputs[0].shape
    out = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_out = None
    if want_res_out:
        if residual is not None and in_place:
            res_out = residual
        else:
            res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run(inputs, residual, res_out, out, scales, gamma, eps, woff, ub)
    torch.cuda.synchronize()
    return out, scales, res_out


def check_against_oracle(orc, inputs_h, gamma_h, eps, woff, ub, res_h, out, scales, res_out,
                         min_exact=0.999):
    q_ref, s_ref, h_ref = orc.arnfp8([_bits(x) for x in inputs_h], _bits(gamma_h), eps, woff, ub,
                                     residual_in=None if res_h is None else _bits(res_h))
    if res_out is not None:
        assert_bits_equal(_bits(res_out), h_ref, "residual_out")
    assert_scales_close(scales.cpu().numpy(), s_ref)
    assert_fp8_close(_fp8(out), q_ref, min_exact=min_exact)
    return q_ref, s_ref, h_ref


# ------------------------------------------------------------------ sum ----

@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 40), (37, 2880), (64, 4096), (5, 7176)])
def test_sum_bf16_bit_exact(arn, orc, P, rows, cols):
    print(f"[sum] P={P} rows={rows} cols={cols}", flush=True)
    g = torch.Generator().manual_seed(1000 * P + rows)
    xs = [(torch.randn((rows, cols), generator=g) * 3.0).to(torch.bfloat16) for _ in range(P)]
    dev = [x.to(DEV) for x in xs]
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arn_sum_bf16(dev, out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out), orc.sum_bf16([_bits(x) for x in xs]), "sum")


def test_sum_workload_full_size(arn, orc, synth):
    w = synth.WORKLOADS["sum_p4_64x4096"]
    print(f"[sum] workload {w.name}", flush=True)
    h = synth.make_inputs(w, device="cpu")
    dev = [x.to(DEV) for x in h["inputs"]]
    out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
    arn.arn_sum_bf16(dev, out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out), orc.sum_bf16([_bits(x) for x in h["inputs"]]), "sum")


@pytest.mark.parametrize("P", [3, 8])
def test_sum_wide_path_ragged_tail(arn, orc, P):
    """The large-tensor path of the sum (4 chunks per lane, a buffer window per
    iteration) on a tensor whose chunk count is not a multiple of the window:
    9001 x 7176 has 8,073,897 chunks.  Every element is compared, and bytes
    past the end of the output stay untouched."""
    rows, cols = 9001, 7176
    print(f"[sum] wide ragged P={P} rows={rows} cols={cols}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(77 + P)
    xs = [torch.randn((rows, cols), generator=g, device=DEV, dtype=torch.bfloat16) for _ in range(P)]
    guard = torch.full((rows * cols + 4096,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = guard[: rows * cols].view(rows, cols)
    arn.arn_sum_bf16(xs, out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out), orc.sum_bf16([_bits(x) for x in xs]), "sum")
    assert torch.all(guard[rows * cols:] == -7.0)


def test_sum_negative_zero_and_ties(arn, orc):
    # P = 1 keeps -0; exact half-ulp ties round to even.
    vals = torch.tensor([[-0.0, 0.0, 16.0, 16.125, 1.0, -16.0, 8.0, 3.0]], dtype=torch.float32)
    x = vals.to(torch.bfloat16)
    out = torch.empty_like(x, device=DEV)
    arn.arn_sum_bf16([x.to(DEV)], out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out), _bits(x), "P=1 identity")
    y = torch.tensor([[0.0, -0.0, 0.0625, 0.0625, 2.0 ** -8, -0.0625, 8.0, 2.0 ** -7]]).to(torch.bfloat16)
    out2 = torch.empty_like(x, device=DEV)
    arn.arn_sum_bf16([x.to(DEV), y.to(DEV)], out2)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(out2), orc.sum_bf16([_bits(x), _bits(y)]), "ties")


# ---------------------------------------------------------------- fused ----

@pytest.mark.parametrize("name", ["tiny_p2_4x256", "decode_p4_32x7168", "unit_offset_p8_128x8192",
                                  "prefill_share_p8_1024x7168"])
def test_fused_workload_full_size(arn, orc, synth, name):
    w = synth.WORKLOADS[name]
    print(f"[fused] workload {w.name}", flush=True)
    h = synth.make_inputs(w, device="cpu")
    dev = [x.to(DEV) for x in h["inputs"]]
    res = None if h["residual"] is None else h["residual"].to(DEV)
    out, scales, res_out = run_fused(arn, dev, h["gamma"].to(DEV), w.eps, w.weight_offset,
                                     w.scale_ub, residual=res, in_place=True)
    check_against_oracle(orc, h["inputs"], h["gamma"], w.eps, w.weight_offset, w.scale_ub,
                         h["residual"], out, scales, res_out)


P2_COLS = [8, 2880, 7168, 7176, 8192, 16384]
P2_ROWS = [1, 32, 37, 64]


@pytest.mark.parametrize("cols", P2_COLS)
@pytest.mark.parametrize("rows", P2_ROWS)
def test_fused_shape_menu(arn, orc, rows, cols):
    """Hidden sizes and token counts of TensorRT-LLM PR #19836's test set."""
    P = 4 if cols % 16 == 0 else 2
    print(f"[fused] menu P={P} rows={rows} cols={cols}", flush=True)
    g = torch.Generator().manual_seed(rows * 100003 + cols)
    xs = [(torch.randn((rows, cols), generator=g) * 0.5).to(torch.bfloat16) for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    out, scales, res_out = run_fused(arn, [x.to(DEV) for x in xs], gamma.to(DEV), 1e-6, 0.0,
                                     1200.0, residual=res.to(DEV), in_place=False)
    check_against_oracle(orc, xs, gamma, 1e-6, 0.0, 1200.0, res, out, scales, res_out,
                         min_exact=0.99 if rows * cols < 4096 else 0.999)


@pytest.mark.parametrize("P", [1, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("res_mode", ["none", "out_only", "in_only", "in_out"])
def test_fused_every_p_and_residual_mode(arn, orc, P, res_mode):
    rows, cols = 9, 1000  # 125 chunks per row: a ragged last wave
    print(f"[fused] P={P} residual={res_mode}", flush=True)
    g = torch.Generator().manual_seed(P * 7 + len(res_mode))
    xs = [torch.randn((rows, cols), generator=g).to(torch.bfloat16) for _ in range(P)]
    gamma = (torch.randn((cols,), generator=g) * 0.1 + 1.0).to(torch.bfloat16)
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    res_in = res.to(DEV) if res_mode in ("in_only", "in_out") else None
    want_out = res_mode in ("out_only", "in_out")
    out, scales, res_out = run_fused(arn, [x.to(DEV) for x in xs], gamma.to(DEV), 1e-5, 0.0,
                                     1200.0, residual=res_in, in_place=False,
                                     want_res_out=want_out)
    check_against_oracle(orc, xs, gamma, 1e-5, 0.0, 1200.0,
                         res if res_in is not None else None, out, scales, res_out, min_exact=0.99)


# ---------------------------------------------------------- edge cases ----

def test_rows_zero_is_a_noop(arn):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, 64), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((0,), dtype=torch.float32, device=DEV)
    g = torch.ones((64,), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run([x, x], None, None, out, s, g, 1e-6, 0.0, 1.0, rows=0, cols=64)
    arn.arn_sum_bf16([x], torch.empty_like(x), rows=0, cols=64)
    torch.cuda.synchronize()


def test_max_cols(arn, orc):
    rows, cols = 3, 65536
    g = torch.Generator().manual_seed(5)
    xs = [torch.randn((rows, cols), generator=g).to(torch.bfloat16) for _ in range(8)]
    gamma = (torch.rand((cols,), generator=g) + 0.5).to(torch.bfloat16)
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    out, scales, res_out = run_fused(arn, [x.to(DEV) for x in xs], gamma.to(DEV), 1e-6, 0.0,
                                     1200.0, residual=res.to(DEV), in_place=True)
    check_against_oracle(orc, xs, gamma, 1e-6, 0.0, 1200.0, res, out, scales, res_out)


def test_zero_and_tiny_rows_take_the_floor(arn, orc):
    rows, cols = 4, 512
    x = torch.zeros((rows, cols), dtype=torch.bfloat16)
    x[2] = 2.0 ** -20
    x[3, 7] = -(2.0 ** -30)
    gamma = torch.ones((cols,), dtype=torch.bfloat16)
    out, scales, res_out = run_fused(arn, [x.to(DEV), x.to(DEV)], gamma.to(DEV), 1.0, 0.0, 1200.0)
    check_against_oracle(orc, [x, x], gamma, 1.0, 0.0, 1200.0, None, out, scales, res_out,
                         min_exact=0.99)
    assert np.all(scales.cpu().numpy() == np.float32(1.0 / 229376.0))


def test_scale_clamps_exactly_at_ub(arn, orc):
    rows, cols = 16, 2048
    g = torch.Generator().manual_seed(6)
    xs = [torch.randn((rows, cols), generator=g).to(torch.bfloat16) for _ in range(4)]
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    ub = 2.5
    out, scales, res_out = run_fused(arn, [x.to(DEV) for x in xs], gamma.to(DEV), 1e-6, 0.0, ub)
    _, s_ref, _ = check_against_oracle(orc, xs, gamma, 1e-6, 0.0, ub, None, out, scales, res_out)
    s = scales.cpu().numpy()
    clamped = s_ref == np.float32(ub / 448.0)
    assert clamped.all()
    assert np.all(s == np.float32(ub / 448.0))


def test_unit_gain_bitwise(arn):
    """gamma = 0 with weight_offset = 1 equals gamma = 1 with weight_offset = 0."""
    rows, cols = 64, 8192
    g = torch.Generator().manual_seed(7)
    xs = [(torch.randn((rows, cols), generator=g) * 0.25).to(torch.bfloat16).to(DEV) for _ in range(8)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16).to(DEV)
    a = run_fused(arn, xs, torch.zeros(cols, dtype=torch.bfloat16, device=DEV), 1e-5, 1.0, 1200.0,
                  residual=res, in_place=False)
    b = run_fused(arn, xs, torch.ones(cols, dtype=torch.bfloat16, device=DEV), 1e-5, 0.0, 1200.0,
                  residual=res, in_place=False)
    assert torch.equal(a[0].view(torch.uint8), b[0].view(torch.uint8))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_repeat_calls_bitwise_deterministic(arn, synth):
    """100 repeated calls of the fused op and of the sum give the same bits."""
    w = synth.WORKLOADS["unit_offset_p8_128x8192"]
    d = synth.make_inputs(w, device=DEV)
    first = run_fused(arn, d["inputs"], d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                      residual=d["residual"], in_place=False)
    s0 = torch.empty_like(d["inputs"][0])
    arn.arn_sum_bf16(d["inputs"], s0)
    s1 = torch.empty_like(s0)
    for _ in range(100):
        again = run_fused(arn, d["inputs"], d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                          residual=d["residual"], in_place=False)
        assert torch.equal(first[0].view(torch.uint8), again[0].view(torch.uint8))
        assert torch.equal(first[1], again[1]) and torch.equal(first[2], again[2])
        s1.zero_()
        arn.arn_sum_bf16(d["inputs"], s1)
        assert torch.equal(s0.view(torch.int16), s1.view(torch.int16))


def test_graph_replay_matches_eager(arn, synth):
    """Capture one fused call in a graph; every replay (with eager work and a
    synchronisation between replays) equals the eager result bitwise."""
    w = synth.WORKLOADS["decode_p4_32x7168"]
    d = synth.make_inputs(w, device=DEV)
    eager = run_fused(arn, d["inputs"], d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                      residual=d["residual"], in_place=False)
    out = torch.empty_like(eager[0])
    scales = torch.empty_like(eager[1])
    res_out = torch.empty_like(eager[2])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the side stream, as graph capture asks
        arn.arnfp8_run(d["inputs"], d["residual"], res_out, out, scales, d["gamma"], w.eps,
                       w.weight_offset, w.scale_ub)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        arn.arnfp8_run(d["inputs"], d["residual"], res_out, out, scales, d["gamma"], w.eps,
                       w.weight_offset, w.scale_ub)
    for k in range(3):
        out.view(torch.uint8).fill_(0x7F)
        scales.fill_(-1.0)
        res_out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), eager[0].view(torch.uint8)), k
        assert torch.equal(scales, eager[1]) and torch.equal(res_out, eager[2]), k
        _ = (d["inputs"][0].float() * 2.0).sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("name", ["decode_p4_32x7168", "prefill_p8_8192x7168"])
def test_in_place_residual_matches_out_of_place(arn, synth, name):
    w = synth.WORKLOADS[name]
    print(f"[fused] in place vs out of place {name}", flush=True)
    d = synth.make_inputs(w, device=DEV)
    res_copy = d["residual"].clone()
    a = run_fused(arn, d["inputs"], d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                  residual=res_copy, in_place=False)
    b = run_fused(arn, d["inputs"], d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                  residual=d["residual"], in_place=True)
    assert torch.equal(a[0].view(torch.uint8), b[0].view(torch.uint8))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_errors_raise_before_launch(arn):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 64), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((4,), dtype=torch.float32, device=DEV)
    g = torch.ones((64,), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_run([x, x], None, x, out, s, g, 1e-6, 0.0, 1.0)  # residual_out aliases inputs
    assert e.value.status == 5
    flat = torch.zeros((4 * 64 + 4,), dtype=torch.bfloat16, device=DEV)
    shifted = flat[4:].view(4, 64)  # contiguous, but 8 bytes past a 16-byte boundary
    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arnfp8_run([shifted], None, None, out, s, g, 1e-6, 0.0, 1.0)
    assert e.value.status == 2
    with pytest.raises(ValueError):  # a strided view is refused by the binding
        arn.arnfp8_run([x[:, 8:]], None, None, out, s, g, 1e-6, 0.0, 1.0, rows=4, cols=56)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,launch", [("unit_offset_p8_128x8192", dict(threads=1024, vpt=1)),
                                         ("unit_offset_p8_128x8192", dict(threads=512, vpt=2)),
                                         ("prefill_p8_8192x7168", None)])
def test_unfused_two_launch_chain_is_bitwise_equal(arn, synth, name, launch):
    """arn_sum_bf16 to HBM, then the fused kernel with P = 1 on the sum: the
    same bytes as the single fused launch in the same launch shape (the fusion
    changes no result), on the benchmark's prefill workload too, where the
    automatic shape is the same for P = 8 and P = 1.  (Between launch shapes
    the scales and codes may differ in the last bits: the order of the row's
    sum of squares follows the shape.)"""
    w = synth.WORKLOADS[name]
    print(f"[fused] unfused chain {name} {launch}", flush=True)
    d = synth.make_inputs(w, device=DEV)

    def run(inputs):
        out = torch.empty((w.rows, w.cols), dtype=torch.float8_e4m3fn, device=DEV)
        scales = torch.empty((w.rows,), dtype=torch.float32, device=DEV)
        res_out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
        arn.arnfp8_run_ex(inputs, d["residual"], res_out, out, scales, d["gamma"], w.eps,
                          w.weight_offset, w.scale_ub, launch=launch)
        torch.cuda.synchronize()
        return out, scales, res_out

    fused = run(d["inputs"])
    s = torch.empty_like(d["inputs"][0])
    arn.arn_sum_bf16(d["inputs"], s)
    unfused = run([s])
    assert torch.equal(fused[0].view(torch.uint8), unfused[0].view(torch.uint8))
    assert torch.equal(fused[1], unfused[1]) and torch.equal(fused[2], unfused[2])


@pytest.mark.parametrize("launch", [dict(threads=960, vpt=1), dict(threads=1024),
                                    dict(stores=1), dict(stores=2), dict(threads=512, vpt=2, stores=1),
                                    dict(threads=64, vpt=16), dict(threads=128, vpt=8),
                                    dict(threads=256, vpt=4), dict(threads=512, vpt=2),
                                    dict(threads=448, vpt=4, grid=7), dict(threads=320, vpt=4, grid=1)])
def test_every_launch_shape_matches_the_oracle(arn, orc, launch):
    rows, cols = 13, 7176  # 897 chunks: ragged for every shape above
    print(f"[fused] launch {launch}", flush=True)
    g = torch.Generator().manual_seed(sum(launch.values()))
    xs = [(torch.randn((rows, cols), generator=g) * 0.5).to(torch.bfloat16) for _ in range(8)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    out = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run_ex([x.to(DEV) for x in xs], res.to(DEV), res_out, out, scales, gamma.to(DEV),
                      1e-6, 0.0, 1200.0, launch=launch)
    torch.cuda.synchronize()
    check_against_oracle(orc, xs, gamma, 1e-6, 0.0, 1200.0, res, out, scales, res_out)


def test_bad_launch_options_rejected(arn):
    x = torch.zeros((4, 1024), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((4,), dtype=torch.float32, device=DEV)
    g = torch.ones((1024,), dtype=torch.bfloat16, device=DEV)
    for bad in (dict(threads=96), dict(threads=1024, vpt=2), dict(threads=1088), dict(vpt=3),
                dict(threads=64, vpt=1),
                dict(grid=-1), dict(variant=9)):
        with pytest.raises(arn.ArnFp8Error) as e:
            arn.arnfp8_run_ex([x], None, None, out, s, g, 1e-6, 0.0, 1.0, launch=bad)
        assert e.value.status == 7, bad


@pytest.mark.parametrize("ngpus", [1, 3, 8, 64])
def test_two_stage_share_and_staging_layout(arn, orc, ngpus):
    """Every rank's share: the staging slot holds the oracle's fp8 rows and
    scales of that share; the share's residual rows are updated, no other row
    is touched; all shares together equal the single full call bitwise."""
    import oracle as orc_mod

    rows, cols, P = 37, 2880, 4
    print(f"[share] ngpus={ngpus}", flush=True)
    g = torch.Generator().manual_seed(ngpus)
    xs = [(torch.randn((rows, cols), generator=g) * 0.5).to(torch.bfloat16) for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    q_ref, s_ref, h_ref = orc.arnfp8([_bits(x) for x in xs], _bits(gamma), 1e-6, 0.0, 1200.0,
                                     residual_in=_bits(res))
    dxs = [x.to(DEV) for x in xs]
    full = run_fused(arn, dxs, gamma.to(DEV), 1e-6, 0.0, 1200.0, residual=res.to(DEV),
                     in_place=False)
    nbytes = arn.arnfp8_stage_bytes(rows, cols, ngpus)
    assert nbytes == orc_mod.stage_bytes(rows, cols, ngpus)
    S = -(-rows // ngpus)
    for rank in range(ngpus):
        staging = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        res_out = torch.full((rows, cols), 7.0, dtype=torch.bfloat16, device=DEV)
        arn.arnfp8_run_share(dxs, res.to(DEV), res_out, staging, gamma.to(DEV), 1e-6, 0.0, 1200.0,
                             ngpus=ngpus, rank=rank)
        torch.cuda.synchronize()
        first, count = orc_mod.share_rows(rows, ngpus, rank)
        want = orc_mod.stage_share(q_ref, s_ref, ngpus, rank, fill=0xA5)
        got = staging.cpu().numpy()
        data_g = got[: S * cols].reshape(S, cols)
        data_w = want[: S * cols].reshape(S, cols)
        assert_fp8_close(data_g[:count], data_w[:count], min_exact=0.99)
        assert np.all(data_g[count:] == 0xA5)
        sc_g = got[S * cols: S * cols + 4 * count].view(np.float32)
        assert_scales_close(sc_g, want[S * cols: S * cols + 4 * count].view(np.float32))
        assert np.all(got[S * cols + 4 * count:] == 0xA5)
        rb = _bits(res_out)
        assert_bits_equal(rb[first:first + count], h_ref[first:first + count], "share residual")
        untouched = np.ones(rows, bool)
        untouched[first:first + count] = False
        assert np.all(rb[untouched] == 0x40E0)  # 7.0 in bf16
        # the share's bytes equal the single full call's rows (same kernel shape)
        full_q = full[0].view(torch.uint8).cpu().numpy()[first:first + count]
        assert np.array_equal(data_g[:count], full_q)
        assert np.array_equal(sc_g, full[1].cpu().numpy()[first:first + count])


def test_two_stage_share_in_place(arn):
    """Every rank's share with the residual updated in place (residual_out ==
    residual_in, as the benchmark also times it): the slot and the share's
    residual rows are the out-of-place share's bits, and rows outside the
    share keep their input values."""
    rows, cols, P, ngpus = 37, 2880, 4, 8
    print(f"[share] in place ngpus={ngpus}", flush=True)
    g = torch.Generator().manual_seed(55)
    dxs = [(torch.randn((rows, cols), generator=g) * 0.5).to(torch.bfloat16).to(DEV)
           for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16).to(DEV)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16).to(DEV)
    nbytes = arn.arnfp8_stage_bytes(rows, cols, ngpus)
    S = -(-rows // ngpus)
    for rank in range(ngpus):
        want_slot = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        want_res = torch.full((rows, cols), 7.0, dtype=torch.bfloat16, device=DEV)
        arn.arnfp8_run_share(dxs, res, want_res, want_slot, gamma, 1e-6, 0.0, 1200.0,
                             ngpus=ngpus, rank=rank)
        slot = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        inplace = res.clone()
        arn.arnfp8_run_share(dxs, inplace, inplace, slot, gamma, 1e-6, 0.0, 1200.0,
                             ngpus=ngpus, rank=rank)
        torch.cuda.synchronize()
        assert torch.equal(slot, want_slot), rank
        first, last = rank * S, min(rows, (rank + 1) * S)
        if first < last:
            assert torch.equal(inplace[first:last].view(torch.int16),
                               want_res[first:last].view(torch.int16)), rank
        outside = torch.ones(rows, dtype=torch.bool, device=DEV)
        outside[first:last] = False
        assert torch.equal(inplace[outside].view(torch.int16), res[outside].view(torch.int16))


def test_slabs_larger_than_4GiB(arn, orc):
    """64-bit offsets: P = 2 slabs of 4.3 GiB each (rows x cols x 2 bytes > 2^32);
    the oracle checks rows past the 4 GiB mark, and the sum kernel the same."""
    rows, cols = 1_100_000, 2048
    print(f"[fused] >4GiB slabs rows={rows} cols={cols}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(99)
    xs = [torch.randn((rows, cols), generator=g, device=DEV, dtype=torch.bfloat16) for _ in range(2)]
    gamma = torch.ones((cols,), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run(xs, None, res_out, out, scales, gamma, 1e-6, 0.0, 1200.0)
    torch.cuda.synchronize()
    pick = torch.tensor([0, 1048575, 1048576, 1048577, rows - 2, rows - 1], device=DEV)
    xs_h = [x.index_select(0, pick).cpu() for x in xs]
    q, s, h = orc.arnfp8([_bits(x) for x in xs_h], _bits(gamma.cpu()), 1e-6, 0.0, 1200.0)
    assert_bits_equal(_bits(res_out.index_select(0, pick)), h, "residual_out")
    assert_scales_close(scales.index_select(0, pick).cpu().numpy(), s)
    assert_fp8_close(out.index_select(0, pick).cpu().numpy(), q, min_exact=0.99)
    del out, scales
    sum_out = res_out
    sum_out.fill_(0)
    arn.arn_sum_bf16(xs, sum_out)
    torch.cuda.synchronize()
    assert_bits_equal(_bits(sum_out.index_select(0, pick)), h, "sum")


def test_graph_replay_of_share_and_formats(arn, synth):
    """The share and the e5m2 / MXFP8 entry points captured in one graph:
    every replay equals the eager result bitwise."""
    w = synth.WORKLOADS["decode_p4_32x7168"]
    d = synth.make_inputs(w, device=DEV)
    rows, cols = w.rows, w.cols
    stg = torch.zeros((arn.arnfp8_stage_bytes(rows, cols, 4),), dtype=torch.uint8, device=DEV)
    q5 = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    s5 = torch.empty((rows,), dtype=torch.float32, device=DEV)
    qm = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    sm = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    ro = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)  # rows outside the share stay 0

    def calls():
        arn.arnfp8_run_share(d["inputs"], d["residual"], ro, stg, d["gamma"], w.eps, 0.0, 1200.0,
                             ngpus=4, rank=2)
        arn.arnfp8_run_fmt(d["inputs"], d["residual"], None, q5, s5, d["gamma"], w.eps, 0.0,
                           1200.0, out_format=arn.FMT_E5M2)
        arn.arnfp8_run_fmt(d["inputs"], d["residual"], None, qm, sm, d["gamma"], w.eps, 0.0,
                           0.0, out_format=arn.FMT_MXFP8)

    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (stg, q5, s5, qm, sm, ro)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for k in range(3):
        for t in (stg, q5, qm, sm):
            t.fill_(0x5A)
        s5.fill_(-1.0)
        ro.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((stg, q5, s5, qm, sm, ro), eager):
            assert torch.equal(a, b), k


def test_concurrent_calls_on_two_streams(arn, synth):
    """arnfp8_run keeps no state between calls: two streams running the fused
    op at the same time, each on its own buffers, give the single-stream
    results bit for bit."""
    w = synth.WORKLOADS["unit_offset_p8_128x8192"]
    print("[fused] two streams", flush=True)
    sets = []
    for seed in (3, 4):
        d = synth.make_inputs(w, device=DEV, seed=seed)
        out = torch.empty((w.rows, w.cols), dtype=torch.float8_e4m3fn, device=DEV)
        sc = torch.empty((w.rows,), dtype=torch.float32, device=DEV)
        ro = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=DEV)
        sets.append((d, out, sc, ro))

    def call(k):
        d, out, sc, ro = sets[k]
        arn.arnfp8_run(d["inputs"], d["residual"], ro, out, sc, d["gamma"], w.eps,
                       w.weight_offset, w.scale_ub)

    ref = []
    for k in range(2):
        call(k)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in sets[k][1:]])
        for t in sets[k][1:]:
            t.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(20):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                call(k)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(2):
        for got, want in zip(sets[k][1:], ref[k]):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), k
