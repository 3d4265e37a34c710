"""GPU parity of the split-row path (arnfp8_run_split) against the CPU oracle.

A row is spread over `parts` workgroups that trade their partial statistics
through a workspace (TensorRT-LLM PR #19836, Description: one token over a
cluster of 8 CTAs).  Bar: the parity bar of the other tests (bf16 bit-exact,
scales within 1e-5, codes within one step).  Beyond parity:
  * the fallback (a part computes a late partner's partial itself) gives the
    same bits as the exchange, so results do not depend on scheduling;
  * the per-row counts in the workspace stay in step across calls of any
    shape and across graph replays;
  * bad workspaces and an in-place residual are refused before launch.
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


def _bits(t):
    from all_reduce_rmsnorm_amd import synth

    return synth.bf16_bits(t)


def _case(seed, rows, cols, P, res_mode, std=0.5):
    g = torch.Generator().manual_seed(seed)
    xs = [(torch.randn((rows, cols), generator=g) * std).to(torch.bfloat16) for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16)
    return xs, (res if res_mode in ("in_only", "in_out") else None), gamma


def _workspace(arn, rows):
    return torch.zeros((max(16, arn.arnfp8_split_workspace_bytes(rows)) // 8,), dtype=torch.int64,
                       device=DEV)


def _run(arn, xs, res, gamma, want_res_out, ws, opts=None, eps=1e-6, woff=0.0, ub=1200.0):
    rows, cols = xs[0].shape
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows,), dtype=torch.float32, device=DEV)
    res_out = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV) if want_res_out else None
    arn.arnfp8_run_split([x.to(DEV) for x in xs], None if res is None else res.to(DEV), res_out,
                         out, scales, gamma.to(DEV), eps, woff, ub, workspace=ws, opts=opts)
    torch.cuda.synchronize()
    return out, scales, res_out


CASES = [  # rows, cols, P, parts (0: automatic), residual mode
    (1, 8192, 8, 0, "in_out"), (1, 7168, 4, 0, "in_out"), (1, 7168, 8, 2, "in_only"),
    (1, 7168, 8, 8, "none"), (3, 2880, 5, 4, "out_only"), (32, 7168, 4, 0, "in_out"),
    (128, 8192, 8, 0, "in_out"), (37, 7176, 3, 8, "in_out"), (2, 65536, 8, 8, "in_out"),
    (5, 8, 1, 1, "in_out"), (6, 1000, 2, 3, "in_out"), (300, 2048, 8, 0, "out_only"),
]


@pytest.mark.parametrize("rows,cols,P,parts,res_mode", CASES)
def test_split_matches_oracle(arn, orc, rows, cols, P, parts, res_mode):
    print(f"[split] rows={rows} cols={cols} P={P} parts={parts} residual={res_mode}", flush=True)
    xs, res, gamma = _case(rows * 7 + cols + P, rows, cols, P, res_mode)
    want_out = res_mode in ("out_only", "in_out")
    ws = _workspace(arn, rows)
    q, s, h = _run(arn, xs, res, gamma, want_out, ws, opts=dict(parts=parts))
    q_ref, s_ref, h_ref = orc.arnfp8([_bits(x) for x in xs], _bits(gamma), 1e-6, 0.0, 1200.0,
                                     residual_in=None if res is None else _bits(res))
    if want_out:
        assert_bits_equal(_bits(h), h_ref, "residual_out")
    assert_scales_close(s.cpu().numpy(), s_ref)
    assert_fp8_close(q.cpu().numpy(), q_ref, min_exact=0.99 if rows * cols < 4096 else 0.999)


@pytest.mark.parametrize("rows,cols,P,parts", [(1, 8192, 8, 8), (32, 7168, 4, 8), (7, 7176, 6, 3)])
def test_fallback_gives_the_same_bits_as_the_exchange(arn, rows, cols, P, parts):
    """With no waiting at all every part computes every partner's partial
    itself: the outputs equal the exchanged ones bit for bit."""
    xs, res, gamma = _case(11 + rows, rows, cols, P, "in_out")
    a = _run(arn, xs, res, gamma, True, _workspace(arn, rows), opts=dict(parts=parts))
    b = _run(arn, xs, res, gamma, True, _workspace(arn, rows),
             opts=dict(parts=parts, spin_polls=-1))
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_counts_stay_in_step_across_shapes(arn):
    """One workspace, calls of several row counts and part counts: after each
    call every slot of every row carries the number of calls with two or more
    parts that touched the row (one part runs the row kernel and leaves the
    workspace alone), and every result equals the one from a fresh
    workspace."""
    cols, P = 4096, 4
    ws = _workspace(arn, 64)
    calls = {}
    for rows, parts in ((8, 8), (3, 2), (64, 1), (5, 4), (8, 8), (1, 8), (64, 2), (2, 3)):
        xs, res, gamma = _case(rows * 31 + parts, rows, cols, P, "in_out")
        got = _run(arn, xs, res, gamma, True, ws, opts=dict(parts=parts))
        fresh = _run(arn, xs, res, gamma, True, _workspace(arn, rows), opts=dict(parts=parts))
        for u, v in zip(got, fresh):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), (rows, parts)
        for r in range(rows if parts > 1 else 0):
            calls[r] = calls.get(r, 0) + 1
        counts = (ws.view(64, 8, 2) >> 32).cpu().numpy()
        for r in range(64):
            assert np.all(counts[r] == calls.get(r, 0)), (rows, parts, r, counts[r])


def test_graph_replay_matches_eager(arn):
    """One split call captured in a graph: every replay (eager work and a
    synchronisation between replays) equals the eager result bitwise, and the
    workspace counts advance by one per replay."""
    rows, cols, P = 4, 8192, 8
    xs, res, gamma = _case(5, rows, cols, P, "in_out")
    xs_d = [x.to(DEV) for x in xs]
    res_d, g_d = res.to(DEV), gamma.to(DEV)
    ws = _workspace(arn, rows)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows,), dtype=torch.float32, device=DEV)
    ro = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)

    def call():
        arn.arnfp8_run_split(xs_d, res_d, ro, out, sc, g_d, 1e-5, 1.0, 1200.0, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, sc, ro)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    before = int((ws.view(rows, 8, 2)[0, 0, 0] >> 32).item())
    for k in range(3):
        out.fill_(0x7F)
        sc.fill_(-1.0)
        ro.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(sc, eager[1]) and torch.equal(ro, eager[2]), k
        _ = (xs_d[0].float() * 2.0).sum().item()
    counts = (ws.view(rows, 8, 2) >> 32).cpu().numpy()
    assert np.all(counts == before + 3)


def test_repeat_calls_bitwise_deterministic(arn):
    rows, cols, P = 16, 7168, 8
    xs, res, gamma = _case(9, rows, cols, P, "in_out")
    ws = _workspace(arn, rows)
    first = _run(arn, xs, res, gamma, True, ws)
    for _ in range(20):
        again = _run(arn, xs, res, gamma, True, ws)
        for u, v in zip(first, again):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_refusals_before_launch(arn):
    rows, cols = 4, 1024
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    res = torch.zeros_like(x)
    out = torch.full((rows, cols), 0x11, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows,), -1.0, dtype=torch.float32, device=DEV)
    g = torch.ones((cols,), dtype=torch.bfloat16, device=DEV)
    ws = _workspace(arn, rows)

    def status(**kw):
        args = dict(inputs=[x], residual_in=res, residual_out=torch.empty_like(x), workspace=ws,
                    opts=None)
        args.update(kw)
        try:
            arn.arnfp8_run_split(args["inputs"], args["residual_in"], args["residual_out"], out,
                                 sc, g, 1e-6, 0.0, 1.0, workspace=args["workspace"],
                                 workspace_bytes=args.get("workspace_bytes"), opts=args["opts"])
            return 0
        except arn.ArnFp8Error as e:
            return e.status

    assert status(residual_out=res) == 5                   # in place refused
    assert status(workspace_bytes=rows * 128 - 8) == 11    # too small
    assert status(workspace=int(ws.data_ptr()) + 8) == 2   # misaligned
    assert status(workspace=res) == 5                      # overlaps an input
    assert status(opts=dict(parts=9)) == 7
    assert status(opts=dict(parts=-1)) == 7
    torch.cuda.synchronize()
    assert torch.all(out == 0x11) and torch.all(sc == -1.0)


@pytest.mark.parametrize("rows,cols,P,parts", [(4, 256, 2, 0), (300, 7168, 8, 0), (9, 4096, 4, 1)])
def test_one_part_runs_the_row_kernel(arn, rows, cols, P, parts):
    """One part per row (automatic for rows under 128 chunks and for larger
    batches, or asked for): the result bits are arnfp8_run's and the workspace
    is not written."""
    xs, res, gamma = _case(3 * rows + cols, rows, cols, P, "in_out")
    ws = torch.full((max(16, arn.arnfp8_split_workspace_bytes(rows)) // 8,), 77, dtype=torch.int64,
                    device=DEV)
    got = _run(arn, xs, res, gamma, True, ws, opts=dict(parts=parts))
    out = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows,), dtype=torch.float32, device=DEV)
    ro = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    arn.arnfp8_run([x.to(DEV) for x in xs], res.to(DEV), ro, out, sc, gamma.to(DEV), 1e-6, 0.0,
                   1200.0)
    torch.cuda.synchronize()
    for u, v in zip(got, (out, sc, ro)):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))
    assert torch.all(ws == 77)


def test_two_streams_with_their_own_workspaces(arn):
    """Split calls running at the same time on two streams, each with its own
    workspace, give the bits of the same calls run one after the other."""
    rows, cols, P = 16, 8192, 8
    cases = [_case(41 + k, rows, cols, P, "in_out") for k in range(2)]
    dev_cases = [([x.to(DEV) for x in xs], res.to(DEV), g.to(DEV)) for xs, res, g in cases]
    wss = [_workspace(arn, rows) for _ in range(2)]
    outs = [(torch.empty((rows, cols), dtype=torch.uint8, device=DEV),
             torch.empty((rows,), dtype=torch.float32, device=DEV),
             torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)) for _ in range(2)]
    seq = []
    for (xs, res, g), ws in zip(dev_cases, wss):
        o = (torch.empty((rows, cols), dtype=torch.uint8, device=DEV),
             torch.empty((rows,), dtype=torch.float32, device=DEV),
             torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV))
        arn.arnfp8_run_split(xs, res, o[2], o[0], o[1], g, 1e-6, 0.0, 1200.0, workspace=ws)
        torch.cuda.synchronize()
        seq.append(o)
    streams = [torch.cuda.Stream() for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(10):
        for (xs, res, g), ws, o, s in zip(dev_cases, wss, outs, streams):
            with torch.cuda.stream(s):
                arn.arnfp8_run_split(xs, res, o[2], o[0], o[1], g, 1e-6, 0.0, 1200.0,
                                     workspace=ws)
    torch.cuda.synchronize()
    for o, want in zip(outs, seq):
        for u, v in zip(o, want):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))
