"""The allocation-free split call (arnfp8_run_split_noalloc) against the split
call with a workspace of the caller's (arnfp8_run_split): same kernels, so the
outputs must agree bit for bit (stricter than the oracle bar of bf16
bit-exact, scales within 1e-5, codes within one step).

The calls run back to back on the library's one per-device array: a larger
call, then a smaller one, then one at the row limit with other part counts, so
the per-row counts the array keeps between calls are exercised across shapes.
Rows beyond the limit are refused before anything is launched.
"""
import ctypes

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


def _case(seed, rows, cols, P, std=0.5):
    g = torch.Generator().manual_seed(seed)
    xs = [(torch.randn((rows, cols), generator=g) * std).to(torch.bfloat16).to(DEV)
          for _ in range(P)]
    res = torch.randn((rows, cols), generator=g).to(torch.bfloat16).to(DEV)
    gamma = (torch.rand((cols,), generator=g) * 0.4 + 0.8).to(torch.bfloat16).to(DEV)
    return xs, res, gamma


def _outputs(rows, cols):
    return (torch.full((rows, cols), 0x7F, dtype=torch.uint8, device=DEV),
            torch.full((rows,), -1.0, dtype=torch.float32, device=DEV),
            torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV))


def _same(a, b):
    return all(torch.equal(u.view(torch.uint8), v.view(torch.uint8)) for u, v in zip(a, b))


# (rows, cols, P, parts): the second call is smaller than the first.
CALLS = [(96, 7168, 8, 0), (1, 8192, 8, 0), (4096, 1024, 2, 2), (7, 7176, 3, 4)]


def test_noalloc_matches_split_with_a_workspace(arn):
    print(f"[noalloc] calls {CALLS}", flush=True)
    results = []
    for rows, cols, P, parts in CALLS:
        xs, res, gamma = _case(rows + cols + P, rows, cols, P)
        got = _outputs(rows, cols)
        arn.arnfp8_run_split_noalloc(xs, res, got[2], got[0], got[1], gamma, 1e-6, 0.0, 1200.0,
                                     opts=dict(parts=parts))
        results.append((xs, res, gamma, got, parts))
    torch.cuda.synchronize()
    for (rows, cols, P, _), (xs, res, gamma, got, parts) in zip(CALLS, results):
        want = _outputs(rows, cols)
        ws = torch.zeros((arn.arnfp8_split_workspace_bytes(rows) // 8,), dtype=torch.int64,
                         device=DEV)
        arn.arnfp8_run_split(xs, res, want[2], want[0], want[1], gamma, 1e-6, 0.0, 1200.0,
                             workspace=ws, opts=dict(parts=parts))
        torch.cuda.synchronize()
        assert _same(got, want), (rows, cols, P, parts)


def test_noalloc_repeated_calls_stay_exact(arn):
    """Many calls on the shared array, alternating shapes: every result equals
    the first result of its shape."""
    shapes = [(32, 7168, 4), (3, 4096, 8)]
    cases = [_case(17 * r + c, r, c, P) for r, c, P in shapes]
    first = []
    for (rows, cols, P), (xs, res, gamma) in zip(shapes, cases):
        o = _outputs(rows, cols)
        arn.arnfp8_run_split_noalloc(xs, res, o[2], o[0], o[1], gamma, 1e-5, 1.0, 1200.0)
        first.append(o)
    torch.cuda.synchronize()
    for k in range(10):
        i = k % 2
        rows, cols, P = shapes[i]
        xs, res, gamma = cases[i]
        o = _outputs(rows, cols)
        arn.arnfp8_run_split_noalloc(xs, res, o[2], o[0], o[1], gamma, 1e-5, 1.0, 1200.0)
        torch.cuda.synchronize()
        assert _same(o, first[i]), (k, shapes[i])


def test_noalloc_refuses_rows_beyond_the_limit(arn):
    rows, cols = arn.NOALLOC_MAX_ROWS + 1, 64
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    out = torch.full((rows, cols), 0x11, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows,), -1.0, dtype=torch.float32, device=DEV)
    g = torch.ones((cols,), dtype=torch.bfloat16, device=DEV)
    L = arn.library()
    inputs = (ctypes.c_void_p * 1)(x.data_ptr())
    st = L.arnfp8_run_split_noalloc(inputs, None, None, out.data_ptr(), sc.data_ptr(),
                                    g.data_ptr(), 1e-6, 0.0, 1.0, rows, cols, 1,
                                    torch.cuda.current_stream().cuda_stream, None)
    assert st == 11
    assert "ARNFP8_NOALLOC_MAX_ROWS" in arn.arnfp8_status_string(st)
    assert L.arnfp8_run_split_noalloc(inputs, None, None, None, None, None, 1e-6, 0.0, 1.0, 0,
                                      cols, 1, None, None) == 0
    torch.cuda.synchronize()
    assert torch.all(out == 0x11) and torch.all(sc == -1.0)


def test_noalloc_in_a_graph_matches_eager(arn):
    """An allocation-free call captured in a graph (after eager calls on the
    device): every replay, with eager work and synchronisations between
    replays, equals the eager result bit for bit."""
    rows, cols, P = 8, 8192, 8
    xs, res, gamma = _case(123, rows, cols, P)
    o = _outputs(rows, cols)

    def call():
        arn.arnfp8_run_split_noalloc(xs, res, o[2], o[0], o[1], gamma, 1e-6, 0.0, 1200.0)

    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in o]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for k in range(3):
        o[0].fill_(0x7F)
        o[1].fill_(-1.0)
        o[2].fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert _same(o, eager), k
        _ = (xs[0].float() * 3.0).sum().item()
