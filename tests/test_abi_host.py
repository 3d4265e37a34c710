"""Host-side checks of the C ABI library (no GPU needed, no kernel launched).

The library must load, export every function ``include/arnfp8.h`` declares,
and reject bad arguments with the documented status codes before touching
the device.  Pointers below are fake addresses: validation reads none of them.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

OK, NULLP, MISALIGNED, BAD_SHAPE, BAD_P, ALIAS = 0, 1, 2, 3, 4, 5
BAD_SCALAR, BAD_WORKSPACE = 10, 11


@pytest.fixture(scope="module")
def L():
    import all_reduce_rmsnorm_amd as arn

    if not os.path.exists(arn.library_path()):
        from all_reduce_rmsnorm_amd import build

        build.build()
    return arn.library()


def declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M):
            names.append(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("arnfp8_run", "arn_sum_bf16", "arnfp8_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} is declared in include/ but not exported"


def test_library_is_built_for_gfx950():
    """The offload bundle of the library built here names the gfx950 target."""
    import all_reduce_rmsnorm_amd as arn

    blob = open(arn.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings(L):
    import all_reduce_rmsnorm_amd as arn

    for code in range(0, 12):
        s = arn.arnfp8_status_string(code)
        assert s and s != "unknown status"
    assert arn.arnfp8_status_string(99) == "unknown status"


def _arr(*ptrs):
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)


BASE = 1 << 40  # fake, well separated, 16-byte aligned addresses
MB = 1 << 20


def run(L, inputs, res_in=None, res_out=None, out=BASE + 100 * MB, scales=BASE + 200 * MB,
        gamma=BASE + 300 * MB, rows=4, cols=256, P=None):
    P = len(inputs) if P is None else P
    return L.arnfp8_run(_arr(*inputs) if inputs is not None else None, res_in, res_out, out, scales,
                        gamma, 1e-6, 0.0, 1.0, rows, cols, P, None)


def test_fused_validation_codes(L):
    x0, x1 = BASE, BASE + 10 * MB
    assert run(L, [x0, x1], cols=255) == BAD_SHAPE
    assert run(L, [x0, x1], cols=0) == BAD_SHAPE
    assert run(L, [x0, x1], rows=-1) == BAD_SHAPE
    assert run(L, [x0, x1], cols=65544) == BAD_SHAPE
    assert run(L, [x0, x1], rows=1 << 62, cols=65536) == BAD_SHAPE
    assert run(L, [x0, x1], P=0) == BAD_P
    assert run(L, [x0] * 9) == BAD_P
    assert run(L, None, P=2) == NULLP
    assert run(L, [x0, None]) == NULLP
    assert run(L, [x0, x1], out=None) == NULLP
    assert run(L, [x0, x1], scales=None) == NULLP
    assert run(L, [x0, x1], gamma=None) == NULLP
    assert run(L, [x0 + 8, x1]) == MISALIGNED
    assert run(L, [x0, x1], out=BASE + 100 * MB + 4) == MISALIGNED
    assert run(L, [x0, x1], gamma=BASE + 300 * MB + 2) == MISALIGNED
    assert run(L, [x0, x1], scales=BASE + 200 * MB + 2) == MISALIGNED
    assert run(L, [x0, x1], res_in=BASE + 400 * MB + 8) == MISALIGNED


def test_fused_alias_rules(L):
    x0, x1 = BASE, BASE + 10 * MB
    r = BASE + 400 * MB
    n = 4 * 256
    # (res_out == res_in is legal; it is not called here, as a legal call launches)
    # outputs overlapping inputs
    assert run(L, [x0, x1], out=x1 + 2 * n - 16) == ALIAS
    assert run(L, [x0, x1], res_out=x0) == ALIAS
    assert run(L, [x0, x1], scales=BASE + 300 * MB) == ALIAS  # scales on gamma
    assert run(L, [x0, x1], res_in=r, res_out=r + 16) == ALIAS  # partial overlap with residual_in
    # outputs overlapping each other
    assert run(L, [x0, x1], res_out=BASE + 100 * MB) == ALIAS
    assert run(L, [x0, x1], scales=BASE + 100 * MB + n - 4) == ALIAS


def test_rows_zero_returns_ok_without_touching_anything(L):
    assert run(L, [BASE, BASE + 10 * MB], rows=0, out=None, scales=None, gamma=None) == OK
    assert L.arn_sum_bf16(_arr(BASE), None, 0, 64, 1, None) == OK


def test_sum_validation_codes(L):
    x0, x1 = BASE, BASE + 10 * MB
    out = BASE + 100 * MB
    assert L.arn_sum_bf16(_arr(x0, x1), out, 4, 12, 2, None) == BAD_SHAPE
    assert L.arn_sum_bf16(_arr(x0, x1), out, 4, 64, 9, None) == BAD_P
    assert L.arn_sum_bf16(_arr(x0, x1), None, 4, 64, 2, None) == NULLP
    assert L.arn_sum_bf16(_arr(x0, x1), out + 2, 4, 64, 2, None) == MISALIGNED
    assert L.arn_sum_bf16(_arr(x0, x1), x1 + 16, 4, 64, 2, None) == ALIAS


def test_binding_raises_with_status(L):
    import all_reduce_rmsnorm_amd as arn

    with pytest.raises(arn.ArnFp8Error) as e:
        arn.arn_sum_bf16([BASE, BASE + 10 * MB], BASE + 100 * MB, rows=4, cols=12, stream=0)
    assert e.value.status == BAD_SHAPE


def test_algorithmic_bytes_of_the_workloads():
    from all_reduce_rmsnorm_amd import synth

    W = synth.WORKLOADS
    assert W["tiny_p2_4x256"].algorithmic_bytes() == 5648
    assert W["sum_p4_64x4096"].algorithmic_bytes() == 2621440
    assert W["decode_p4_32x7168"].algorithmic_bytes() == 2996352
    assert W["unit_offset_p8_128x8192"].algorithmic_bytes() == 22036992
    assert W["prefill_p8_8192x7168"].algorithmic_bytes() == 1233172480


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "all_reduce_rmsnorm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", text).lower() or f == "synth.py", f


def test_stage_bytes_agrees_with_the_oracle(L):
    import oracle

    for rows in (0, 1, 5, 33, 1000, 8192):
        for cols in (8, 24, 2880, 7168):
            for ngpus in (1, 2, 3, 4, 8):
                assert L.arnfp8_stage_bytes(rows, cols, ngpus) == oracle.stage_bytes(rows, cols, ngpus)
    assert L.arnfp8_stage_bytes(-1, 8, 1) == -1
    assert L.arnfp8_stage_bytes(4, 0, 1) == -1
    assert L.arnfp8_stage_bytes(4, 8, 0) == -1


def test_share_validation_codes(L):
    x0, x1 = BASE, BASE + 10 * MB
    stg, g = BASE + 100 * MB, BASE + 300 * MB

    def share(ngpus, rank, staging=stg, rows=16, cols=256, inputs=(x0, x1), gamma=g):
        return L.arnfp8_run_share(_arr(*inputs), None, None, staging, gamma, 1e-6, 0.0, 1.0,
                                  rows, cols, len(inputs), ngpus, rank, None)

    assert share(0, 0) == 8
    assert share(4, 4) == 8
    assert share(4, -1) == 8
    assert share(4, 1, staging=None) == NULLP
    assert share(4, 1, staging=stg + 8) == MISALIGNED
    assert share(4, 1, staging=x1 + 512) == ALIAS
    assert share(4, 1, gamma=None) == NULLP
    assert share(4, 1, cols=12) == BAD_SHAPE
    # an empty share validates and returns OK without launching
    assert share(8, 7, rows=5) == OK


def test_bad_launch_options_rejected_without_device(L):
    import all_reduce_rmsnorm_amd as arn

    x0, x1 = BASE, BASE + 10 * MB
    for bad in (arn.Launch(threads=96), arn.Launch(threads=1024, vpt=2), arn.Launch(vpt=3),
                arn.Launch(threads=64, vpt=1), arn.Launch(grid=-1), arn.Launch(variant=9),
                arn.Launch(threads=512, vpt=2, grid=2**31 - 1), arn.Launch(stores=3)):
        st = L.arnfp8_run_ex(_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 200 * MB,
                             BASE + 300 * MB, 1e-6, 0.0, 1.0, 4, 1024, 2, None, ctypes.byref(bad))
        assert st == 7, (bad.threads, bad.vpt, bad.grid, bad.variant)
    st = L.arnfp8_run_fmt(_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 200 * MB,
                          BASE + 300 * MB, 1e-6, 0.0, 1.0, 4, 1024, 2, 5, None, None)
    assert st == 9
    st = L.arnfp8_run_fmt(_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 200 * MB,
                          BASE + 300 * MB, 1e-6, 0.0, 1.0, 4, 1000, 2, 2, None, None)
    assert st == BAD_SHAPE  # MXFP8 needs cols % 32 == 0


def test_binding_refuses_what_the_library_cannot_read():
    import torch

    import all_reduce_rmsnorm_amd as arn

    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    out = torch.zeros((4, 64), dtype=torch.uint8)
    s = torch.zeros((4,), dtype=torch.float32)
    g = torch.zeros((64,), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        arn.arnfp8_run([x[:, 8:]], None, None, out, s, g, 1e-6, 0.0, 1.0, rows=4, cols=56)
    with pytest.raises(TypeError, match="dtype"):
        arn.arnfp8_run([x.float()], None, None, out, s, g, 1e-6, 0.0, 1.0)
    with pytest.raises(TypeError, match="dtype"):
        arn._ptr(s.double(), arn._F32, "scales")
    with pytest.raises(ValueError, match="device"):
        arn.arnfp8_run([x], None, None, out, s, g, 1e-6, 0.0, 1.0)


def test_binding_refuses_buffers_smaller_than_the_shape():
    import torch

    import all_reduce_rmsnorm_amd as arn

    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    out = torch.zeros((4, 64), dtype=torch.uint8)
    s = torch.zeros((4,), dtype=torch.float32)
    g = torch.zeros((64,), dtype=torch.bfloat16)
    cases = [
        ("out_fp8", dict(out_fp8=out[:3])),
        ("scales", dict(scales=s[:3])),
        ("gamma", dict(gamma=g[:56])),
        ("residual_out", dict(residual_out=x[:3])),
        ("inputs[1]", dict(inputs=[x, x[:2]])),
    ]
    for what, change in cases:
        args = dict(inputs=[x], residual_in=None, residual_out=None, out_fp8=out, scales=s,
                    gamma=g)
        args.update(change)
        with pytest.raises(ValueError, match=r"\b" + what.replace("[", r"\[").replace("]", r"\]")
                           + " holds"):
            arn.arnfp8_run(args["inputs"], args["residual_in"], args["residual_out"],
                           args["out_fp8"], args["scales"], args["gamma"], 1e-6, 0.0, 1.0,
                           rows=4, cols=64)
    mx = torch.zeros((4, 1), dtype=torch.uint8)  # needs 4 x (64 / 32) bytes
    with pytest.raises(ValueError, match="scales holds"):
        arn.arnfp8_run_fmt([x], None, None, out, mx, g, 1e-6, 0.0, 1.0, out_format=arn.FMT_MXFP8)
    with pytest.raises(ValueError, match="out holds"):
        arn.arn_sum_bf16([x], x[:2])
    with pytest.raises(ValueError, match="staging holds"):
        arn.arnfp8_run_share([x], None, None, torch.zeros(8, dtype=torch.uint8), g, 1e-6, 0.0,
                             1.0, ngpus=2, rank=0)
    with pytest.raises(ValueError, match="out holds"):
        arn.arnfp8_convert_f32(torch.zeros(16), torch.zeros(8, dtype=torch.uint8), arn.FMT_E4M3FN)


NAN, INF = float("nan"), float("inf")


@pytest.mark.parametrize("eps,woff,ub", [(-1e-6, 0.0, 1.0), (NAN, 0.0, 1.0), (INF, 0.0, 1.0),
                                         (1e-6, NAN, 1.0), (1e-6, -INF, 1.0), (1e-6, 0.0, 0.0),
                                         (1e-6, 0.0, -3.0), (1e-6, 0.0, NAN)])
def test_bad_scalars_rejected_before_launch(L, eps, woff, ub):
    """eps must be finite and >= 0, weight_offset finite, scale_ub > 0; the
    check comes before the rows == 0 shortcut, so no call here launches."""
    x0, x1 = BASE, BASE + 10 * MB
    args = (_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 200 * MB, BASE + 300 * MB,
            eps, woff, ub)
    for rows in (0, 4):
        assert L.arnfp8_run(*args, rows, 256, 2, None) == BAD_SCALAR
        assert L.arnfp8_run_ex(*args, rows, 256, 2, None, None) == BAD_SCALAR
        assert L.arnfp8_run_fmt(*args, rows, 256, 2, 1, None, None) == BAD_SCALAR
        assert L.arnfp8_run_share(_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 300 * MB,
                                  eps, woff, ub, rows, 256, 2, 4, 1, None) == BAD_SCALAR
    # the MX output has no scale_ub: only eps and the offset are checked
    only_ub_bad = eps == 1e-6 and woff == 0.0
    mx = L.arnfp8_run_fmt(*args, 0, 256, 2, 2, None, None)
    assert mx == (OK if only_ub_bad else BAD_SCALAR)


def test_good_scalar_edges_are_accepted(L):
    """eps = 0, scale_ub = +inf and large finite values pass validation (rows
    = 0: nothing is launched)."""
    x0, x1 = BASE, BASE + 10 * MB
    for eps, woff, ub in ((0.0, 0.0, 1.0), (1e-6, 0.0, INF), (3e38, -3e38, 1e-30)):
        assert L.arnfp8_run(_arr(x0, x1), None, None, BASE + 100 * MB, BASE + 200 * MB,
                            BASE + 300 * MB, eps, woff, ub, 0, 256, 2, None) == OK


def test_split_workspace_bytes(L):
    """Two 64-bit words for each of 8 slots per row; negative or overflowing
    row counts give -1."""
    assert L.arnfp8_split_workspace_bytes(0) == 0
    assert L.arnfp8_split_workspace_bytes(1) == 128
    assert L.arnfp8_split_workspace_bytes(37) == 37 * 128
    assert L.arnfp8_split_workspace_bytes(-1) == -1
    assert L.arnfp8_split_workspace_bytes(1 << 60) == -1


def test_split_validation_codes(L):
    """arnfp8_run_split refuses before any launch: bad shapes, scalars and part
    counts first (also at rows = 0), then the buffers, then the workspace."""
    import all_reduce_rmsnorm_amd as arn

    x0, x1 = BASE, BASE + 10 * MB
    out, sc, g = BASE + 100 * MB, BASE + 200 * MB, BASE + 300 * MB
    ws = BASE + 500 * MB

    def split(rows=4, cols=1024, res_in=None, res_out=None, workspace=ws, wbytes=None,
              parts=2, eps=1e-6, ub=1.0, inputs=(x0, x1), gamma=g):
        wbytes = 128 * max(rows, 0) if wbytes is None else wbytes
        opt = arn.SplitOpts(parts=parts, spin_polls=0)
        return L.arnfp8_run_split(_arr(*inputs), res_in, res_out, out, sc, gamma, eps, 0.0, ub,
                                  rows, cols, len(inputs), workspace, wbytes, None,
                                  ctypes.byref(opt))

    for rows in (0, 4):
        assert split(rows=rows, cols=12) == BAD_SHAPE
        assert split(rows=rows, eps=-1.0) == BAD_SCALAR
        assert split(rows=rows, ub=0.0) == BAD_SCALAR
        assert split(rows=rows, parts=9) == 7
        assert split(rows=rows, parts=-1) == 7
        assert split(rows=rows, cols=65536, parts=1) == 7  # 8192 chunks > 1024 lanes
    assert split(inputs=()) == BAD_P
    assert split(rows=0, workspace=None) == OK
    assert split(gamma=None) == NULLP
    assert split(workspace=None) == NULLP
    assert split(workspace=ws + 8) == MISALIGNED
    assert split(wbytes=4 * 128 - 8) == BAD_WORKSPACE
    r = BASE + 400 * MB
    assert split(res_in=r, res_out=r) == ALIAS            # no in-place residual
    assert split(workspace=x1 + 1024) == ALIAS            # workspace on an input
    assert split(workspace=out + 16) == ALIAS             # workspace on the output
    assert split(workspace=sc - 64) == ALIAS              # workspace runs into the scales
    assert split(res_out=r, workspace=r + 4 * 1024 * 2 - 16) == ALIAS


def test_noalloc_split_refuses_before_touching_the_device(L):
    """Rows beyond ARNFP8_NOALLOC_MAX_ROWS give BAD_WORKSPACE after the shape
    check; rows = 0 validates and returns OK (no device is looked at)."""
    import all_reduce_rmsnorm_amd as arn

    x0, x1 = BASE, BASE + 10 * MB
    out, sc, g = BASE + 100 * MB, BASE + 200 * MB, BASE + 300 * MB

    def noalloc(rows, cols=256, eps=1e-6, parts=0):
        opt = arn.SplitOpts(parts=parts, spin_polls=0)
        return L.arnfp8_run_split_noalloc(_arr(x0, x1), None, None, out, sc, g, eps, 0.0, 1.0,
                                          rows, cols, 2, None, ctypes.byref(opt))

    assert arn.NOALLOC_MAX_ROWS == 4096
    assert noalloc(arn.NOALLOC_MAX_ROWS + 1) == BAD_WORKSPACE
    assert noalloc(arn.NOALLOC_MAX_ROWS + 1, cols=12) == BAD_SHAPE
    assert noalloc(-1) == BAD_SHAPE
    assert noalloc(0) == OK
    assert noalloc(0, eps=-1.0) == BAD_SCALAR
    assert noalloc(0, parts=9) == 7
    # rows > 0: every argument is checked before the library's array is looked up
    assert noalloc(4, parts=9) == 7
    assert noalloc(4, cols=65536, parts=1) == 7
    assert L.arnfp8_run_split_noalloc(_arr(x0, x1), None, None, out, sc, None, 1e-6, 0.0, 1.0,
                                      4, 256, 2, None, None) == NULLP
    assert L.arnfp8_run_split_noalloc(_arr(x0, x1), None, None, out + 8, sc, g, 1e-6, 0.0, 1.0,
                                      4, 256, 2, None, None) == MISALIGNED
    r = BASE + 400 * MB
    assert L.arnfp8_run_split_noalloc(_arr(x0, x1), r, r, out, sc, g, 1e-6, 0.0, 1.0,
                                      4, 256, 2, None, None) == ALIAS
    assert L.arnfp8_run_split_noalloc(_arr(x0, x1), None, x1, out, sc, g, 1e-6, 0.0, 1.0,
                                      4, 256, 2, None, None) == ALIAS


def test_split_parts_rule_without_a_device(L):
    """The automatic part count: the largest power of two up to 8 with rows x
    parts within the compute units (256 assumed when no device answers) and
    at least 64 chunks per part, and enough parts for 1024 lanes each."""
    import all_reduce_rmsnorm_amd as arn

    try:
        import torch

        if torch.cuda.is_available():
            pytest.skip("the device's own compute-unit count applies")
    except ImportError:
        pass
    assert arn.arnfp8_split_parts(1, 8192) == 8
    assert arn.arnfp8_split_parts(1, 7168) == 8        # 896 chunks: 8 parts of 112
    assert arn.arnfp8_split_parts(32, 7168) == 8
    assert arn.arnfp8_split_parts(64, 7168) == 4
    assert arn.arnfp8_split_parts(128, 8192) == 2
    assert arn.arnfp8_split_parts(300, 7168) == 1
    assert arn.arnfp8_split_parts(4, 256) == 1         # 32 chunks: under one wave per part
    assert arn.arnfp8_split_parts(1, 1024) == 2        # 128 chunks: two parts of 64
    assert arn.arnfp8_split_parts(1000, 65536) == 8    # 8192 chunks need 8 parts of 1024
    assert arn.arnfp8_split_parts(0, 256) == -1
    assert arn.arnfp8_split_parts(4, 12) == -1
