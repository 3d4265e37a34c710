"""The C ABI from a plain C program on the GPU (no Python, no PyTorch in the
process): hipMalloc'd buffers, arnfp8_run and arn_sum_bf16 on the null stream,
results against the CPU oracle linked into the same program."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build_roundtrip(out_path):
    import all_reduce_rmsnorm_amd as arn

    lib = arn.library_path()
    if not os.path.exists(lib):
        pytest.fail("libarnfp8.so is not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'oracle')}", f"-I{os.path.join(rocm, 'include')}",
           os.path.join(ROOT, "tests", "c", "gpu_roundtrip.c"),
           os.path.join(ROOT, "oracle", "arnfp8_oracle.c"), "-o", str(out_path),
           f"-L{os.path.dirname(lib)}", "-larnfp8", f"-Wl,-rpath,{os.path.dirname(lib)}",
           f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_round_trip(tmp_path):
    exe = tmp_path / "gpu_roundtrip"
    build_roundtrip(exe)
    print("[c] gpu_roundtrip 37 x 7176, P = 5: fused, sum, split, allocation-free split", flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu_roundtrip: ok" in r.stdout
