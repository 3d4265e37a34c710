"""The C ABI from plain C: include/arnfp8.h compiles as C99 with gcc -Wall
-Werror, links against libarnfp8.so, and its validation paths return the
documented codes (no launch, no GPU needed)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_compiles_as_c99_and_validation_codes_hold(tmp_path):
    import all_reduce_rmsnorm_amd as arn

    lib = arn.library_path()
    if not os.path.exists(lib):
        pytest.skip("libarnfp8.so is not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(rocm, 'include')}",
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe),
           f"-L{os.path.dirname(lib)}", "-larnfp8", f"-Wl,-rpath,{os.path.dirname(lib)}",
           f"-L{os.path.join(rocm, 'lib')}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout


def test_gpu_round_trip_program_builds(tmp_path):
    """The plain-C GPU round trip (run by the GPU suite) compiles and links
    here too, with gcc -Werror."""
    from tests.test_gpu_c_roundtrip import build_roundtrip

    build_roundtrip(tmp_path / "gpu_roundtrip")
    assert (tmp_path / "gpu_roundtrip").exists()
