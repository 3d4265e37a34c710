"""Pin strength: plant a plausible mistake in a copy of the oracle (on the CPU)
and check that the pin suite rejects every such mutant.

Each mutant is the oracle's C source with one textual change, compiled with the
oracle's own gcc flags into a temporary directory; the pin tests are then run
in a subprocess against that library (``ARNFP8_ORACLE_LIB``) and must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "arnfp8_oracle.c")
PIN_FILES = ["tests/test_oracle_sum.py", "tests/test_oracle_norm.py", "tests/test_oracle_codecs.py",
             "tests/test_oracle_quant_variants.py", "tests/test_oracle_share.py"]

MUTANTS = {
    "bf16_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "bf16_truncate": ("dropped > 0x8000u ||", "0 &&"),
    "acc_from_zero": ("float acc = oracle_bf16_to_f32(inputs[0][k]);\n    for (int p = 1;",
                      "float acc = 0.0f;\n    for (int p = 0;"),
    "reverse_rank_order": ("float acc = oracle_bf16_to_f32(inputs[0][k]);\n    for (int p = 1; p < P; ++p)\n        acc = acc + oracle_bf16_to_f32(inputs[p][k]);",
                           "float acc = oracle_bf16_to_f32(inputs[P - 1][k]);\n    for (int p = P - 2; p >= 0; --p)\n        acc = acc + oracle_bf16_to_f32(inputs[p][k]);"),
    "residual_not_rounded_once": ("hb = oracle_f32_to_bf16(t);", "hb = oracle_f32_to_bf16(t + 1e-3f * t);"),
    "drop_eps": ("double den = ms + (double)eps;", "double den = ms;"),
    "sum_not_mean": ("double ms = sumsq / (double)cols;", "double ms = sumsq;"),
    "gamma_reversed": ("oracle_bf16_to_f32(gamma[j])", "oracle_bf16_to_f32(gamma[cols - 1 - j])"),
    "drop_weight_offset": ("oracle_bf16_to_f32(gamma[j]) + weight_offset;", "oracle_bf16_to_f32(gamma[j]);"),
    "drop_scale_clamp": ("fminf(amax, scale_ub)", "amax"),
    "drop_scale_floor": ("1.0f / (fmax * 512.0f)", "0.0f"),
    "fnuz_max_240": ("const float fmax = e5m2 ? 57344.0f : 448.0f;", "const float fmax = e5m2 ? 57344.0f : 240.0f;"),
    "fp8_ties_away": ("(frac == 0.5 && fmod(lo, 2.0) == 1.0)", "(frac == 0.5)"),
    "fp8_wrong_subnormal_edge": ("round_to_grid(a, -6, 3)", "round_to_grid(a, -7, 3)"),
    "sign_dropped": ("y[j] = h[j] * r * (double)g;", "y[j] = fabs(h[j]) * r * (double)g;"),
    "e5m2_wrong_subnormal_edge": ("round_to_grid(a, -14, 2)", "round_to_grid(a, -15, 2)"),
    "e5m2_uses_e4m3_max": ("const float fmax = e5m2 ? 57344.0f : 448.0f;", "const float fmax = 448.0f;"),
    "mx_emax_7": ("int e = (k - 1) - 8;", "int e = (k - 1) - 7;"),
    "mx_zero_block_exp_0": ("        return -127;\n    int k;", "        return 0;\n    int k;"),
    "mx_amax_of_half_block": ("for (int i = 0; i < n; ++i)\n        if (fabs(v[i]) > amax)",
                              "for (int i = 0; i < n / 2; ++i)\n        if (fabs(v[i]) > amax)"),
    "share_floor_not_ceil": ("int64_t S = (rows + ngpus - 1) / ngpus;\n    int64_t lo", "int64_t S = rows / ngpus + 1;\n    int64_t lo"),
    "stage_no_padding": ("(scale_bytes + simd_width - 1) / simd_width * simd_width", "scale_bytes"),
    "rsqrt_not_inverse": ("1.0 / sqrt(den)", "1.0 / den"),
    "eps_zero_row_nan": ("double r = den > 0.0 ? 1.0 / sqrt(den) : 0.0;", "double r = 1.0 / sqrt(den);"),
    "accept_negative_eps": ("!isfinite(eps) || eps < 0.0f ||", "!isfinite(eps) ||"),
    "accept_nonfinite_eps": ("!isfinite(eps) || eps < 0.0f ||", "eps < 0.0f ||"),
    "accept_nonpositive_ub": ("if (check_ub && !(scale_ub > 0.0f))", "if (check_ub && scale_ub < 0.0f)"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique / missing"
    mdir = tmp_path / name
    mdir.mkdir()
    csrc = mdir / "arnfp8_oracle.c"
    csrc.write_text(src.replace(old, new))
    (mdir / "arnfp8_oracle.h").write_text(open(SRC.replace(".c", ".h")).read())
    sys.path.insert(0, ROOT)
    import oracle

    lib = mdir / "liboracle_mutant.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-w", "-o", str(lib), str(csrc), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    env = dict(os.environ, ARNFP8_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pin suite:\n{r.stdout[-2000:]}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same procedure with no change passes."""
    MUTANTS["__none__"] = ("#include <math.h>", "#include <math.h>")
    try:
        lib = _build_mutant(tmp_path, "__none__")
    finally:
        del MUTANTS["__none__"]
    env = dict(os.environ, ARNFP8_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
