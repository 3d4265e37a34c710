"""CPU checks of the input recipe and of bench.py's host logic (no GPU)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_outlier_mask_is_shared_and_clamps_rows(orc):
    """The prefill recipe multiplies the same 0.1 % of [rows, cols] positions
    by 100 in every slab, so scale_ub = 64 clamps a sizeable fraction of rows
    (about 14 % measured on the full workload); independent masks would
    not clamp any row."""
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS["prefill_p8_8192x7168"]
    d = synth.make_inputs(w, device="cpu", rows=192)
    xs = [synth.bf16_bits(x) for x in d["inputs"]]
    big = [np.abs(torch_f32(x)) > 20.0 for x in xs]  # |N(0, 0.5)| > 20 only via the x100
    # The outlier positions coincide across slabs: most positions that are
    # large in slab 0 are large in every other slab too (independent masks
    # would share about 0.1 % of them).
    for b in big[1:]:
        assert np.sum(big[0] & b) > 0.5 * np.sum(big[0])
    frac = np.mean(big[0])
    assert 0.0003 < frac < 0.002
    _, s, _ = orc.arnfp8(xs, synth.bf16_bits(d["gamma"]), w.eps, w.weight_offset, w.scale_ub,
                         residual_in=synth.bf16_bits(d["residual"]))
    clamped = np.mean(s == np.float32(w.scale_ub / 448.0))
    assert 0.05 < clamped < 0.30, clamped


def torch_f32(bits):
    import torch

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()


def test_workload_shapes_and_laws():
    from all_reduce_rmsnorm_amd import synth

    W = synth.WORKLOADS
    assert (W["tiny_p2_4x256"].P, W["tiny_p2_4x256"].rows, W["tiny_p2_4x256"].cols) == (2, 4, 256)
    assert W["tiny_p2_4x256"].residual_std is None
    assert W["decode_p4_32x7168"].residual_std == 1.0 and W["decode_p4_32x7168"].x_std == 0.5
    u = W["unit_offset_p8_128x8192"]
    assert u.weight_offset == 1.0 and u.eps == 1e-5 and u.gamma_law == ("normal", 0.0, 0.02)
    p = W["prefill_p8_8192x7168"]
    assert p.scale_ub == 64.0 and p.outlier_frac == 0.001 and p.outlier_mult == 100.0
    d = synth.make_inputs(W["tiny_p2_4x256"], device="cpu")
    d2 = synth.make_inputs(W["tiny_p2_4x256"], device="cpu")
    for a, b in zip(d["inputs"], d2["inputs"]):
        assert np.array_equal(synth.bf16_bits(a), synth.bf16_bits(b))  # seeded
    assert not np.array_equal(synth.bf16_bits(d["inputs"][0]), synth.bf16_bits(d["inputs"][1]))


def test_traffic_reported_only_for_matching_device_code(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_hash()
    good = tmp_path / "good.md"
    good.write_text(f"kernel_source_hash: {h}\ntraffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(good))
    assert bench.read_traffic(h) == 123456
    stale = tmp_path / "stale.md"
    stale.write_text("kernel_source_hash: 0000000000000000\ntraffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(stale))
    assert bench.read_traffic(h) is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.read_traffic(h) is None


def test_committed_counter_summary_matches_the_device_code():
    """The committed HBM-counter summary was taken on the current device code
    (else bench reports traffic as null and the summary must be re-taken)."""
    sys.path.insert(0, ROOT)
    import bench

    assert bench.read_traffic(bench.kernel_source_hash()) is not None


def test_every_committed_profile_matches_the_device_code():
    """Every workload's committed kernel trace and counter summary (the row or
    sum kernel for each workload the benchmark reports, the split kernel for
    the workloads it times through arnfp8_run_split) was taken on the current
    device code."""
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_hash()
    names = [bench.DEFAULT_WORKLOAD, bench.SHARE_WORKLOAD] + list(bench.LATENCY_WORKLOADS)
    wanted = [(n, False) for n in names] + [(n, True) for n in bench.SPLIT_PROFILE_WORKLOADS]
    for name, split in wanted:
        trace = bench.profile_path(name, "kernel_trace", split)
        traffic = bench.profile_path(name, "hbm_traffic", split)
        assert bench.read_profile(trace, "mean_us", h) is not None, trace
        assert bench.read_profile(traffic, "traffic_bytes_per_launch", h) is not None, traffic


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    sys.path.insert(0, ROOT)
    import bench

    d = tmp_path / "pmc"
    d.mkdir()
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    (d / "a_counter_collection.csv").write_text(
        hdr + '1,"void arnfp8::arn_sum_kernel<1, 4>(x)",FETCH_SIZE,524288\n'
              '2,"void arnfp8::arnfp8_row_kernel<0, 8, 2, true, true, true>(y)",FETCH_SIZE,500000\n')
    (d / "b_counter_collection.csv").write_text(
        hdr + '1,"void arnfp8::arn_sum_kernel<1, 4>(x)",WRITE_SIZE,1048576\n'
              '2,"void arnfp8::arnfp8_row_kernel<0, 8, 2, true, true, true>(y)",WRITE_SIZE,100000\n')
    out = tmp_path / "summary.md"
    bench.summarize_pmc(str(d), str(out), "prefill_p8_8192x7168")
    text = out.read_text()
    # FETCH scaled x2 (copy read 1 GiB, counter 512 MiB), WRITE x1
    want = int(round(500000 * 1024 * 2.0 + 100000 * 1024 * 1.0))
    assert f"traffic_bytes_per_launch: {want}" in text


def test_cpu_figures_cover_every_row_and_agree_in_units():
    """Both CPU figures time the oracle over the whole workload and report the
    same algorithmic bytes per pass."""
    import torch

    import bench
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS["decode_p4_32x7168"]
    d = synth.make_inputs(w)
    one = bench.cpu_baseline(w, d, torch, min_seconds=0.0, max_passes=1)
    many = bench.cpu_oracle_threaded(w, d, torch, passes=1)
    assert one["cores"] == 1 and one["kind"] == "oracle" and one["unit"] == many["unit"] == "GB/s"
    for r in (one, many):
        gbs = w.algorithmic_bytes() / (r["ms_per_step"] * 1e-3) / 1e9
        assert abs(gbs - r["value"]) <= 1e-3 * gbs + 1e-4
    assert 1 <= many["threads"] <= 16
    assert "32 rows" in one["sample"] or "(32 rows)" in one["sample"]


def test_input_hash_is_reproducible_and_covers_every_tensor():
    import torch

    import bench
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS["decode_p4_32x7168"]
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    assert bench.input_sha256(a, torch) == bench.input_sha256(b, torch)
    assert bench.input_sha256(synth.make_inputs(w, seed=1), torch) != bench.input_sha256(a, torch)
    for key in ("residual", "gamma"):
        c = dict(a)
        c[key] = a[key].clone()
        c[key].view(-1)[-1] += 1
        assert bench.input_sha256(c, torch) != bench.input_sha256(a, torch), key
    c = dict(a)
    c["inputs"] = [a["inputs"][1], a["inputs"][0]] + a["inputs"][2:]
    assert bench.input_sha256(c, torch) != bench.input_sha256(a, torch)


def test_counter_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    import bench

    cpp = tmp_path / "k.hpp"
    py = tmp_path / "b.py"
    cpp.write_text("// a comment\nint f() { return 1; } /* block\ncomment */\n")
    py.write_text("# a comment\nFLAGS = ['-O3']\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(cpp), str(py)])
    h0 = bench.kernel_source_hash()
    cpp.write_text("// another comment\nint f() {   return 1; }\n")
    py.write_text("# reworded\n\nFLAGS = ['-O3']\n")
    assert bench.kernel_source_hash() == h0
    cpp.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0
    cpp.write_text("int f() { return 1; }\n")
    py.write_text("FLAGS = ['-O2']\n")
    assert bench.kernel_source_hash() != h0


def test_output_sets_exceed_twice_the_infinity_cache_on_the_headline():
    """The timed prefill step writes a fresh output set on every call: the sets
    together exceed 512 MiB, so no call finds its outputs in the 256 MB cache."""
    import bench
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    n = bench.out_sets_for(w)
    per_set = w.numel * (1 + 2) + 4 * w.rows  # fp8 + bf16 residual out + scales
    assert n >= 2 and n * per_set >= bench.CACHE_FLUSH_BYTES
    assert 1 <= bench.out_sets_for(synth.WORKLOADS["tiny_p2_4x256"]) <= bench.MAX_OUT_SETS


def test_rotating_calls_each_function_in_turn():
    import bench

    seen = []
    f = bench.rotating([lambda: seen.append(0), lambda: seen.append(1), lambda: seen.append(2)])
    for _ in range(7):
        f()
    assert seen == [0, 1, 2, 0, 1, 2, 0]


def test_summarize_pmc_split_picks_the_split_kernel(tmp_path):
    """With split, the summary counts the split-row kernel's dispatches of the
    workload's P, not the row kernel's."""
    sys.path.insert(0, ROOT)
    import bench

    d = tmp_path / "pmc"
    d.mkdir()
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    rows = ('1,"void arnfp8::arn_sum_kernel<1, 4>(x)",{c},1048576\n'
            '2,"void arnfp8::arnfp8_row_kernel<0, 8, 1, false, true, true>(y)",{c},999\n'
            '3,"void arnfp8::arnfp8_split_kernel<8, false, true>(arnfp8::SplitArgs)",{c},100\n'
            '4,"void arnfp8::arnfp8_split_kernel<4, false, true>(arnfp8::SplitArgs)",{c},777\n')
    (d / "a_counter_collection.csv").write_text(hdr + rows.format(c="FETCH_SIZE"))
    (d / "b_counter_collection.csv").write_text(hdr + rows.format(c="WRITE_SIZE"))
    out = tmp_path / "summary.md"
    bench.summarize_pmc(str(d), str(out), "token_p8_1x8192", split=True)
    text = out.read_text()
    assert f"traffic_bytes_per_launch: {int(round(100 * 1024 * 2))}" in text
    assert "arnfp8_split_kernel" in text and "--split" in text
    assert bench.profile_path("token_p8_1x8192", "kernel_trace", True).endswith(
        "arnfp8_split_kernel_token_p8_1x8192_kernel_trace.md")
