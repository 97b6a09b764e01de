"""Host-side pieces of bench.py (no GPU): argument rules, the oracle
baseline record, the profile summaries and the recorded-traffic lookup."""

from __future__ import annotations

import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench

REPO = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, str(REPO / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_record():
    rec = bench.run_cpu_baseline(2, 64, 0.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["cores"] == 1
    assert rec["value"] > 0 and "T=2, H=64" in rec["sample"]


def test_algorithmic_bytes_per_token():
    T, H = 3, 7168
    assert bench.fwd_bytes(T, H) == T * (10 * H + 16)
    assert bench.bwd_bytes(T, H) == T * (18 * H + 32)
    assert bench.bwd_acc_bytes(T, H) == T * (26 * H + 32)
    # other expansion rates, counted from the buffers: n = 2 reads 2 x 2H of
    # residual and 8 B of pre per token; n = 8 reads 8 x 2H and 32 B
    assert bench.fwd_bytes(T, H, 2) == T * (2 * 2 * H + 8 + 2 * H)
    assert bench.fwd_bytes(T, H, 8) == T * (8 * 2 * H + 32 + 2 * H)
    assert bench.bwd_bytes(T, H, 2) == T * (2 * 2 * H + 2 * H + 8 + 2 * 2 * H + 8)
    assert bench.bwd_bytes(T, H, 8) == T * (8 * 2 * H + 2 * H + 32 + 8 * 2 * H + 32)
    assert bench.bwd_acc_bytes(T, H, 8) == bench.bwd_bytes(T, H, 8) + T * 8 * 2 * H


def test_probe_record_fractions():
    rec = bench.probe_record(1000, 1.0, {"block": [2.0, 2.0, 2.0], "bytes": 1000}, "bwd")
    assert rec["kernel_gbps"] == 1.0 and rec["probe_gbps"] == 0.5 and rec["frac_of_probe"] == 2.0
    assert rec["mix"] == "5:4"
    rec = bench.probe_record(1000, 1.0, {"block": [1.0], "bytes": 500}, "fwd")
    assert rec["mix"] == "4:1" and rec["frac_of_probe"] == 2.0
    assert bench.probe_record(10, 1.0, {"block": [1.0], "bytes": 8192}, "read")["mix"] == "8:0"


def test_round_stats_any_count():
    """One round gives its value for every percentile (the driver's short
    runs never reach a quantile of a single point)."""
    assert bench.round_stats([5.0]) == {"us_median": 5.0, "us_p20_p50_p80": [5.0, 5.0, 5.0],
                                        "rounds": 1}
    r = bench.round_stats([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0])
    assert r["us_median"] == 4.0 and r["us_p20_p50_p80"][1] == 4.0
    assert r["us_p20_p50_p80"][0] < 4.0 < r["us_p20_p50_p80"][2]


def _fake_gpu(steps_seen):
    """A stand-in for run_gpu with the shape of its result (made-up times)."""
    def run(T, H, steps, warmup, nsets, copy_calibration, sample=32, shapes=True, probes=True):
        steps_seen.append(steps)
        blk = [22.0 + 0.01 * i for i in range(7)]
        out = {"wall_s": steps * 35e-6, "region_gpu_us": steps * 34.8,
               "step_block": [34.7] * 7, "fwd_block": [12.1] * 7, "bwd_block": blk,
               "fwd_sampled": [11.9] * sample if sample else None,
               "bwd_sampled": [21.3] * sample if sample else None,
               "fwd_plan": {"block_threads": 64}, "fwd_grid": 14336,
               "bwd_plan": {"layout": 2}, "bwd_grid": 1024,
               "device": "stub", "torch": "stub", "hip": None}
        if probes:
            out["probes"] = {k: {"bytes": 132153344, "block": [22.5] * 7}
                             for k in ("bwd", "fwd", "read", "write")}
        if shapes:
            out["shapes"] = [{"direction": d, "T": t, "H": H, "sets": n, "block": [40.0] * 7,
                              "sampled": [39.0]} for d, t, n in bench.SHAPES]
        return out
    return run


@pytest.mark.parametrize("argv", [["--gpus", "1", "--steps", "20", "--warmup", "5"],
                                  ["--steps", "1", "--warmup", "0"],
                                  ["--steps", "3", "--sample", "0", "--no-shapes",
                                   "--no-probes"]])
def test_main_record_at_the_driver_command_line(argv, capsys):
    """main() at the driver's command line (and at 1 step) prints one JSON
    line with the contract's fields, a roofline from the block-timed
    backward and the CPU baseline; the GPU part is stubbed."""
    seen = []
    rc = bench.main(argv + ["--cpu-seconds", "0", "--tokens", "4", "--hidden", "64"],
                    gpu_runner=_fake_gpu(seen))
    assert rc == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    steps = int(argv[argv.index("--steps") + 1])
    assert seen == [steps] and rec["steps"] == steps
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "git_sha", "tree_sha256"):
        assert key in rec, key
    assert rec["config"]["workload"].startswith("h_aggregate forward+backward")
    assert rec["config"]["seed"] == 0
    rf = rec["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert rf["achieved"] == pytest.approx(bench.bwd_bytes(4, 64) / 22.03e-6 / 1e9, abs=0.05)
    assert rf["frac"] == pytest.approx(rf["achieved"] / 8000.0, abs=1e-4)
    assert rec["cpu_baseline"]["kind"] == "oracle" and rec["cpu_baseline"]["cores"] >= 1
    assert rec["ms_per_step"] * rec["steps"] == pytest.approx(steps * 35e-3, rel=1e-3)
    if "--no-shapes" not in argv:
        assert [(s["direction"], s["T"]) for s in rec["shapes"]] == \
            [(d, t) for d, t, _ in bench.SHAPES]
        assert set(rec["stream_probes"]) == {"bwd", "fwd", "read_only", "write_only"}
    else:
        assert "shapes" not in rec and "stream_probes" not in rec
    assert (rec["bwd"].get("dispatch_event_us") is None) == ("--sample" in argv)


def test_summaries_parse_rocprof_csv(tmp_path, capsys):
    stats = tmp_path / "kernel_stats.csv"
    stats.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs"\n'
                     '"void (anonymous namespace)::hagg_bwd_rows_kernel<8, 8, false>(unsigned short'
                     ' const*, float const*)",10,220000,22000.0,60.0,21000,23000\n')
    bench.summarize_stats(str(stats))
    out = capsys.readouterr().out
    assert "| hagg_bwd_rows_kernel<8, 8, false> | 10 | 22.000 |" in out
    pmc = tmp_path / "counter_collection.csv"
    pmc.write_text('"Grid_Size","Kernel_Name","Counter_Name","Counter_Value"\n'
                   '262144,"void (anonymous namespace)::hagg_bwd_rows_kernel<8, 8, false>(int)",'
                   '"FETCH_SIZE",100.0\n'
                   '262144,"void (anonymous namespace)::hagg_bwd_rows_kernel<8, 8, false>(int)",'
                   '"FETCH_SIZE",300.0\n')
    bench.summarize_pmc([str(pmc)])
    out = capsys.readouterr().out
    assert "| hagg_bwd_rows_kernel<8, 8, false> | 262144 | FETCH_SIZE | 2 | 200.0 |" in out


def test_recorded_traffic_is_tied_to_the_kernel_source():
    """The profile's traffic figure is used only for the kernel and shape it
    was measured on, and only while that kernel's code is unchanged (else
    null)."""
    value = bench.recorded_traffic(1024, 7168, "hagg_bwd_rows_kernel")
    assert value is None or value > 0
    assert bench.recorded_traffic(512, 7168, "hagg_bwd_rows_kernel") is None
    assert bench.recorded_traffic(1024, 4096, "hagg_bwd_rows_kernel") is None
    assert bench.recorded_traffic(1024, 7168, "hagg_bwd_kernel (split") is None
    fake = ("# HBM traffic - hagg_bwd_rows_kernel, T=1024, H=7168\n"
            "traffic_bytes_per_launch: 123\ndevice_code_sha256: " + "0" * 64 + "\n")
    assert bench.recorded_traffic(1024, 7168, "hagg_bwd_rows_kernel", fake) is None  # digest


def test_all_core_baseline_record():
    rec = bench.run_cpu_baseline_all_cores(4, 64, 0.0, 2)
    assert rec["kind"] == "oracle" and rec["cores"] == 2 and rec["value"] > 0
    assert "2 token slices" in rec["sample"]


def test_device_code_digest(built_library, tmp_path):
    """The digest names the built library's gfx950 kernels; no library, no
    digest."""
    d = bench.device_code_sha256(built_library)
    assert d is not None and len(d) == 64 and int(d, 16) >= 0
    assert bench.device_code_sha256(tmp_path / "missing.so") is None


def test_coefficient_epilogue_bytes():
    # n = 4: per row mix 96 + pre/post/grad_pre/grad_post 64 + grad_res 64
    # read, grad_mix 96 written = 320; plus alpha, grad_b, grad_alpha.
    assert bench.coeff_bytes(1, 4) == 320 + 12 + 96 + 12
    assert bench.coeff_bytes(8192, 4) == 8192 * 320 + 120
    assert bench.coeff_bytes(10, 2) == 10 * (64 + 48) + 12 + 32 + 12
    assert bench.coeff_bytes(10, 8) == 10 * (256 + 768) + 12 + 320 + 12
    assert [r for r, n, d in bench.COEFF_SWEEP if n == 4 and d == "f32"] == [512, 2048, 8192]
    assert [r for r, n, d in bench.COEFF_SWEEP if d == "bf16"] == [512, 2048, 8192]
    assert bench.coeff_bytes(10, 4, 2) == 10 * 160 + 12 + 96 + 12


def test_counter_cases_are_valid_launch_shapes(built_library):
    """Every launch shape the counter runs compare passes the library's own
    plan check at T=1024, H=7168 (fake addresses; no GPU)."""
    from hyper_connection_residual_mhc_amd import ops
    T, H = 1024, 7168
    base = 1 << 34
    res, pre, g, gr, gp = base, base + (1 << 30), base + (2 << 30), base + (3 << 30), base + (4 << 30)
    layouts = {}
    for case, launch in bench.COUNTER_CASES.items():
        plan, grid = ops.mhc_h_aggregate_plan_bwd(res, pre, g, gr, gp, T, H, launch=launch)
        layouts[case] = (plan["layout"], plan["block_threads"], plan["vec_width"], grid)
    assert layouts["rows"] == (2, 256, 8, 1024)
    assert layouts["rows-1-per-block"] == (2, 64, 8, 4096)
    assert layouts["split"][0] == 1
    assert layouts["rows-v4"][2] == 4
    fwd = {}
    for case, launch in bench.FWD_COUNTER_CASES.items():
        plan, grid = ops.mhc_h_aggregate_plan_fwd(res, pre, base + (5 << 30), T, H, launch=launch)
        fwd[case] = (plan["block_threads"], plan["vec_width"])
    assert fwd == {"fwd": (64, 8), "fwd-v2": (64, 2), "fwd-1024": (1024, 8)}


def test_coefficient_cpu_baseline_record():
    rec = bench.run_coeff_cpu_baseline(64, 4, min_seconds=0.05)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "us/call"
    assert rec["value"] > 0 and "64-row" in rec["sample"]


def test_wave_clock_summary_reads_the_stamps():
    import numpy as np
    # 100 kHz ticks of 10 us; XCD 3 starts 2 ticks after XCD 0 and ends last
    stamps = np.array([
        [100, 105, 110, 0 | (7 << 32)],
        [101, 104, 108, 0],
        [102, 110, 120, 3],
        [104, 106, 107, 3],
    ], dtype=np.int64)
    rec = bench.wave_clock_summary(stamps, 100, dispatch_us=250.0)
    assert rec["waves"] == 4 and rec["xcd"] == [0, 3] and rec["xcd_waves"] == [2, 2]
    assert rec["span_us"] == 200.0
    assert rec["xcd_first_start_us"] == [0.0, 20.0]
    assert rec["xcd_last_end_us"] == [100.0, 200.0]
    assert rec["xcd_wave_us_median"] == [85.0, 105.0]
    assert rec["start_stagger_us"] == 20.0 and rec["end_spread_us"] == 100.0
    assert rec["dispatch_us"] == 250.0
    med = bench.median_records([rec, dict(rec, span_us=100.0), dict(rec, span_us=300.0)])
    assert med["span_us"] == 200.0 and med["xcd"] == [0, 3]
    with pytest.raises(AssertionError):
        bench.median_records([rec, dict(rec, xcd=[0, 4])])
