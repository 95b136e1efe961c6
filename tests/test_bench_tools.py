"""CPU tests of bench.py's profile tooling: the kernel-trace and counter
summaries pick the timed steps' up and down GEMM launches by order, and the
HBM traffic per launch is the counter value scaled by the copy kernel's
calibration.  Synthetic rocprofv3-style CSVs stand in for a GPU run."""

import csv
import json

import pytest

import bench

V5 = "nvfp4::(anonymous namespace)::gemm_nvfp4_v5_kernel<false>(unsigned char const*, int)"
QUANT = "nvfp4::(anonymous namespace)::quantize_resident_kernel(uint4 const*, unsigned int)"


def _step_launches(warmup, steps):
    """The v5 launch sequence of a bench run: setup, warm-up, timed and the
    pass with per-stage events, one [up, down] pair per step; each launch is
    tagged with its pass so a test can see which were picked."""
    seq = [("setup", 0)] + [("warmup", i) for i in range(warmup)] + \
          [("timed", i) for i in range(steps)] + [("events", i) for i in range(steps)]
    out = []
    for kind, i in seq:
        out.append((kind, i, "up"))
        out.append((kind, i, "down"))
    return out


def _duration(kind, i, which):
    # distinct durations (us) per pass, so a wrong selection changes the mean
    base = {"setup": 5000.0, "warmup": 3000.0, "timed": 1000.0, "events": 2000.0}[kind]
    return base + (0.0 if which == "up" else 500.0) + i


def _write_trace(path, warmup, steps):
    t = 0
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for kind, i, which in _step_launches(warmup, steps):
            w.writerow({"Kernel_Name": QUANT, "Grid_Size_X": 256 * 1024, "Workgroup_Size_X": 1024,
                        "Start_Timestamp": t, "End_Timestamp": t + 30000})
            t += 40000
            d = int(_duration(kind, i, which) * 1000)
            w.writerow({"Kernel_Name": V5, "Grid_Size_X": 256 * 256, "Workgroup_Size_X": 256,
                        "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 1000


def _write_counters(path, counter, warmup, steps, up_kib, down_kib, extra=()):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Workgroup_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        d = 0
        for kind, i, which in _step_launches(warmup, steps):
            d += 1
            # only the timed launches carry the values the test expects
            v = (up_kib if which == "up" else down_kib) if kind == "timed" else 1.0
            # a counter can come in several rows per dispatch (one per XCD):
            # the summary adds them
            for part in (0.25, 0.75):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": V5, "Grid_Size": 256 * 256,
                            "Workgroup_Size": 256, "Counter_Name": counter,
                            "Counter_Value": v * part})
        for name, value in extra:
            d += 1
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": 4096 * 256,
                        "Workgroup_Size": 256, "Counter_Name": counter, "Counter_Value": value})


def test_short_kernel_name():
    assert bench._short_kernel_name(V5) == "gemm_nvfp4_v5_kernel<false>"
    assert bench._short_kernel_name("ns::k<ns::C<64, 64>>(int, float)") == "k<ns::C<64, 64>>"


@pytest.mark.parametrize("warmup,steps", [(1, 3), (5, 20)])
def test_summarize_trace_picks_the_timed_steps(tmp_path, warmup, steps):
    path = tmp_path / "trace.csv"
    _write_trace(path, warmup, steps)
    rows, headline = bench.summarize_trace(str(path), warmup, steps)
    assert headline["gemm_up_gelu_amax"]["launches"] == steps
    assert headline["gemm_down"]["launches"] == steps
    up = [_duration("timed", i, "up") for i in range(steps)]
    down = [_duration("timed", i, "down") for i in range(steps)]
    assert headline["gemm_up_gelu_amax"]["avg_us"] == pytest.approx(sum(up) / steps, abs=0.01)
    assert headline["gemm_down"]["avg_us"] == pytest.approx(sum(down) / steps, abs=0.01)
    assert headline["gemm_up_gelu_amax"]["min_us"] == pytest.approx(min(up), abs=0.01)
    by_kernel = {(r["kernel"], r["workgroups"]): r for r in rows}
    assert by_kernel[("gemm_nvfp4_v5_kernel<false>", 256)]["launches"] == 2 * (1 + warmup + 2 * steps)
    assert by_kernel[("quantize_resident_kernel", 256)]["launches"] == 2 * (1 + warmup + 2 * steps)


def test_summarize_trace_too_few_launches(tmp_path):
    path = tmp_path / "trace.csv"
    _write_trace(path, 1, 3)
    _, headline = bench.summarize_trace(str(path), 5, 20)
    assert headline is None


def test_traffic_json_scales_by_the_copy_calibration(tmp_path):
    warmup, steps = 1, 3
    f_csv, w_csv = tmp_path / "fetch.csv", tmp_path / "write.csv"
    cf_csv, cw_csv = tmp_path / "copy_fetch.csv", tmp_path / "copy_write.csv"
    _write_counters(f_csv, "FETCH_SIZE", warmup, steps, up_kib=300000.0, down_kib=270000.0)
    _write_counters(w_csv, "WRITE_SIZE", warmup, steps, up_kib=400000.0, down_kib=150000.0)
    # the 1 GiB copy: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    _write_counters(cf_csv, "FETCH_SIZE", 0, 0, 0, 0,
                    extra=[("calib_copy_kernel(uint4 const*, uint4*, long)", 524288.0)])
    _write_counters(cw_csv, "WRITE_SIZE", 0, 0, 0, 0,
                    extra=[("calib_copy_kernel(uint4 const*, uint4*, long)", 1048576.0)])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(out), str(f_csv), str(w_csv), str(cf_csv), str(cw_csv), warmup, steps)
    rec = json.loads(out.read_text())
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    up = rec["kernels"]["gemm_nvfp4_v5_kernel"]
    assert up["read_bytes"] == 300000 * 1024 * 2
    assert up["written_bytes"] == 400000 * 1024
    assert up["bytes_per_launch"] == up["read_bytes"] + up["written_bytes"]
    down = rec["kernels"]["gemm_nvfp4_v5_kernel (down)"]
    assert down["read_bytes"] == 270000 * 1024 * 2
    assert down["written_bytes"] == 150000 * 1024


def test_traffic_json_needs_the_copy_kernel(tmp_path):
    f_csv = tmp_path / "fetch.csv"
    _write_counters(f_csv, "FETCH_SIZE", 1, 3, 1.0, 1.0)
    with pytest.raises(SystemExit):
        bench.write_traffic(str(tmp_path / "o.json"), str(f_csv), str(f_csv), str(f_csv),
                            str(f_csv), 1, 3)
