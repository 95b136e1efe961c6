"""Throughput of the NVFP4 DiT-linear hot path on one MI355X.

One step = the DiT MLP at 2048x2048 (16384 image + 512 text tokens, hidden
3072, MLP 12288) as an NVFP4 model runs it:

    quantize(X)                      single-pass quantizer          (X bf16 [16896,3072])
                                     (dynamic amax agreed on chip)
    H = gemm(Xq, Wup_q, GELU, amax)  block-scaled W4A4 GEMM         (16896 x 12288 x 3072)
    quantize(H, amax)                quantizer, producer's amax     (H bf16 [16896,12288])
    Y = gemm(Hq, Wdown_q)            block-scaled W4A4 GEMM         (16896 x 3072 x 12288)

The weights are quantized once before timing (load-time weight quantization),
and their quantization is timed separately.  `value` is the two GEMMs' FLOPs
(2*M*N*K each) over the whole step's time, in TFLOP/s.  The JSON line also
carries the per-stage times, the roofline of the dominant kernel (the up
GEMM, timed with HIP events on the stream it runs on), the standalone
quantize / dequantize rates on the [16896,3072] activation read cold from
HBM (rotating copies), the bf16 passthrough on a modulation-shaped layer, and the CPU
oracle timed on a row sample of the same step.

The roofline object also carries what this part sustains, measured in the
same run by calibration kernels with known work (an fp16 MFMA loop on
data-bearing operands, with the shader clock it ran at; streaming HBM read
and copy), and the dominant kernel's average duration from the committed
rocprofv3 kernel trace of this command when that trace was taken on the
current kernel sources.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --calib-copy     (1 GiB streaming copy kernel, for counter calibration)
       python bench.py --summarize-trace kernel_trace.csv [--trace-json out.json]
                                         (per-kernel, per-grid durations of a rocprofv3
                                          --kernel-trace CSV; no GPU needed)
       python bench.py --summarize-counters counter_collection.csv
                                         (per-kernel means of a rocprofv3 --pmc CSV)
       (both take the profiled run's --steps / --warmup to find its timed GEMMs)
"""

import argparse
import hashlib
import json
import os
import sys
import time
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TOKENS, HIDDEN, MLP = 16896, 3072, 12288
GEMM_FLOP = 2 * TOKENS * MLP * HIDDEN              # each of up and down
PEAK_MFMA_F16 = 2500.0                              # TFLOP/s, dense fp16/bf16 MFMA
PEAK_MFMA_FP8 = 5000.0                              # TFLOP/s, dense fp8 MFMA
PEAK_HBM = 8000.0                                   # GB/s
QUANT_BYTES_PER_ELEM = 2 + 0.5 + 1.0 / 16           # bf16 read + codes + scales


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-graphs", action="store_true", help="skip the HIP-graph section")
    p.add_argument("--no-extras", action="store_true",
                   help="only the headline step, quantize and bf16 sections (profiling runs)")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="token rows of the CPU oracle's pass through the whole step")
    p.add_argument("--cpu-g2-rows", type=int, default=64,
                   help="rows of the exact int64 GEMM form timed per shape (extrapolated)")
    p.add_argument("--calib-copy", action="store_true")
    p.add_argument("--summarize-trace", metavar="CSV",
                   help="summarize a rocprofv3 kernel_trace.csv and exit")
    p.add_argument("--trace-json", metavar="JSON", help="with --summarize-trace: also write JSON")
    p.add_argument("--trace-command", default="", help="with --trace-json: the profiled command")
    p.add_argument("--summarize-counters", metavar="CSV",
                   help="summarize a rocprofv3 --pmc counter_collection.csv and exit (JSON)")
    p.add_argument("--traffic-json", nargs=5, metavar=("OUT", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="write the up GEMM's HBM bytes per launch to OUT from the FETCH_SIZE and "
                        "WRITE_SIZE counter CSVs of this script and of its --calib-copy run; exit")
    return p.parse_args()


def _progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the HIP / C++ sources the library is built from (the counter
    summary under profiles/ is valid only for the sources it was taken on).
    The test-only probe library's sources are left out."""
    from nvfp4_block_scaled_05_amd import build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_block_scaled_05_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        path = os.path.join(csrc, name)
        if not os.path.isfile(path) or not name.endswith((".hip", ".hpp", ".cpp", ".h")):
            continue
        if name in build.PROBE_SOURCES:
            continue
        with open(path, "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, launches_per_step):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


UP_TILES = ((TOKENS + 255) // 256) * ((MLP + 255) // 256)   # 256x256 tiles of the up GEMM


def _short_kernel_name(name):
    """A kernel's name without namespaces and argument list, template
    arguments kept: 'nvfp4::(anonymous namespace)::k<2>(int, ...)' -> 'k<2>'."""
    name = name.replace("(anonymous namespace)", "anon")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    base, depth, last = name[:cut], 0, 0
    for i, ch in enumerate(base):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0:
            last = i + 1
    return base[last:].strip()


def summarize_trace(csv_path, warmup, steps):
    """Per (kernel, grid size) dispatch statistics of a rocprofv3
    --kernel-trace CSV of this script (launches, mean / median / min / max
    duration in us), and the headline step's two GEMMs on their own: the
    v5 kernel's launches come first in the run, as [up, down] once while the
    step's buffers are set up, `warmup` times, then `steps` timed times (the
    pass with per-stage events follows them), so the timed up and down
    launches are picked by their index."""
    import csv
    groups, v5 = {}, []
    with open(csv_path, newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    for row in rows:
        name = _short_kernel_name(row.get("Kernel_Name", ""))
        grid = row.get("Grid_Size_X") or row.get("Grid_Size") or "0"
        wg = row.get("Workgroup_Size_X") or row.get("Workgroup_Size") or "1"
        dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        groups.setdefault((name, int(grid) // max(int(wg), 1)), []).append(dur)
        if name == "gemm_nvfp4_v5_kernel<false>":
            v5.append(dur)

    def stats(d):
        a = np.array(d)
        return {"launches": len(d), "avg_us": round(float(a.mean()), 2),
                "median_us": round(float(np.median(a)), 2), "min_us": round(float(a.min()), 2),
                "max_us": round(float(a.max()), 2), "total_us": round(float(a.sum()), 1)}
    out = [{"kernel": name, "workgroups": wgs, **stats(d)} for (name, wgs), d in groups.items()]
    out.sort(key=lambda r: -r["total_us"])
    first = 2 * (1 + warmup)
    headline = None
    if len(v5) >= first + 2 * steps:
        headline = {"gemm_up_gelu_amax": stats(v5[first:first + 2 * steps:2]),
                    "gemm_down": stats(v5[first + 1:first + 2 * steps:2]),
                    "selection": f"gemm_nvfp4_v5_kernel<false> launches {first}, {first + 2}, ... "
                                 f"(up) and {first + 1}, {first + 3}, ... (down): the {steps} timed "
                                 f"steps after the setup call and {warmup} warm-up steps"}
    return out, headline


LIBRARY_KERNEL_PREFIXES = ("gemm_nvfp4", "gemm_fp8", "gemm_bf16", "gemv_bf16", "quantize_",
                           "amax_partial", "dequantize", "v5_split_reduce", "split_reduce",
                           "fp8_", "zero_", "calib_")


def print_trace_summary(rows, headline, source_hash, command, json_path=None):
    print("| kernel | workgroups | launches | average us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['kernel']} | {r['workgroups']} | {r['launches']} | {r['avg_us']} | "
              f"{r['median_us']} | {r['min_us']} | {r['max_us']} |")
    if headline:
        print()
        print("| headline step kernel | launches | average us | median us | min us | max us |")
        print("|---|---|---|---|---|---|")
        for k in ("gemm_up_gelu_amax", "gemm_down"):
            r = headline[k]
            print(f"| {k} | {r['launches']} | {r['avg_us']} | {r['median_us']} | {r['min_us']} | "
                  f"{r['max_us']} |")
    if json_path:
        # the library's own kernels only (torch's fills, casts and the
        # yardstick GEMMs stay in the printed table)
        own = [r for r in rows if r["kernel"].startswith(LIBRARY_KERNEL_PREFIXES)]
        with open(json_path, "w") as f:
            json.dump({"source_hash": source_hash, "command": command, "headline": headline,
                       "dispatches": own}, f, indent=1)
            f.write("\n")


def summarize_counters(csv_path, warmup, steps):
    """Per (kernel, grid size) mean of every counter in a rocprofv3 --pmc
    counter_collection CSV of this script, and the same for the headline
    step's up and down GEMMs, picked by launch index as in summarize_trace."""
    import csv
    disp = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            d = disp.setdefault(int(row["Dispatch_Id"]), {
                "kernel": _short_kernel_name(row.get("Kernel_Name", "")),
                "workgroups": int(row.get("Grid_Size") or 0) // max(int(row.get("Workgroup_Size") or 1), 1),
                "counters": {}})
            name = row["Counter_Name"]
            d["counters"][name] = d["counters"].get(name, 0.0) + float(row["Counter_Value"])
    order = [disp[k] for k in sorted(disp)]

    def mean(ds):
        names = sorted({n for d in ds for n in d["counters"]})
        return {"launches": len(ds),
                **{n: float(np.mean([d["counters"].get(n, 0.0) for d in ds])) for n in names}}
    groups = {}
    for d in order:
        groups.setdefault((d["kernel"], d["workgroups"]), []).append(d)
    rows = [{"kernel": k, "workgroups": w, **mean(ds)} for (k, w), ds in groups.items()]
    v5 = [d for d in order if d["kernel"] == "gemm_nvfp4_v5_kernel<false>"]
    first = 2 * (1 + warmup)
    headline = None
    if len(v5) >= first + 2 * steps:
        headline = {"gemm_up_gelu_amax": mean(v5[first:first + 2 * steps:2]),
                    "gemm_down": mean(v5[first + 1:first + 2 * steps:2])}
    return rows, headline


def write_traffic(out, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, warmup, steps):
    """HBM bytes per launch of the headline up GEMM from two counter runs of
    this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled
    by what the same counter reads for the calibration copy kernel, which
    reads and writes 1 GiB per launch (--calib-copy)."""
    n = 1 << 30

    def copy_kib(csv_path, counter):
        rows, _ = summarize_counters(csv_path, 0, 0)
        r = [x for x in rows if x["kernel"] == "calib_copy_kernel"]
        if not r or counter not in r[0]:
            raise SystemExit(f"no calib_copy_kernel {counter} in {csv_path}")
        return r[0][counter]
    fetch_factor = n / 1024 / copy_kib(copy_fetch_csv, "FETCH_SIZE")
    write_factor = n / 1024 / copy_kib(copy_write_csv, "WRITE_SIZE")
    _, hf = summarize_counters(fetch_csv, warmup, steps)
    _, hw = summarize_counters(write_csv, warmup, steps)
    if not hf or not hw:
        raise SystemExit("the counter runs do not hold the headline step's GEMM launches")
    rd = hf["gemm_up_gelu_amax"]["FETCH_SIZE"] * 1024 * fetch_factor
    wr = hw["gemm_up_gelu_amax"]["WRITE_SIZE"] * 1024 * write_factor
    rd_down = hf["gemm_down"]["FETCH_SIZE"] * 1024 * fetch_factor
    wr_down = hw["gemm_down"]["WRITE_SIZE"] * 1024 * write_factor
    rec = {"source_hash": kernel_source_hash(), "fetch_factor": fetch_factor,
           "write_factor": write_factor,
           "kernels": {"gemm_nvfp4_v5_kernel": {
               "bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "written_bytes": int(wr),
               "launch": "up projection (GELU + amax), timed steps"},
               "gemm_nvfp4_v5_kernel (down)": {
               "bytes_per_launch": int(rd_down + wr_down), "read_bytes": int(rd_down),
               "written_bytes": int(wr_down), "launch": "down projection, timed steps"}}}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def profiled_up_gemm():
    """The up GEMM's average duration over the timed steps in the committed
    kernel trace of this command, if that trace was taken on the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "dit_mlp_2048_kernel_trace.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or not rec.get("headline"):
        return None
    r = rec["headline"]["gemm_up_gelu_amax"]
    return {"avg_launch_us": r["avg_us"], "median_us": r["median_us"], "launches": r["launches"],
            "command": rec.get("command", "")}


def calibration(ev, stream):
    """What this part sustains, from kernels with known work (calib.h in the
    package sources): the fp16 MFMA rate with constant and with data-bearing
    operands and the shader clock under that load, and streaming HBM read
    and copy rates over 1 GiB buffers (four times the last-level cache)."""
    import ctypes
    import torch
    from nvfp4_block_scaled_05_amd import build
    lib = ctypes.CDLL(build.PROBE_LIB)
    P = ctypes.c_void_p
    lib.nvfp4_calib_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P]
    lib.nvfp4_calib_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.nvfp4_calib_copy.argtypes = [P, P, ctypes.c_size_t, P]
    units = lib.nvfp4_calib_units()
    sink = torch.empty(units * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(units * 4 * 2, dtype=torch.int64, device="cuda")
    s = stream.cuda_stream

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    out = {"what": "calibration kernels with known work, same run"}
    iters = 20000
    flop = units * 4 * iters * 16 * 32768
    for mode, name in ((0, "mfma_f16_constant_operands"), (1, "mfma_f16_data_operands"),
                       (2, "mfma_f16_nvfp4_valued_operands")):
        def run(mode=mode):
            rc = lib.nvfp4_calib_mfma_f16(iters, mode, sink.data_ptr(), clocks.data_ptr(), s)
            if rc != 0:
                raise RuntimeError(f"nvfp4_calib_mfma_f16: {rc}")
        t = timed(run, 3)
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.mean(c[:, 0] / np.maximum(c[:, 1], 1))) * 0.1
        out[name] = {"TFLOPs": round(flop / t / 1e12, 1), "clock_GHz": round(ghz, 3),
                     "us": round(t * 1e6, 1)}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    red = torch.empty(4096, dtype=torch.int32, device="cuda")
    t_read = timed(lambda: lib.nvfp4_calib_read(src.data_ptr(), n, red.data_ptr(), s), 5)
    t_copy = timed(lambda: lib.nvfp4_calib_copy(src.data_ptr(), dst.data_ptr(), n, s), 5)
    out["hbm_read_GBps"] = round(n / t_read / 1e9, 1)
    out["hbm_copy_GBps"] = round(2 * n / t_copy / 1e9, 1)
    del src, dst
    return out


def main():
    args = parse()
    if args.summarize_counters:
        rows, headline = summarize_counters(args.summarize_counters, args.warmup, args.steps)
        print(json.dumps({"source_hash": kernel_source_hash(), "headline": headline,
                          "dispatches": rows}, indent=1))
        return
    if args.traffic_json:
        write_traffic(*args.traffic_json, args.warmup, args.steps)
        return
    if args.summarize_trace:
        rows, headline = summarize_trace(args.summarize_trace, args.warmup, args.steps)
        print_trace_summary(rows, headline, kernel_source_hash(), args.trace_command,
                            args.trace_json)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard along tokens, each GPU holding the full quantized "
              "weights; inside a layer only the 4-byte amax of each dynamically quantized "
              "tensor would be exchanged, by an all-reduce of the max)", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_block_scaled_05_amd as nv
    from nvfp4_block_scaled_05_amd import inputs

    if args.calib_copy:
        import ctypes
        from nvfp4_block_scaled_05_amd import build
        lib = ctypes.CDLL(build.PROBE_LIB)
        lib.nvfp4_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            lib.nvfp4_calib_copy(a.data_ptr(), b.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_kernel": "calib_copy_kernel", "launches": 5,
                          "bytes_read_per_launch": n, "bytes_written_per_launch": n}))
        return

    nv.load()
    dev = "cuda"

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------------------------------------------------------- setup --
    t0 = time.time()
    data = inputs.mlp_2048()
    x = to_dev(data["x"])
    w_up, w_down = to_dev(data["w_up"]), to_dev(data["w_down"])
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # weight pre-quantization (load time), timed separately: W_up through the
    # same quantizer into preallocated outputs, 5 calls back to back (the 75 MB
    # weight stays in the 256 MB last-level cache between them)
    wq_up = nv.quantize_weight(w_up)
    wq_down = nv.quantize_weight(w_down)
    w_ws = nv.quantize_workspace(dev)
    w_out = (wq_up.codes.clone(), wq_up.scales.clone(), wq_up.tensor_scale.clone())
    for _ in range(2):
        nv.quantize(w_up, workspace=w_ws, out=w_out)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(5):
        nv.quantize(w_up, workspace=w_ws, out=w_out)
    e1.record(stream)
    torch.cuda.synchronize()
    wquant_us = e0.elapsed_time(e1) * 1e3 / 5
    del w_out, w_ws

    # preallocated step buffers
    ws = nv.quantize_workspace(dev)
    xq = nv.quantize(x, workspace=ws)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    ws_up = nv.gemm_workspace(TOKENS, MLP, HIDDEN, device=dev)      # K-split of the tail tiles
    ws_down = nv.gemm_workspace(TOKENS, HIDDEN, MLP, device=dev)
    h = nv.gemm(xq, wq_up, epilogue="gelu", y_amax=amax, workspace=ws_up)
    hq = nv.quantize(h, amax=amax)
    y = nv.gemm(hq, wq_down, workspace=ws_down)
    xq_out = (xq.codes, xq.scales, xq.tensor_scale)
    hq_out = (hq.codes, hq.scales, hq.tensor_scale)

    stage_names = ["quantize_x", "gemm_up_gelu_amax", "quantize_h", "gemm_down"]

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        nv.quantize(x, workspace=ws, out=xq_out)
        if events is not None:
            events[1].record(stream)
        nv.gemm(xq, wq_up, epilogue="gelu", y_amax=amax, out=h, workspace=ws_up)
        if events is not None:
            events[2].record(stream)
        nv.quantize(h, amax=amax, out=hq_out)
        if events is not None:
            events[3].record(stream)
        nv.gemm(hq, wq_down, out=y, workspace=ws_down)
        if events is not None:
            events[4].record(stream)

    # The timed steps: nothing but the step's own launches between the two
    # synchronizations.  An event recorded between two kernels adds a gap of
    # about 5 us before the next; replaying the step as a HIP graph ran each
    # GEMM 2-3% slower, with an 8 us gap between replays.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    # then the same number of steps again with events between the stages,
    # for the per-stage times (not part of the headline figure)
    ev_sets = [[ev() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(ev_sets[i])
    torch.cuda.synchronize()
    stage_us = {n: float(np.mean([s[j].elapsed_time(s[j + 1]) * 1e3 for s in ev_sets]))
                for j, n in enumerate(stage_names)}
    step_ev_ms = np.array([s[0].elapsed_time(s[-1]) for s in ev_sets])
    step_pct = {f"p{q}": round(float(np.percentile(step_ev_ms, q)), 4) for q in (10, 50, 90)}
    value = 2 * GEMM_FLOP / (ms_per_step * 1e-3) / 1e12

    extras = SimpleNamespace(x=x, xq=xq, xq_out=xq_out, wq_up=wq_up, wq_down=wq_down, amax=amax,
                             y=y, h=h, ws_up=ws_up, ws_down=ws_down, w_up=w_up, w_down=w_down,
                             stream=stream, ev=ev, steps=args.steps, warmup=args.warmup)
    _progress(f"step timed: {ms_per_step:.3f} ms; extra sections")
    static = None if args.no_extras else static_section(extras)
    fp8 = None if args.no_extras else fp8_section(extras)
    yardstick = None if args.no_extras else yardstick_section(extras)

    # roofline of the dominant kernel: the up GEMM, timed by the events around
    # its call in the pass with per-stage events (which also enqueues the one-word zeroing of the amax
    # the epilogue reduces into, so the figure is a little above the kernel's
    # own duration in the kernel trace)
    _progress("extra sections done; calibration kernels")
    calib = calibration(ev, stream)
    up_us = stage_us["gemm_up_gelu_amax"]
    achieved = GEMM_FLOP / (up_us * 1e-6) / 1e12
    traffic = measured_traffic("gemm_nvfp4_v5_kernel", 2)
    measured_peak = calib["mfma_f16_nvfp4_valued_operands"]["TFLOPs"]
    prof = profiled_up_gemm()
    roofline = {"kernel": "gemm_nvfp4_v5_kernel 256x256, 4 waves (up projection, GELU + amax epilogue)",
                "bound": "mfma",
                "achieved": round(achieved, 1), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_F16, 4), "traffic": traffic,
                "algorithmic_flop_per_launch": GEMM_FLOP, "avg_launch_us": round(up_us, 2),
                "peak_measured": measured_peak,
                "peak_measured_what": "fp16 32x32x16 MFMA loop on NVFP4-valued operands "
                                      "(E2M1 x E4M3 products, as the GEMM feeds), same run",
                "frac_measured": round(achieved / measured_peak, 4),
                "clock_GHz": calib["mfma_f16_nvfp4_valued_operands"]["clock_GHz"],
                "profile": prof,
                "frac_profile": (round(GEMM_FLOP / (prof["avg_launch_us"] * 1e-6) / 1e12 / PEAK_MFMA_F16, 4)
                                 if prof else None)}

    # ------------------------------------- standalone quantize / dequantize --
    # R distinct copies of the activation (R * 104 MB exceeds the 256 MB
    # last-level cache), quantized back to back between two events: every
    # call reads cold data and the event overhead is spread over R calls.
    R = 8
    act0 = to_dev(inputs.quantize_act()["x"])
    acts = [act0.clone() for _ in range(R)]
    ws2 = [nv.quantize_workspace(dev) for _ in range(R)]
    qas = [nv.quantize(acts[r], workspace=ws2[r]) for r in range(R)]
    qa_outs = [(q.codes, q.scales, q.tensor_scale) for q in qas]
    y_acts = [torch.empty_like(act0) for _ in range(R)]
    act_amax = torch.tensor([float(act0.float().abs().max())], dtype=torch.float32, device=dev)

    def timed_rotating(fn, iters=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(iters):
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / R)
        return float(np.median(ts))

    n_act = TOKENS * HIDDEN
    q_bytes = n_act * QUANT_BYTES_PER_ELEM
    q_us = timed_rotating(lambda: [nv.quantize(acts[r], workspace=ws2[r], out=qa_outs[r]) for r in range(R)])
    # the same quantize through the two-pass kernels (amax pass + encode), for context
    saved = os.environ.get("NVFP4_QUANT_KERNEL")
    os.environ["NVFP4_QUANT_KERNEL"] = "twopass"
    try:
        q2_us = timed_rotating(lambda: [nv.quantize(acts[r], workspace=ws2[r], out=qa_outs[r]) for r in range(R)])
    finally:
        if saved is None:
            del os.environ["NVFP4_QUANT_KERNEL"]
        else:
            os.environ["NVFP4_QUANT_KERNEL"] = saved
    q1_us = timed_rotating(lambda: [nv.quantize(acts[r], amax=act_amax, out=qa_outs[r]) for r in range(R)])
    dq_us = timed_rotating(lambda: [nv.dequantize(qas[r], out=y_acts[r]) for r in range(R)])
    # warm: one copy R times in a row, so its 104 MB stays in the last-level
    # cache after the first call (reported apart; not an HBM figure)
    qw_us = timed_rotating(lambda: [nv.quantize(acts[0], workspace=ws2[0], out=qa_outs[0]) for _ in range(R)])
    dqw_us = timed_rotating(lambda: [nv.dequantize(qas[0], out=y_acts[0]) for _ in range(R)])
    quant = {"workload": "activation [16896,3072] N(0,1) + 0.1% outliers x50",
             "method": f"{R} distinct copies (cold in cache) quantized back to back",
             "algorithmic_bytes": int(q_bytes),
             "quantize_us": round(q_us, 2), "quantize_GBps": round(q_bytes / q_us / 1e3, 1),
             "quantize_frac_hbm": round(q_bytes / q_us / 1e3 / PEAK_HBM, 4),
             "quantize_frac_hbm_copy_measured": round(q_bytes / q_us / 1e3 / calib["hbm_copy_GBps"], 4),
             "quantize_kernel": "single pass (input held on chip while the amax is agreed)",
             "quantize_two_pass_us": round(q2_us, 2),
             "quantize_two_pass_GBps": round(q_bytes / q2_us / 1e3, 1),
             "quantize_amax_given_us": round(q1_us, 2),
             "quantize_amax_given_GBps": round(q_bytes / q1_us / 1e3, 1),
             "dequantize_us": round(dq_us, 2), "dequantize_GBps": round(q_bytes / dq_us / 1e3, 1),
             "dequantize_frac_hbm": round(q_bytes / dq_us / 1e3 / PEAK_HBM, 4),
             "warm": {"method": f"one copy quantized {R} times in a row (input resident in the "
                                "256 MB last-level cache; not an HBM figure)",
                      "quantize_us": round(qw_us, 2), "quantize_GBps": round(q_bytes / qw_us / 1e3, 1),
                      "dequantize_us": round(dqw_us, 2),
                      "dequantize_GBps": round(q_bytes / dqw_us / 1e3, 1)}}
    h_bytes = TOKENS * MLP * QUANT_BYTES_PER_ELEM
    quant["quantize_h_in_step_GBps"] = round(h_bytes / stage_us["quantize_h"] / 1e3, 1)
    quant["with_concurrent_gemm"] = concurrent_quantize(extras, acts[0], ws2[0], qas[0])
    del acts, y_acts

    # bf16 passthrough on a modulation-shaped layer kept high precision
    temb = to_dev(inputs.random_matrix(81, (2, HIDDEN)))
    w_mod = to_dev(inputs.random_matrix(82, (6 * HIDDEN, HIDDEN), std=0.02))
    ymod = nv.gemm_bf16(temb, w_mod)
    mod_us = timed_rotating(lambda: [nv.gemm_bf16(temb, w_mod, out=ymod) for _ in range(R)])
    bf16_pass = {"layer": "modulation [2,3072] x [18432,3072]^T (bf16 by the exclude pattern)",
                 "selected_bf16": not nv.layer_is_quantized("blocks.0.double_stream_modulation.lin"),
                 "us": round(mod_us, 2),
                 "GBps_weight_read": round(6 * HIDDEN * HIDDEN * 2 / mod_us / 1e3, 1)}

    _progress("quantize and bf16 sections done; graphs and shapes")
    graphs = None if args.no_graphs or args.no_extras else graph_section(to_dev, ev, stream)
    shapes = None if args.no_extras else shapes_section(to_dev, ev, stream)

    # ----------------------------------------------------------- CPU oracle --
    cpu = None
    _progress("GPU sections done")
    if not args.no_cpu:
        _progress("CPU oracle baseline (about a minute)")
        cpu = cpu_baseline(data, args.cpu_rows, args.cpu_g2_rows)

    rec = {
        "metric": "NVFP4 GEMM TFLOP/s + quantize HBM GB/s on DiT linear shapes (% of peak)",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 e2m1/e4m3 operands, exact f16 decode, f16 MFMA, f32 accumulate, bf16 out",
        "data": "synthetic (seeded: X Student-t(3), W 0.02*N(0,1))",
        "config": {"workload": "dit_mlp_2048: quantize X -> GEMM up + GELU + amax -> "
                               "quantize H -> GEMM down",
                   "tokens": TOKENS, "hidden": HIDDEN, "mlp": MLP,
                   "flop_per_step": 2 * GEMM_FLOP, "parallelism": "single GPU"},
        "timing": "wall clock over the timed steps between two synchronizations, no events "
                  "between the stages; stages_us from as many further steps with events",
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        "step_ms_events": step_pct,
        "weight_quantize_us": round(wquant_us, 2),
        "weight_quantize": "W_up [12288,3072], preallocated outputs, mean of 5 back-to-back calls",
        "roofline": roofline,
        "calibration": calib,
        "quantize": quant,
        "bf16_passthrough": bf16_pass,
        "mfma_yardstick": yardstick,
        "static_scale": static,
        "fp8_rowwise": fp8,
        "graphs": graphs,
        "dit_linear_shapes": shapes,
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(rec))


def concurrent_quantize(c, act, ws, ref):
    """The single-pass quantize of the activation while the up GEMM runs on a
    second (default-priority) stream: its workgroups cannot all be resident,
    so the ones that start first reach their wait limit and read the ranges
    of the ones not yet arrived.  Reports the quantize's time on its own
    stream, the GEMM's, and whether the bytes equal the uncontended call's."""
    import torch
    import nvfp4_block_scaled_05_amd as nv
    other = torch.cuda.Stream()           # default priority
    codes = torch.empty_like(ref.codes)
    scales = torch.empty_like(ref.scales)
    ts = torch.empty_like(ref.tensor_scale)
    q_us, g_us = [], []
    for _ in range(5):
        torch.cuda.synchronize()
        g0, g1, q0, q1 = c.ev(), c.ev(), c.ev(), c.ev()
        other.wait_stream(c.stream)
        with torch.cuda.stream(other):
            g0.record(other)
            nv.gemm(c.xq, c.wq_up, epilogue="gelu", y_amax=c.amax, out=c.h, workspace=c.ws_up)
            g1.record(other)
        q0.record(c.stream)
        nv.quantize(act, workspace=ws, out=(codes, scales, ts))
        q1.record(c.stream)
        torch.cuda.synchronize()
        q_us.append(q0.elapsed_time(q1) * 1e3)
        g_us.append(g0.elapsed_time(g1) * 1e3)
    same = bool(torch.equal(codes, ref.codes) and torch.equal(scales, ref.scales)
                and torch.equal(ts, ref.tensor_scale))
    return {"what": "single-pass quantize of the activation while the up GEMM runs on a "
                    "second default-priority stream (median of 5)",
            "quantize_us": round(float(np.median(q_us)), 1),
            "gemm_us": round(float(np.median(g_us)), 1), "bytes_equal_uncontended": same}


def timed_sequence(c, fn, names):
    """Warm up, then time c.steps runs of fn(events) (events bracket its
    len(names) stages); returns (ms per run, {stage: mean us})."""
    import torch
    for _ in range(c.warmup):
        fn(None)
    torch.cuda.synchronize()
    evs = [[c.ev() for _ in range(len(names) + 1)] for _ in range(c.steps)]
    t0 = time.perf_counter()
    for i in range(c.steps):
        fn(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / c.steps
    stages = {n: round(float(np.mean([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])), 2)
              for j, n in enumerate(names)}
    return ms, stages


def static_section(c):
    """The step under static (calibrated) tensor scales: X quantized in one
    pass, H written in NVFP4 by the up projection's epilogue (no bf16 H)."""
    import torch
    import nvfp4_block_scaled_05_amd as nv
    x_static = torch.tensor([float(c.x.float().abs().max())], dtype=torch.float32, device=c.x.device)
    h_static = c.amax.clone()                   # calibrated on the dynamic step
    hq = nv.gemm_quantized(c.xq, c.wq_up, h_static, epilogue="gelu")
    hq_out = (hq.codes, hq.scales, hq.tensor_scale)

    def run(events):
        mark = (lambda k: events[k].record(c.stream)) if events else (lambda k: None)
        mark(0)
        nv.quantize(c.x, amax=x_static, out=c.xq_out)
        mark(1)
        nv.gemm_quantized(c.xq, c.wq_up, h_static, epilogue="gelu", out=hq_out)
        mark(2)
        nv.gemm(hq, c.wq_down, out=c.y, workspace=c.ws_down)
        mark(3)
    ms, stages = timed_sequence(c, run, ["quantize_x_one_pass", "gemm_up_gelu_to_nvfp4", "gemm_down"])
    return {"workload": "same step with static tensor scales (calibrated amax of X and H)",
            "ms_per_step": round(ms, 4), "TFLOPs": round(2 * GEMM_FLOP / (ms * 1e-3) / 1e12, 1),
            "stages_us": stages}


def fp8_section(c):
    """The FP8 row-wise variant ("fp8r") of the step: per-token activation
    scales, per-channel weight scales, native FP8 matrix cores."""
    import nvfp4_block_scaled_05_amd as nv
    fw_up, fw_down = nv.fp8_quantize(c.w_up), nv.fp8_quantize(c.w_down)
    fx = nv.fp8_quantize(c.x)
    dev = c.x.device
    ws_up = nv.fp8_gemm_workspace(TOKENS, MLP, HIDDEN, device=dev)
    ws_down = nv.fp8_gemm_workspace(TOKENS, HIDDEN, MLP, device=dev)
    h8 = nv.fp8_gemm(fx, fw_up, epilogue="gelu", workspace=ws_up)
    fh = nv.fp8_quantize(h8)
    y8 = nv.fp8_gemm(fh, fw_down, workspace=ws_down)

    def run(events):
        mark = (lambda k: events[k].record(c.stream)) if events else (lambda k: None)
        mark(0)
        nv.fp8_quantize(c.x, out=(fx.codes, fx.scales))
        mark(1)
        nv.fp8_gemm(fx, fw_up, epilogue="gelu", out=h8, workspace=ws_up)
        mark(2)
        nv.fp8_quantize(h8, out=(fh.codes, fh.scales))
        mark(3)
        nv.fp8_gemm(fh, fw_down, out=y8, workspace=ws_down)
        mark(4)
    ms, st = timed_sequence(c, run, ["quantize_x", "gemm_up_gelu", "quantize_h", "gemm_down"])
    up = GEMM_FLOP / (st["gemm_up_gelu"] * 1e-6) / 1e12
    return {"workload": "same step, FP8 row-wise (per-token / per-channel E4M3, native FP8 MFMA)",
            "ms_per_step": round(ms, 4), "TFLOPs": round(2 * GEMM_FLOP / (ms * 1e-3) / 1e12, 1),
            "stages_us": st,
            "roofline_gemm_up": {"bound": "mfma", "peak": PEAK_MFMA_FP8, "unit": "TFLOP/s",
                                 "achieved": round(up, 1), "frac": round(up / PEAK_MFMA_FP8, 4)},
            "quantize_x_GBps": round(TOKENS * HIDDEN * 3 / st["quantize_x"] / 1e3, 1),
            "quantize_h_GBps": round(TOKENS * MLP * 3 / st["quantize_h"] / 1e3, 1)}


def yardstick_section(c):
    """What the vendor library reaches on the same GEMM shapes in plain fp16
    (hipBLASLt through torch.matmul, no decode, no epilogue): the practical
    matrix-core ceiling of this power-limited part, next to the 2.5 PF spec."""
    import torch
    out = {}
    for name, (m, n, k) in (("gemm_up", (TOKENS, MLP, HIDDEN)), ("gemm_down", (TOKENS, HIDDEN, MLP))):
        a = torch.randn(m, k, device=c.x.device).to(torch.float16)
        w = torch.randn(n, k, device=c.x.device).to(torch.float16)
        y = torch.empty(m, n, device=c.x.device, dtype=torch.float16)

        def run(events, a=a, w=w, y=y):
            mark = (lambda q: events[q].record(c.stream)) if events else (lambda q: None)
            mark(0)
            torch.matmul(a, w.t(), out=y)
            mark(1)
        _, st = timed_sequence(c, run, ["mm"])
        flop = 2 * m * n * k
        out[name] = {"shape": [m, n, k], "us": st["mm"], "TFLOPs": round(flop / (st["mm"] * 1e-6) / 1e12, 1)}
        del a, w, y
    out["fp8"] = fp8_yardstick(c)
    return {"what": "hipBLASLt fp16 GEMM (torch.matmul), same shapes, no decode or epilogue", **out}


def fp8_yardstick(c):
    """hipBLASLt's FP8 GEMM (torch._scaled_mm: E4M3 operands, one scale per
    tensor, bf16 out, no epilogue) on the same shapes, beside the row-wise FP8
    path.  Reports the error instead if this torch build does not run it."""
    import torch
    out = {}
    try:
        for name, (m, n, k) in (("gemm_up", (TOKENS, MLP, HIDDEN)), ("gemm_down", (TOKENS, HIDDEN, MLP))):
            a = torch.randn(m, k, device=c.x.device).to(torch.float8_e4m3fn)
            w = torch.randn(n, k, device=c.x.device).to(torch.float8_e4m3fn)
            one = torch.ones((), device=c.x.device, dtype=torch.float32)

            def run(events, a=a, w=w, one=one):
                mark = (lambda q: events[q].record(c.stream)) if events else (lambda q: None)
                mark(0)
                torch._scaled_mm(a, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
                mark(1)
            _, st = timed_sequence(c, run, ["mm"])
            flop = 2 * m * n * k
            out[name] = {"shape": [m, n, k], "us": st["mm"],
                         "TFLOPs": round(flop / (st["mm"] * 1e-6) / 1e12, 1)}
            del a, w
    except Exception as e:   # an fp8 GEMM this torch build cannot run: say so
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    return {"what": "hipBLASLt FP8 GEMM (torch._scaled_mm, per-tensor scales, bf16 out, no epilogue)",
            **out}


def shapes_section(to_dev, ev, stream):
    """The DiT linears at other real shapes, each GEMM and its dynamic quantize
    of X timed on its own: the QKV projection at 1024^2 (4608 tokens), and one
    GPU's share of every linear when the 2048^2 block is split over 8 GPUs by
    tokens: 4224 tokens (CFG 2 x Ulysses 4 over 33792) and 2112 (Ulysses 8
    over 16896).  Weights ~ 0.02 N(0,1), quantized once; X ~ N(0,1)."""
    import torch
    import nvfp4_block_scaled_05_amd as nv
    from nvfp4_block_scaled_05_amd import inputs

    def per_call_us(fn, iters=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    wshape = {"qkv": (3 * HIDDEN, HIDDEN), "o": (HIDDEN, HIDDEN), "up": (MLP, HIDDEN),
              "down": (HIDDEN, MLP)}
    wq = {k: nv.quantize_weight(to_dev(inputs.random_matrix(90 + i, shp, std=0.02)))
          for i, (k, shp) in enumerate(wshape.items())}
    cases = [("qkv_1024x1024_cfg2", "qkv", 4608)]
    cases += [(f"{tag}_{k}", k, m) for tag, m in (("share_of_8_cfg2_ulysses4", 33792 // 8),
                                                 ("share_of_8_ulysses8", TOKENS // 8))
              for k in ("qkv", "o", "up", "down")]
    out = {}
    for name, k, M in cases:
        N, K = wshape[k]
        x = to_dev(inputs.random_matrix(100 + M + N, (M, K)))
        qx = nv.quantize(x)
        qws = nv.quantize_workspace(x.device)
        ws = nv.gemm_workspace(M, N, K, device=x.device)
        epi = "gelu" if k == "up" else "none"
        y = nv.gemm(qx, wq[k], epilogue=epi, workspace=ws)
        q_us = per_call_us(lambda: nv.quantize(x, workspace=qws, out=(qx.codes, qx.scales, qx.tensor_scale)))
        g_us = per_call_us(lambda: nv.gemm(qx, wq[k], epilogue=epi, out=y, workspace=ws))
        out[name] = {"M": M, "N": N, "K": K, "epilogue": epi, "quantize_x_us": round(q_us, 2),
                     "gemm_us": round(g_us, 2),
                     "gemm_TFLOPs": round(2 * M * N * K / (g_us * 1e-6) / 1e12, 1)}
        del x, qx, y, ws
    return out


def graph_section(to_dev, ev, stream):
    """Launch overhead removed by HIP-graph capture: the launch-bound single
    linear (X [128,1024], W [1024,1024], both quantized per call) and the
    linear layers of one DiT block at 2048^2 with a CFG pair (33792 tokens)."""
    import torch
    import nvfp4_block_scaled_05_amd as nv
    from nvfp4_block_scaled_05_amd import inputs
    from nvfp4_block_scaled_05_amd.dit_block import DitBlockLinears, LAYERS, gemm_flops
    from nvfp4_block_scaled_05_amd.graph import capture

    def per_call_us(fn, iters):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    d = inputs.linear_small()
    x, w = to_dev(d["x"]), to_dev(d["w"])
    qx = nv.quantize(x)
    qw = nv.quantize(w)
    y = nv.gemm(qx, qw)
    ws_x = nv.quantize_workspace(x.device)
    ws_w = nv.quantize_workspace(x.device)

    def small():
        nv.quantize(x, workspace=ws_x, out=(qx.codes, qx.scales, qx.tensor_scale))
        nv.quantize(w, workspace=ws_w, out=(qw.codes, qw.scales, qw.tensor_scale))
        nv.gemm(qx, qw, out=y, workspace=None)
    small_eager = per_call_us(small, 200)
    g_small = capture(small)
    small_graph = per_call_us(g_small.replay, 200)

    blk = inputs.dit_block_2048()
    wts = {k: to_dev(blk[k]) for k in ("w_mod", "w_qkv", "w_o", "w_up", "w_down")}
    acts = [to_dev(blk[k]) for k in ("temb", "x_qkv", "x_o", "x_mlp")]
    del blk
    block = DitBlockLinears(wts, tokens=acts[1].shape[0])
    run = lambda: block(*acts)
    block_eager = per_call_us(run, 5)
    g_block = capture(run)
    block_graph = per_call_us(g_block.replay, 5)
    shapes = {"temb": tuple(acts[0].shape), "x_qkv": tuple(acts[1].shape),
              "x_o": tuple(acts[2].shape), "x_mlp": tuple(acts[3].shape),
              "h": (acts[3].shape[0], wts["w_up"].shape[0])}
    shapes.update({k: tuple(v.shape) for k, v in wts.items()})
    flops = gemm_flops(shapes)
    total = sum(flops.values())
    return {"linear_small_128x1024x1024": {"eager_us": round(small_eager, 2),
                                           "graph_us": round(small_graph, 2)},
            "dit_block_2048": {"layers": {k: ("nvfp4" if block.quantized[k] else "bf16")
                                          for k in LAYERS},
                               "tokens": acts[1].shape[0], "gflop": round(total / 1e9, 1),
                               "eager_ms": round(block_eager / 1e3, 3),
                               "graph_ms": round(block_graph / 1e3, 3),
                               "graph_TFLOPs": round(total / (block_graph * 1e-6) / 1e12, 1)}}


def cpu_baseline(data, rows, g2_rows):
    """The CPU oracle as it stands (never tuned for speed), timed in the same
    process after the GPU figures, on the same seeded inputs:

      value             the MLP step's two GEMMs' FLOPs per second of the
                        oracle's pass through the whole step (amax over all of
                        X, quantize, float64-BLAS GEMM up + GELU, quantize H
                        with its amax, GEMM down) on `rows` token rows, all
                        BLAS threads;
      quantize /        the activation [16896,3072] in full, one core (numpy's
      dequantize        elementwise work is single-threaded), in GB/s of the
                        same algorithmic bytes as the GPU figures;
      gemm_fp64         the float64-BLAS form on the full single-linear, QKV
                        and MLP shapes (operand decode, tensor scales and bf16
                        rounding included; quantization of the inputs and the
                        GELU not: the step above times the GELU);
      gemm_exact_int64  the exact int64 form on `g2_rows` rows of each shape,
                        its time per row extrapolated linearly to all rows.
    """
    import oracle
    from oracle.formats import bf16_bits_to_f32
    from nvfp4_block_scaled_05_amd import inputs
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count()
    t_all = time.perf_counter()
    x = data["x"]
    rwu = oracle.quantize(data["w_up"])
    rwd = oracle.quantize(data["w_down"])

    # the whole step on a row sample
    rng = np.random.default_rng(0)
    sel = np.sort(rng.choice(TOKENS, rows, replace=False))
    t0 = time.perf_counter()
    amax = np.abs(bf16_bits_to_f32(x)).max()
    rx = oracle.quantize(x[sel], amax=amax)
    h_bits, _ = oracle.gemm_fp64(rx, rwu, HIDDEN, gelu=True)
    h_amax = np.abs(bf16_bits_to_f32(h_bits)).max()
    rh = oracle.quantize(h_bits, amax=h_amax)
    oracle.gemm_fp64(rh, rwd, MLP)
    dt_step = time.perf_counter() - t0
    step_flop = 2 * 2 * rows * MLP * HIDDEN

    # quantize / dequantize of the full activation, one core
    act = inputs.quantize_act()["x"]
    n_act = act.size
    if threadpool_limits is not None:
        with threadpool_limits(1):
            t0 = time.perf_counter()
            qa = oracle.quantize(act)
            t_q = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.dequantize(qa.codes, qa.scales, qa.tensor_scale, HIDDEN)
            t_dq = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        qa = oracle.quantize(act)
        t_q = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.dequantize(qa.codes, qa.scales, qa.tensor_scale, HIDDEN)
        t_dq = time.perf_counter() - t0
    qbytes = n_act * QUANT_BYTES_PER_ELEM
    del act, qa

    # float64-BLAS and exact int64 forms on the full shapes
    small = inputs.linear_small()
    c1 = (oracle.quantize(small["x"]), oracle.quantize(small["w"]), 1024)
    qkv = inputs.qkv_1024()
    c3 = (oracle.quantize(qkv["x"]), oracle.quantize(qkv["w"]), HIDDEN)
    rx_full = oracle.quantize(x)
    # an operand of the down projection's full shape, for timing only: the
    # sampled rows' quantized H repeated down to 16896 rows (the float64 form
    # does the same work whatever the codes are)
    reps = -(-TOKENS // rows)
    h_full = oracle.Quantized(codes=np.tile(rh.codes, (reps, 1))[:TOKENS],
                              scales=np.tile(rh.scales, (reps, 1))[:TOKENS],
                              tensor_scale=rh.tensor_scale, amax=rh.amax, s_enc=rh.s_enc,
                              degenerate=rh.degenerate)
    shapes = {"linear_128x1024x1024": (c1, False),
              "qkv_4608x9216x3072": (c3, False),
              "mlp_up_16896x12288x3072": ((rx_full, rwu, HIDDEN), False),
              "mlp_down_16896x3072x12288": ((h_full, rwd, MLP), False)}
    g3, g2 = {}, {}
    for name, ((qa_, qw_, K), gelu) in shapes.items():
        M, N = qa_.codes.shape[0], qw_.codes.shape[0]
        t0 = time.perf_counter()
        oracle.gemm_fp64(qa_, qw_, K, gelu=gelu)
        dt = time.perf_counter() - t0
        g3[name] = {"s": round(dt, 3), "TFLOPs": round(2 * M * N * K / dt / 1e12, 5)}
        if M > g2_rows:
            r = np.arange(g2_rows) * (M // g2_rows)
            t0 = time.perf_counter()
            oracle.gemm_exact_rows(qa_, qw_, K, r, gelu=gelu)
            dt = time.perf_counter() - t0
            full = dt * M / g2_rows
            g2[name] = {"rows_timed": g2_rows, "s_timed": round(dt, 3),
                        "s_extrapolated_all_rows": round(full, 1),
                        "TFLOPs_extrapolated": round(2 * M * N * K / full / 1e12, 6)}
    total = time.perf_counter() - t_all
    return {"value": round(step_flop / dt_step / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {TOKENS} token rows through the whole MLP step (amax over all "
                      f"of X, quantize, float64-BLAS GEMM up + GELU, quantize H, GEMM down); "
                      f"weights quantized beforehand (not counted)",
            "seconds": round(dt_step, 2),
            "quantize_activation_16896x3072": {
                "cores": 1, "quantize_s": round(t_q, 2), "quantize_GBps": round(qbytes / t_q / 1e9, 4),
                "dequantize_s": round(t_dq, 2), "dequantize_GBps": round(qbytes / t_dq / 1e9, 4)},
            "gemm_fp64_full_shapes": {"cores": int(threads), **g3},
            "gemm_exact_int64_extrapolated": {"cores": 1, **g2},
            "down_operand": "the sampled rows' quantized H repeated to 16896 rows (timing only)",
            "total_cpu_seconds": round(total, 1),
            "host": _host_info(threads)}


def _host_info(blas_threads):
    """The CPU the baseline ran on: model, logical CPUs, the ones this process
    may use, and the BLAS thread count."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "usable_cpus": usable,
            "blas_threads": int(blas_threads)}


if __name__ == "__main__":
    main()
