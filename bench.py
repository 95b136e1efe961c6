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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --calib-copy     (plain 1 GiB device copy, for counter calibration)
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
    p.add_argument("--cpu-rows", type=int, default=12288)
    p.add_argument("--calib-copy", action="store_true")
    return p.parse_args()


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


def main():
    args = parse()
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
        n = 1 << 30
        a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n}))
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
    w_ws = torch.empty(nv.quantize_workspace_bytes(*w_up.shape), dtype=torch.uint8, device=dev)
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
    ws = torch.empty(nv.quantize_workspace_bytes(TOKENS, HIDDEN), dtype=torch.uint8, device=dev)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev_sets = [[ev() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev_sets[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    stage_us = {n: float(np.mean([s[j].elapsed_time(s[j + 1]) * 1e3 for s in ev_sets]))
                for j, n in enumerate(stage_names)}
    step_ev_ms = np.array([s[0].elapsed_time(s[-1]) for s in ev_sets])
    step_pct = {f"p{q}": round(float(np.percentile(step_ev_ms, q)), 4) for q in (10, 50, 90)}
    value = 2 * GEMM_FLOP / (ms_per_step * 1e-3) / 1e12

    extras = SimpleNamespace(x=x, xq=xq, xq_out=xq_out, wq_up=wq_up, wq_down=wq_down, amax=amax,
                             y=y, ws_down=ws_down, w_up=w_up, w_down=w_down, stream=stream, ev=ev,
                             steps=args.steps, warmup=args.warmup)
    static = None if args.no_extras else static_section(extras)
    fp8 = None if args.no_extras else fp8_section(extras)
    yardstick = None if args.no_extras else yardstick_section(extras)

    # roofline of the dominant kernel: the up GEMM
    up_us = stage_us["gemm_up_gelu_amax"]
    achieved = GEMM_FLOP / (up_us * 1e-6) / 1e12
    traffic = measured_traffic("gemm_nvfp4_v5_kernel", 2)
    roofline = {"kernel": "gemm_nvfp4_v5_kernel 256x256, 4 waves (up projection, GELU + amax epilogue)",
                "bound": "mfma",
                "achieved": round(achieved, 1), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_F16, 4), "traffic": traffic,
                "algorithmic_flop_per_launch": GEMM_FLOP, "avg_launch_us": round(up_us, 2)}

    # ------------------------------------- standalone quantize / dequantize --
    # R distinct copies of the activation (R * 104 MB exceeds the 256 MB
    # last-level cache), quantized back to back between two events: every
    # call reads cold data and the event overhead is spread over R calls.
    R = 8
    act0 = to_dev(inputs.quantize_act()["x"])
    acts = [act0.clone() for _ in range(R)]
    ws2 = [torch.empty(nv.quantize_workspace_bytes(TOKENS, HIDDEN), dtype=torch.uint8, device=dev)
           for _ in range(R)]
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
             "quantize_kernel": "single pass (input held on chip while the amax is agreed)",
             "quantize_two_pass_us": round(q2_us, 2),
             "quantize_two_pass_GBps": round(q_bytes / q2_us / 1e3, 1),
             "quantize_amax_given_us": round(q1_us, 2),
             "quantize_amax_given_GBps": round(q_bytes / q1_us / 1e3, 1),
             "dequantize_us": round(dq_us, 2), "dequantize_GBps": round(q_bytes / dq_us / 1e3, 1),
             "warm": {"method": f"one copy quantized {R} times in a row (input resident in the "
                                "256 MB last-level cache; not an HBM figure)",
                      "quantize_us": round(qw_us, 2), "quantize_GBps": round(q_bytes / qw_us / 1e3, 1),
                      "dequantize_us": round(dqw_us, 2),
                      "dequantize_GBps": round(q_bytes / dqw_us / 1e3, 1)}}
    h_bytes = TOKENS * MLP * QUANT_BYTES_PER_ELEM
    quant["quantize_h_in_step_GBps"] = round(h_bytes / stage_us["quantize_h"] / 1e3, 1)
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

    graphs = None if args.no_graphs or args.no_extras else graph_section(to_dev, ev, stream)
    shapes = None if args.no_extras else shapes_section(to_dev, ev, stream)

    # ----------------------------------------------------------- CPU oracle --
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(data, args.cpu_rows)

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
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        "step_ms_events": step_pct,
        "weight_quantize_us": round(wquant_us, 2),
        "weight_quantize": "W_up [12288,3072], preallocated outputs, mean of 5 back-to-back calls",
        "roofline": roofline,
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
    return {"what": "hipBLASLt fp16 GEMM (torch.matmul), same shapes, no decode or epilogue", **out}


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
        qws = torch.empty(nv.quantize_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
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
    ws_x = torch.empty(nv.quantize_workspace_bytes(*x.shape), dtype=torch.uint8, device=x.device)
    ws_w = torch.empty(nv.quantize_workspace_bytes(*w.shape), dtype=torch.uint8, device=x.device)

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


def cpu_baseline(data, rows):
    """The CPU oracle, untuned, on a row sample of the same step."""
    import oracle
    from oracle.formats import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    rng = np.random.default_rng(0)
    sel = np.sort(rng.choice(TOKENS, rows, replace=False))
    x = data["x"]
    t_w = time.perf_counter()
    rwu = oracle.quantize(data["w_up"])
    rwd = oracle.quantize(data["w_down"])
    t_w = time.perf_counter() - t_w
    t0 = time.perf_counter()
    amax = np.abs(bf16_bits_to_f32(x)).max()
    rx = oracle.quantize(x[sel], amax=amax)
    h_bits, _ = oracle.gemm_fp64(rx, rwu, HIDDEN, gelu=True)
    h_amax = np.abs(bf16_bits_to_f32(h_bits)).max()
    rh = oracle.quantize(h_bits, amax=h_amax)
    oracle.gemm_fp64(rh, rwd, MLP)
    dt = time.perf_counter() - t0
    flop = 2 * 2 * rows * MLP * HIDDEN
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {TOKENS} token rows through the whole step (amax over all of X, "
                      f"quantize, float64-BLAS GEMM up + GELU, quantize H, GEMM down); "
                      f"weights quantized beforehand in {t_w:.1f}s (not counted)",
            "seconds": round(dt, 2), "host": _host_info(threads)}


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
