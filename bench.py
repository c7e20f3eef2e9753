#!/usr/bin/env python3
"""Throughput of the fused W8A8 INT8 linear on one MI355X.

One step = one pass of the whole hot path over the 1024px DiT MLP workload
(4096 tokens, hidden 3072, MLP width 12288), on synthetic seeded inputs that
are resident in HBM before timing starts:
  1. the fused linear w8a8_linear, up-proj (M=4096, K=3072, N=12288):
     per-token quantization of X into its workspace, then the int8 GEMM with
     the dequant/bias epilogue
  2. GELU + per-token quantization of the up-proj output [4096, 12288]
  3. int8 GEMM + dequant/bias epilogue, down-proj (M=4096, K=12288, N=3072)
Weight quantization (per output channel) is offline and not timed.  Weights
rotate over several copies so that the 256 MB last-level cache cannot hold
them across steps.

Output: one JSON line.  `value` is int8 tera-operations per second over the
whole step (2*M*N*K per GEMM), from the wall clock around the timed steps.
`fused_linear` is the w8a8_linear call of step 1 (its TOPS and fraction of
the 5.0 POP/s dense int8 matrix peak), from a HIP event pair around the call
in every timed step.  `roofline` reports the up-proj GEMM kernel alone: a
second timed loop runs the same steps with step 1's two kernels issued
through their own entry points (w8a8_quantize_act, w8a8_gemm_dequant: the
same kernels w8a8_linear enqueues), with an event pair around the GEMM.
Events are recorded on the stream the kernels run on.  The timed loops record
only those pairs (each recorded event costs a step ~1-3 us), so `kernels_ms`
(every kernel bracketed) comes from a third, untimed pass.  `cpu_baseline`
times the CPU oracle on a bounded row sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 matrix peak, 5.0 POP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, 8 TB/s
METRIC = "fused W8A8 linear TOPS and % of MI355X INT8 MFMA peak, DiT shapes"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_mlp_up_m4096_k3072_n12288.json")
GEMM_SRC = os.path.join(ROOT, "w8a8_int8_quantized_quantize_amd", "csrc", "gemm.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the chip's clock moves for the first tens of steps (on some boxes up, on
    # others down) before it holds: 20 untimed steps (~8 ms) let it settle
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4, help="weight copies cycled across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time every GEMM configuration on every workload shape instead")
    ap.add_argument("--sweep-iters", type=int, default=20)
    ap.add_argument("--shapes", default="",
                    help="comma-separated workload shape names for --sweep / --compare (default: all)")
    ap.add_argument("--fp8", action="store_true",
                    help="run the step through the FP8 (e4m3) entry points instead of int8")
    ap.add_argument("--compare", action="store_true",
                    help="per workload shape: fused INT8 linear vs the 'fake INT8' path "
                         "(quantize, dequantize to bf16, bf16 GEMM) vs a plain bf16 GEMM")
    ap.add_argument("--interlayer", action="store_true",
                    help="in-step A/B of the MLP step: GELU + quantize as its own pass vs GELU and the "
                         "row absmax folded into the up-projection's epilogue + an absmax-given quantizer")
    ap.add_argument("--profile-shapes", default="",
                    help="comma-separated workload shape names: run the fused linear (w8a8_linear) "
                         "on each, --iters times, weights rotated (a workload for rocprofv3 counter runs)")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device-to-device copy of known size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("GEMM_FETCH", "GEMM_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of a bench run and of a "
                         "--copy-calibration run): write the up-proj GEMM's HBM bytes per launch")
    return ap.parse_args()


def gemm_src_hash() -> str:
    """Hash of the GEMM source's code: line comments and blank lines are left
    out, so that editing a comment does not invalidate the counters."""
    import re
    with open(GEMM_SRC) as f:
        lines = (re.sub(r"//.*", "", ln).rstrip() for ln in f)
        code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_entry():
    """HBM bytes per launch of the up-proj GEMM from rocprofv3 counters, if
    they were taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_src_sha256_16") != gemm_src_hash():
        return None
    return t.get("bytes_per_launch")


COPY_BYTES = 512 << 20  # bytes read and bytes written by one calibration copy


def copy_calibration(torch):
    """A plain device-to-device copy of COPY_BYTES, run a few times: the
    counters FETCH_SIZE / WRITE_SIZE read for it calibrate the GEMM's."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 5}))


def _counter_rows(folder, counter):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append(r)
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def up_kernel_name(cfg_name):
    """The leading part of the up-proj GEMM kernel's name as the profiler
    prints it, for its configuration: the ping-pong kernel (names ending in
    _pp) or the tiled kernel, with the tile's size."""
    import re
    bm, bn = (int(v) for v in re.match(r"bm(\d+)_bn(\d+)_", cfg_name).groups())
    kern = "gemm_pp_kernel" if cfg_name.endswith("_pp") else "gemm_kernel"
    return f"{kern}<w8a8::(anonymous namespace)::Tile<{bm}, {bn},"


def write_traffic(gf, gw, cf, cw):
    """Per-launch HBM bytes of the up-proj GEMM (the dispatch of the gemm kernel
    with the up-proj grid) from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by bytes-moved / counter-reading of the calibration copy."""
    def copy_factor(folder, counter):
        vals = [float(r["Counter_Value"]) * 1024 for r in _counter_rows(folder, counter)
                if "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower()]
        if not vals:
            raise SystemExit(f"no copy kernel rows for {counter} in {folder}")
        return max(vals) / COPY_BYTES  # counter bytes per real byte

    import w8a8_int8_quantized_quantize_amd as w8
    name = w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(4096, 12288, 3072))
    down = w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(4096, 3072, 12288))
    kname = up_kernel_name(name)

    def gemm_bytes(folder, counter):
        rows = sorted((r for r in _counter_rows(folder, counter) if kname in r["Kernel_Name"]),
                      key=lambda r: int(r["Dispatch_Id"]))
        if down == name:  # one kernel for both: the step launches up-proj first
            rows = rows[::2]
        vals = [float(r["Counter_Value"]) * 1024 for r in rows]
        if not vals:
            raise SystemExit(f"no up-proj gemm rows for {counter} in {folder}")
        return sum(vals) / len(vals), len(vals)

    ff, fw = copy_factor(cf, "FETCH_SIZE"), copy_factor(cw, "WRITE_SIZE")
    (fb, nf), (wb, nw) = gemm_bytes(gf, "FETCH_SIZE"), gemm_bytes(gw, "WRITE_SIZE")
    out = {"kernel": f"{kname}...> ({name}), up-proj M=4096 K=3072 N=12288",
           "gemm_src_sha256_16": gemm_src_hash(),
           "fetch_bytes_per_launch": fb / ff, "write_bytes_per_launch": wb / fw,
           "bytes_per_launch": fb / ff + wb / fw,
           "raw_fetch_size_kib": fb / 1024, "raw_write_size_kib": wb / 1024,
           "copy_factor_fetch": ff, "copy_factor_write": fw, "launches": [nf, nw],
           "algorithmic_bytes_per_launch": 4096 * 3072 + 12288 * 3072 + 6 * 12288 + 4 * 4096 + 2 * 4096 * 12288}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def make_inputs(torch, w8, synthetic, rotate, fp8=False):
    dev = "cuda:0"
    up, down = synthetic.CONFIGS["dit1024_mlp"]
    inp = {}
    qw_fn = w8.w8a8_quantize_weight_fp8 if fp8 else w8.w8a8_quantize_weight
    code = torch.uint8 if fp8 else torch.int8

    def lin(shape):
        st = synthetic.streams(0, shape.config_id, shape.layer_id)
        x = synthetic.activations_bf16(st, shape.M, shape.K, shape.outlier_frac).to(dev)
        w = torch.from_numpy(synthetic.weights_f32(st, shape.N, shape.K)).to(dev)
        b = synthetic.bias_bf16(st, shape.N).to(dev)
        wq, sw = qw_fn(w)
        del w
        copies = [(wq, sw)] + [(wq.clone(), sw.clone()) for _ in range(rotate - 1)]
        return x, copies, b

    inp["x_up"], inp["w_up"], inp["b_up"] = lin(up)
    _, inp["w_down"], inp["b_down"] = lin(down)
    M = up.M
    inp["q_x"] = torch.empty((M, up.K), dtype=code, device=dev)
    inp["s_x"] = torch.empty((M,), dtype=torch.float32, device=dev)
    inp["y_up"] = torch.empty((M, up.N), dtype=torch.bfloat16, device=dev)
    inp["q_h"] = torch.empty((M, down.K), dtype=code, device=dev)
    inp["s_h"] = torch.empty((M,), dtype=torch.float32, device=dev)
    inp["y_down"] = torch.empty((M, down.N), dtype=torch.bfloat16, device=dev)
    return up, down, inp


def cpu_baseline(up, down, seconds):
    """The CPU oracle on rows 0..S-1 of the same step, S sized to ~`seconds`."""
    import numpy as np

    import oracle
    import synthetic

    def host_inputs(shape):
        st = synthetic.streams(0, shape.config_id, shape.layer_id)
        x = synthetic.bf16_bits(synthetic.activations_bf16(st, shape.M, shape.K, shape.outlier_frac))
        w = synthetic.weights_f32(st, shape.N, shape.K)
        b = synthetic.bf16_bits(synthetic.bias_bf16(st, shape.N))
        return x, w, b

    x, wu, bu = host_inputs(up)
    _, wd, bd = host_inputs(down)
    wuq, wus = oracle.quantize_rows_f32(wu)   # offline, untimed
    wdq, wds = oracle.quantize_rows_f32(wd)

    def step(S):
        t0 = time.perf_counter()
        y = oracle.linear(x[:S], wuq, wus, bu)["y"]
        h = oracle.gelu_bf16(y)
        oracle.linear(h, wdq, wds, bd)
        return time.perf_counter() - t0

    # size the sample from a 64-row probe; the whole step (all M rows) is the
    # cap -- on a 16-core host the full step takes a few seconds
    S0 = 64
    t = step(S0)
    S = int(max(S0, min(up.M, S0 * seconds / max(t, 1e-6))))
    t = step(S)
    ops = 2.0 * S * (up.N * up.K + down.N * down.K)
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"rows 0..{S - 1} of the MLP step (per-token quantize + int64 GEMM + epilogue "
                      f"for up-proj, fp64 GELU of its output + quantize + GEMM + epilogue for down-proj), "
                      f"{t:.1f} s wall, weights pre-quantized untimed",
            "seconds": t}


def sweep(args, torch, w8, synthetic):
    dev = "cuda:0"
    shapes = [s for v in synthetic.CONFIGS.values() for s in v]
    if args.shapes:
        shapes = [s for s in shapes if s.name in args.shapes.split(",")]
    for s in shapes:
        # the workload's own seeded inputs: the matrix cores draw power in
        # proportion to the bits that toggle, so the code distribution (small
        # per-token activation codes, wider per-channel weight codes) sets the
        # clock the GEMM runs at; uniform random codes would run slower
        st = synthetic.streams(0, s.config_id, s.layer_id)
        x = synthetic.activations_bf16(st, s.M, s.K, s.outlier_frac).to(dev)
        w = torch.from_numpy(synthetic.weights_f32(st, s.N, s.K)).to(dev)
        b = synthetic.bias_bf16(st, s.N).to(dev)
        down = "down" in s.name  # input: GELU of a random tensor, quantized per token
        q, sx = (w8.w8a8_gelu_quantize_act if down else w8.w8a8_quantize_act)(x)[:2]
        qf, sxf = (w8.w8a8_gelu_quantize_act_fp8 if down else w8.w8a8_quantize_act_fp8)(x)[:2]
        wq, sw = w8.w8a8_quantize_weight(w)
        wq8, sw8 = w8.w8a8_quantize_weight_fp8(w)
        del w, x
        # weight copies cycled call to call, > 512 MB in all, so that no call
        # finds its weights in the 256 MB last-level cache (MALL)
        ncopy = max(1, min(64, -(-600_000_000 // max(1, s.N * s.K))))
        wqs = [wq] + [wq.clone() for _ in range(ncopy - 1)]
        y = torch.empty((s.M, s.N), dtype=torch.bfloat16, device=dev)
        sel = w8.w8a8_gemm_select_config(s.M, s.N, s.K)
        for c in range(w8.w8a8_gemm_num_configs()):
            for i in range(3):
                w8.w8a8_gemm_ex(q, sx, wqs[i % ncopy], sw, b, out=y, config=c)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.sweep_iters + 1)]
            torch.cuda.synchronize()
            # keep the GPU busy while the host enqueues the timed calls, so that
            # each event pair brackets GPU work only, not host launch latency
            torch.cuda._sleep(20_000_000)
            evs[0].record()
            for i in range(args.sweep_iters):
                w8.w8a8_gemm_ex(q, sx, wqs[i % ncopy], sw, b, out=y, config=c)
                evs[i + 1].record()
            torch.cuda.synchronize()
            ts = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.sweep_iters))
            med = ts[len(ts) // 2]
            tops = 2.0 * s.M * s.N * s.K / (med * 1e-3) / 1e12
            gbs = (s.M * s.K + s.N * s.K + 2 * s.M * s.N + 6 * s.N) / (med * 1e-3) / 1e9
            print(json.dumps({"sweep": s.name, "config": c, "name": w8.w8a8_gemm_config_name(c),
                              "selected": c == sel, "us_median": round(med * 1e3, 2),
                              "us_min": round(ts[0] * 1e3, 2), "TOPS": round(tops, 1),
                              "GBs": round(gbs, 1), "hbm_frac": round(gbs / 8000.0, 3),
                              "mfma_frac": round(tops / 5000.0, 3)}), flush=True)
        # the FP8 GEMM's configurations on the same shape (e4m3 codes of the same inputs)
        del wqs
        wfs = [wq8] + [wq8.clone() for _ in range(ncopy - 1)]
        for c in range(w8.w8a8_gemm_fp8_num_configs()):
            for i in range(3):
                w8.w8a8_gemm_dequant_fp8(qf, sxf, wfs[i % ncopy], sw8, b, out=y, config=c)
            med, mn = _time_calls(torch, lambda i: w8.w8a8_gemm_dequant_fp8(qf, sxf, wfs[i], sw8, b, out=y,
                                                                           config=c),
                                  args.sweep_iters, ncopy)
            tops = 2.0 * s.M * s.N * s.K / (med * 1e-6) / 1e12
            print(json.dumps({"sweep": s.name, "fp8_config": c, "name": w8.w8a8_gemm_fp8_config_name(c),
                              "us_median": round(med, 2), "us_min": round(mn, 2), "TOPS": round(tops, 1),
                              "mfma_frac": round(tops / 5000.0, 3)}), flush=True)
        del wfs, q, qf, wq, wq8


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _call_times(torch, fn, n_iter, n_copy):
    """Microseconds of each of n_iter back-to-back calls fn(i % n_copy), in call
    order (HIP events between calls; the stream is primed with a GPU sleep so
    that each event pair brackets GPU work only)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_iter + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    evs[0].record()
    for i in range(n_iter):
        fn(i % n_copy)
        evs[i + 1].record()
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_iter)]


def _time_calls(torch, fn, n_iter, n_copy):
    """Median and min microseconds of fn(i) over n_iter calls (copy i % n_copy);
    the stream is primed with a GPU sleep so that each event pair brackets GPU
    work only."""
    for i in range(3):
        fn(i % n_copy)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_iter + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    evs[0].record()
    for i in range(n_iter):
        fn(i % n_copy)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ts = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_iter))
    return ts[len(ts) // 2], ts[0]


def profile_shapes(args, torch, w8, synthetic):
    """The fused linear w8a8_linear on each named workload shape, `iters`
    back-to-back calls with weight copies rotated past the last-level cache,
    for rocprofv3 counter and trace runs (one dispatch per kernel per call)."""
    dev = "cuda:0"
    names = args.profile_shapes.split(",")
    shapes = {s.name: s for v in synthetic.CONFIGS.values() for s in v}
    for name in names:
        s = shapes[name]
        st = synthetic.streams(0, s.config_id, s.layer_id)
        x = synthetic.activations_bf16(st, s.M, s.K, s.outlier_frac).to(dev)
        w = torch.from_numpy(synthetic.weights_f32(st, s.N, s.K)).to(dev)
        b = synthetic.bias_bf16(st, s.N).to(dev)
        wq, sw = w8.w8a8_quantize_weight(w)
        del w
        ncopy = max(1, min(64, -(-600_000_000 // (s.N * s.K))))
        ws_ = [(wq, sw)] + [(wq.clone(), sw.clone()) for _ in range(ncopy - 1)]
        y = torch.empty((s.M, s.N), dtype=torch.bfloat16, device=dev)
        work = torch.empty((w8.w8a8_linear_workspace_bytes(s.M, s.K),), dtype=torch.uint8, device=dev)
        med, mn = _time_calls(torch, lambda i: w8.w8a8_linear(x, ws_[i][0], ws_[i][1], b, out=y, workspace=work),
                              args.iters, ncopy)
        cfg = w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(s.M, s.N, s.K))
        print(json.dumps({"profile_shape": name, "M": s.M, "K": s.K, "N": s.N, "gemm_config": cfg,
                          "linear_us_median": round(med, 2), "linear_us_min": round(mn, 2),
                          "calls": args.iters + 3}), flush=True)
        del ws_, x, y, work


def interlayer_ab(args, torch, w8, synthetic):
    """In-step A/B of the inter-layer fusion (the MLP step with the up-proj
    GEMM and the down-proj GEMM unchanged):
      A: gemm_dequant(up) -> y;  gelu_quantize_act(y) -> q_h
      B: gemm_dequant_gelu_amax(up) -> h, amax;  quantize_act_amax(h, amax) -> q_h
    Blocks of `steps` steps alternate A, B, A, B, ... (`rounds` pairs) after
    `warmup` steps of each; every step is bracketed by an event pair, and the
    up-proj + inter-layer segment by another.  Reports the means per variant."""
    up, down, inp = make_inputs(torch, w8, synthetic, args.rotate)
    stream = torch.cuda.current_stream()
    h = torch.empty_like(inp["y_up"])
    amax = torch.empty((up.M,), dtype=torch.int32, device="cuda:0")

    def step(i, variant, ev):
        wu, su = inp["w_up"][i % len(inp["w_up"])]
        wd, sd = inp["w_down"][i % len(inp["w_down"])]
        ev[0].record(stream)
        w8.w8a8_quantize_act(inp["x_up"], inp["q_x"], inp["s_x"])
        if variant == "A":
            w8.w8a8_gemm_dequant(inp["q_x"], inp["s_x"], wu, su, inp["b_up"], out=inp["y_up"])
            w8.w8a8_gelu_quantize_act(inp["y_up"], inp["q_h"], inp["s_h"])
        else:
            w8.w8a8_gemm_dequant_gelu_amax(inp["q_x"], inp["s_x"], wu, su, inp["b_up"], h_out=h, amax=amax)
            w8.w8a8_quantize_act_amax(h, amax, inp["q_h"], inp["s_h"])
        ev[1].record(stream)
        w8.w8a8_gemm_dequant(inp["q_h"], inp["s_h"], wd, sd, inp["b_down"], out=inp["y_down"])
        ev[2].record(stream)

    res = {"A": [[], []], "B": [[], []]}
    for v in ("A", "B"):
        for i in range(args.warmup):
            step(i, v, [torch.cuda.Event(enable_timing=True) for _ in range(3)])
    rounds = 3
    for r in range(rounds):
        for v in ("A", "B"):
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
            for i in range(args.steps):
                step(i, v, evs[i])
            torch.cuda.synchronize()
            res[v][0] += [e[0].elapsed_time(e[2]) * 1e3 for e in evs]
            res[v][1] += [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    out = {"interlayer_ab": "dit1024_mlp", "steps_per_block": args.steps, "rounds": rounds}
    for v, name in (("A", "gelu_quantize_pass"), ("B", "gelu_amax_epilogue")):
        out[name] = {"step_us": round(sum(res[v][0]) / len(res[v][0]), 2),
                     "quantize_up_gelu_quantize_us": round(sum(res[v][1]) / len(res[v][1]), 2)}
    print(json.dumps(out), flush=True)


def fake_int8_forward(w8, x, wq, sw, bias, operands=False):
    """The "fake INT8" forward the pages start from (Abstract; news write-up,
    second paragraph): the same per-token int8 quantization of x, then the
    activation and weight codes dequantized to bf16 (code * scale in fp32,
    rounded to bf16) and a bf16 GEMM through torch (hipBLASLt), bias added by
    the GEMM.  With `operands`, also returns the two dequantized matrices."""
    import torch
    import torch.nn.functional as F
    q, sx = w8.w8a8_quantize_act(x)
    xd = (q.float() * sx[:, None]).to(torch.bfloat16)
    wd = (wq.float() * sw[:, None]).to(torch.bfloat16)
    y = F.linear(xd, wd, bias)
    return (y, xd, wd) if operands else y


def compare(args, torch, w8, synthetic):
    """The pages' per-GEMM comparison on MI355X.  For each workload shape, from
    the same bf16 activations, int8 weights + per-channel scales and bf16 bias:
      int8:  the fused linear (per-token quantize, int8 GEMM, fused epilogue);
      fake:  the 'fake INT8' forward the pages start from -- the same per-token
             quantization, then activations and weights dequantized to bf16
             and a bf16 GEMM (torch / hipBLASLt), bias added by the GEMM;
      bf16:  a plain bf16 GEMM on the unquantized bf16 weights.
    Weight copies rotate past the 256 MB last-level cache for every leg; the
    legs are timed in 3 interleaved rounds (median over all their calls)."""
    import torch.nn.functional as F
    dev = "cuda:0"
    shapes = [s for k, v in synthetic.CONFIGS.items() if k != "unit" for s in v]
    if args.shapes:
        shapes = [s for s in shapes if s.name in args.shapes.split(",")]
    for s in shapes:
        st = synthetic.streams(0, s.config_id, s.layer_id)
        x = synthetic.activations_bf16(st, s.M, s.K, s.outlier_frac).to(dev)
        w = torch.from_numpy(synthetic.weights_f32(st, s.N, s.K)).to(dev)
        b = synthetic.bias_bf16(st, s.N).to(dev)
        wq, sw = w8.w8a8_quantize_weight(w)
        wq8, sw8 = w8.w8a8_quantize_weight_fp8(w)
        wb = w.to(torch.bfloat16)
        del w
        n8 = max(1, min(64, -(-600_000_000 // (s.N * s.K))))
        n16 = max(1, min(64, -(-600_000_000 // (2 * s.N * s.K))))
        w8s = [(wq, sw)] + [(wq.clone(), sw.clone()) for _ in range(n8 - 1)]
        wf8 = [(wq8, sw8)] + [(wq8.clone(), sw8.clone()) for _ in range(n8 - 1)]
        wbs = [wb] + [wb.clone() for _ in range(n16 - 1)]
        y = torch.empty((s.M, s.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((w8.w8a8_linear_workspace_bytes(s.M, s.K),), dtype=torch.uint8, device=dev)

        def int8(i):
            w8.w8a8_linear(x, w8s[i][0], w8s[i][1], b, out=y, workspace=ws)

        def fp8(i):
            w8.w8a8_linear_fp8(x, wf8[i][0], wf8[i][1], b, out=y, workspace=ws)

        def fake(i):
            return fake_int8_forward(w8, x, w8s[i][0], w8s[i][1], b)

        def bf16(i):
            return F.linear(x, wbs[i], b)

        # the legs take turns: 3 rounds of sweep_iters calls each, the order
        # reversed every other round, so that none of them is always timed
        # first after the shape's setup (the chip's clock settles over a run)
        legs = [("int8", int8, n8), ("fp8", fp8, n8), ("fake", fake, n8), ("bf16", bf16, n16)]
        for _, fn, nc in legs:
            for i in range(3):
                fn(i % nc)
        calls = {name: [] for name, _, _ in legs}
        for rnd in range(3):
            for name, fn, nc in (legs if rnd % 2 == 0 else legs[::-1]):
                calls[name] += _call_times(torch, fn, args.sweep_iters, nc)
        t8, tf8, tf, tb = ((_median(calls[n]), min(calls[n])) for n in ("int8", "fp8", "fake", "bf16"))
        int8(0)
        yf = fake(0)
        cos = F.cosine_similarity(y.float().flatten(), yf.float().flatten(), dim=0).item()
        ops = 2.0 * s.M * s.N * s.K
        print(json.dumps({"compare": s.name, "M": s.M, "K": s.K, "N": s.N,
                          "int8_fused_us": round(t8[0], 2), "fp8_fused_us": round(tf8[0], 2),
                          "fake_int8_us": round(tf[0], 2),
                          "bf16_us": round(tb[0], 2),
                          "int8_TOPS": round(ops / t8[0] / 1e6, 1), "bf16_TFLOPS": round(ops / tb[0] / 1e6, 1),
                          "speedup_vs_fake_int8": round(tf[0] / t8[0], 2),
                          "speedup_vs_bf16": round(tb[0] / t8[0], 2),
                          "cos_int8_vs_fake": round(cos, 6)}), flush=True)
        del w8s, wf8, wbs, ws, y, x, wq, sw, wq8, sw8, wb


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer "
              f"would shard over tokens or output channels, with no communication between GPUs).",
              file=sys.stderr)
        return 2

    import torch

    import synthetic
    import w8a8_int8_quantized_quantize_amd as w8

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return 0
    if args.sweep:
        sweep(args, torch, w8, synthetic)
        return 0
    if args.compare:
        compare(args, torch, w8, synthetic)
        return 0
    if args.profile_shapes:
        profile_shapes(args, torch, w8, synthetic)
        return 0
    if args.interlayer:
        interlayer_ab(args, torch, w8, synthetic)
        return 0

    up, down, inp = make_inputs(torch, w8, synthetic, args.rotate, args.fp8)
    stream = torch.cuda.current_stream()
    if args.fp8:
        quantize, gemm, gelu_quantize, linear = (w8.w8a8_quantize_act_fp8, w8.w8a8_gemm_dequant_fp8,
                                                 w8.w8a8_gelu_quantize_act_fp8, w8.w8a8_linear_fp8)
    else:
        quantize, gemm, gelu_quantize, linear = (w8.w8a8_quantize_act, w8.w8a8_gemm_dequant,
                                                 w8.w8a8_gelu_quantize_act, w8.w8a8_linear)
    ws = torch.empty((w8.w8a8_linear_workspace_bytes(up.M, up.K),), dtype=torch.uint8, device="cuda:0")
    ws_codes = ws[:up.M * up.K].view(inp["q_x"].dtype).view(up.M, up.K)

    # One step.  fused=True: the up-projection through the fused entry
    # w8a8_linear (quantize into the workspace + GEMM), an event pair around
    # the call (ev_lin).  fused=False: the same two kernels through their own
    # entry points, so that an event pair (ev_up) brackets the GEMM kernel
    # alone.  ev: 5 events around every kernel (breakdown pass only).
    def step(i, fused, ev=None, ev_up=None, ev_lin=None):
        wu, su = inp["w_up"][i % len(inp["w_up"])]
        wd, sd = inp["w_down"][i % len(inp["w_down"])]
        if fused:
            if ev_lin is not None:
                ev_lin[0].record(stream)
            linear(inp["x_up"], wu, su, inp["b_up"], out=inp["y_up"], workspace=ws)
            if ev_lin is not None:
                ev_lin[1].record(stream)
        else:
            if ev is not None:
                ev[0].record(stream)
            quantize(inp["x_up"], inp["q_x"], inp["s_x"])
            if ev is not None:
                ev[1].record(stream)
            if ev_up is not None:
                ev_up[0].record(stream)
            gemm(inp["q_x"], inp["s_x"], wu, su, inp["b_up"], out=inp["y_up"])
            if ev_up is not None:
                ev_up[1].record(stream)
            if ev is not None:
                ev[2].record(stream)
        gelu_quantize(inp["y_up"], inp["q_h"], inp["s_h"])
        if ev is not None:
            ev[3].record(stream)
        gemm(inp["q_h"], inp["s_h"], wd, sd, inp["b_down"], out=inp["y_down"])
        if ev is not None:
            ev[4].record(stream)

    def pairs(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]

    for i in range(args.warmup):
        step(i, True)
    # timed region 1: the step through the fused entry (value, ms_per_step)
    lin_events = pairs(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True, ev_lin=lin_events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # timed region 2: the same step with the up-projection's two kernels
    # issued through their own entry points, the GEMM kernel event-timed
    up_events = pairs(args.steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(i, False, ev_up=up_events[i])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    # per-kernel breakdown: the same steps again, every kernel bracketed (untimed)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, False, events[i])
    torch.cuda.synchronize()
    # the fused entry wrote the same codes and scales as the split one
    assert torch.equal(ws_codes, inp["q_x"]), "fused and split up-projection disagree"

    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_split = (t3 - t2) * 1e3 / args.steps
    lin_ms = sum(ev[0].elapsed_time(ev[1]) for ev in lin_events) / args.steps
    up_ms = sum(ev[0].elapsed_time(ev[1]) for ev in up_events) / args.steps
    seg = [[ev[j].elapsed_time(ev[j + 1]) for ev in events] for j in range(4)]
    avg = [sum(s) / len(s) for s in seg]
    ops_up = 2.0 * up.M * up.N * up.K
    ops_down = 2.0 * down.M * down.N * down.K
    value = (ops_up + ops_down) / (ms_step * 1e-3) / 1e12
    gemm_up_tops = ops_up / (up_ms * 1e-3) / 1e12
    lin_tops = ops_up / (lin_ms * 1e-3) / 1e12
    gemm_down_tops = ops_down / (avg[3] * 1e-3) / 1e12
    q_bytes = 3.0 * up.M * up.K + 4 * up.M
    g_bytes = 3.0 * down.M * down.K + 4 * down.M

    up_cfg = w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(up.M, up.N, up.K))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if args.fp8 else "int8",
        "data": "synthetic",
        "config": {"workload": "dit1024_mlp: 4096 tokens; up-proj K=3072 N=12288; "
                               "GELU+requantize of its output; down-proj K=12288 N=3072",
                   "M": up.M, "hidden": up.K, "mlp": up.N, "weight_copies_rotated": args.rotate},
        "roofline": {"bound": "mfma", "achieved": round(gemm_up_tops, 1), "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": round(gemm_up_tops / PEAK_INT8_TOPS, 4),
                     "traffic": traffic_entry(),
                     "kernel": f"{up_kernel_name(up_cfg)}...> ({up_cfg}), up-proj M=4096 K=3072 "
                               "N=12288 (int8 ops per launch 2*M*N*K / mean HIP-event duration)"},
        # the fused entry w8a8_linear at the headline shape (quantize + GEMM +
        # epilogue, one call), event-timed in every step of timed region 1
        "fused_linear": {"entry": "w8a8_linear", "M": up.M, "K": up.K, "N": up.N,
                         "us": round(lin_ms * 1e3, 2), "TOPS": round(lin_tops, 1),
                         "frac": round(lin_tops / PEAK_INT8_TOPS, 4)},
        # the up-proj GEMM kernel in timed region 2 (the roofline's figure), and
        # every kernel in the untimed pass with all kernels bracketed
        "gemm_up_ms_timed": round(up_ms, 4),
        "ms_per_step_split_entries": round(ms_step_split, 4),
        "kernels_ms": {"quantize_x": round(avg[0], 4), "gemm_up": round(avg[1], 4),
                       "gelu_quantize": round(avg[2], 4), "gemm_down": round(avg[3], 4)},
        "per_kernel": {
            "gemm_up_TOPS": round(gemm_up_tops, 1), "gemm_down_TOPS": round(gemm_down_tops, 1),
            "quantize_x_GBs": round(q_bytes / (avg[0] * 1e-3) / 1e9, 1),
            "gelu_quantize_GBs": round(g_bytes / (avg[2] * 1e-3) / 1e9, 1),
            "gemm_up_config": w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(up.M, up.N, up.K)),
            "gemm_down_config": w8.w8a8_gemm_config_name(w8.w8a8_gemm_select_config(down.M, down.N, down.K)),
        },
    }
    if args.fp8:
        # the FP8 step: same workload on the e4m3 path (fp8 dense peak 5.0 PFLOP/s);
        # no counters or CPU baseline for it
        out["metric"] = METRIC + " (FP8 e4m3 variant)"
        out["unit"] = "TFLOPS"
        out["roofline"].update({"unit": "TFLOP/s", "traffic": None,
                                "kernel": "gemm_kernel (FP8), up-proj M=4096 K=3072 N=12288"})
        out["per_kernel"].pop("gemm_up_config")
        out["per_kernel"].pop("gemm_down_config")
        args.no_cpu_baseline = True
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(up, down, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
