"""Benchmark of the fp32 convolution hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]

One "step" is one call of the library's entry point over one batch of the
headline workload, the long strided and dilated Conv1d (x[64,64,524280],
w[128,64,3], stride 3, dilation 4), the largest configuration. The same run
also times every other workload and reports it under "shapes":

* the tiny, general and asymmetric Conv3d and the fused Conv3d+min+softmax;
* the four plain convolutions and the fused op again on channels-last tensors
  through conv_fwd_channels_last and conv3d_min_softmax_channels_last
  ("<workload>_channels_last");
* the five workloads on the generic kernels, with the build-time
  specialisations switched off ("<workload>_generic", CONVHIP_TAP=0);
* the four plain convolutions on the vector-ALU direct kernel
  ("<workload>_valu", CONVHIP_VALU=1): the per-shape comparison of the vector
  ALU with the matrix cores;
* neighbouring shapes that no specialisation was built for, and the fused op
  with the minimum over H or W and with groups (synth.VARIANTS).

Inputs are seeded synthetic tensors already resident in device memory; each
entry is first run back to back for at least 0.5 s (the GPU's clocks ramp up
from idle over that time), then the timed region is K back-to-back calls
between two device synchronisations, timed with events on the stream the
kernels are launched on. Each entry also reports the median of single launches
after a 512 MiB write that evicts L2 and the MALL (ms_cold_median).

Prints one JSON line. Throughput = 2 * MACs / time, with MACs = outputs x
(C_in/groups) x kernel volume (every tap, padded ones included). Each entry
carries a roofline object against MI355X's published fp32 matrix peak
(157.3 TFLOP/s) and, where a counter summary of the current sources exists,
the HBM bytes one launch moves. The CPU baseline is the fp64 oracle on the
headline's batch slice n in {0, 63}, timed on the host cores; the headline's
parity is checked on the same slice.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3
WARM_S = 0.5  # default seconds of warm-up calls per workload (--warm-seconds)
PEAK_HBM_GBS = 8000.0
HEADLINE = "long_conv1d"
HEADLINE_SLICE = (0, 63)  # batch samples the oracle computes for the CPU baseline and parity
CL_SUFFIX = "_channels_last"
GEN_SUFFIX = "_generic"
VALU_SUFFIX = "_valu"
VALU_WORKLOADS = ("tiny_conv3d", "general_conv3d", "asym_conv3d", "long_conv1d")
WORKLOAD_NAMES = ["tiny_conv3d", "general_conv3d", "conv3d_min_softmax", "asym_conv3d", "long_conv1d"]
ORDER = (WORKLOAD_NAMES
         + [n + CL_SUFFIX for n in ("tiny_conv3d", "general_conv3d", "asym_conv3d", "long_conv1d",
                                    "conv3d_min_softmax")]
         + [n + GEN_SUFFIX for n in WORKLOAD_NAMES]
         + [n + VALU_SUFFIX for n in VALU_WORKLOADS]
         + ["asym_conv3d_48", "general_conv3d_24", "long_conv1d_c96_d2", "conv3d_min_softmax_min_h",
            "conv3d_min_softmax_min_w", "conv3d_min_softmax_groups3"])
KERNEL_SOURCES = [os.path.join(ROOT, "implicit_gemm_convolution_direct_amd", "csrc", f)
                  for f in ("conv_kernels.hip", "valu_kernels.hip", "convhip_plan.cpp", "convhip_plan.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def geometry(cfg):
    """Output shape, MACs and algorithmic bytes (x, w, bias read once, y written once).
    MACs count (C_in/groups) x kernel volume per conv output: a grouped conv does
    no products across groups."""
    xs, ws = cfg["x"], cfg["w"]
    nd = cfg["nd"]
    out = []
    for a in range(nd):
        L, k, s, d, p = xs[2 + a], ws[2 + a], cfg["stride"][a], cfg["dilation"][a], cfg["padding"][a]
        out.append((L + 2 * p - d * (k - 1) - 1) // s + 1)
    kred = int(np.prod(ws[1:]))
    conv_elems = xs[0] * ws[0] * int(np.prod(out))
    macs = conv_elems * kred
    if cfg["fused"]:
        md = cfg.get("min_dim", 2)
        y_elems = xs[0] * ws[0] * int(np.prod([o for a, o in enumerate(out) if a != md - 2]))
    else:
        y_elems = conv_elems
    nbytes = 4 * (int(np.prod(xs)) + int(np.prod(ws)) + (ws[0] if cfg["bias"] else 0) + y_elems)
    return out, macs, nbytes, conv_elems, y_elems


def read_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def split_name(name):
    """(workload, channels_last, mode): a "<workload>_channels_last" entry times
    the same workload with x [N, spatial..., C_in] and y [N, out..., C_out]; a
    "<workload>_generic" entry (mode "generic") times it with the build-time
    specialisations off; a "<workload>_valu" entry (mode "valu") on the
    vector-ALU direct kernel. mode is None otherwise."""
    if name.endswith(CL_SUFFIX):
        return name[:-len(CL_SUFFIX)], True, None
    if name.endswith(GEN_SUFFIX):
        return name[:-len(GEN_SUFFIX)], False, "generic"
    if name.endswith(VALU_SUFFIX):
        return name[:-len(VALU_SUFFIX)], False, "valu"
    return name, False, None


def roofline(tflops, name, latency_bound=False):
    """The roofline object of one entry: the fp32 matrix cores, or for "_valu"
    entries the vector ALU ("alu"; its fp32 peak is the same 157.3 TFLOP/s);
    tiny Conv3d: launch latency binds before either peak."""
    bound = "alu" if split_name(name)[2] == "valu" else "mfma"
    rec = {"bound": bound, "achieved": tflops, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tflops / PEAK_FP32_TFLOPS, 4), "traffic": read_traffic(name)}
    if latency_bound:
        rec["limited_by"] = "launch latency"
    return rec


def make_device_inputs(name, torch, ch, synth, channels_last=False):
    cfg = synth.config(name)
    dev = torch.device("cuda:0")
    sx, sw, sb = cfg["seeds"]
    xs = cfg["x"]
    if channels_last:
        xs = (xs[0], *xs[2:], xs[1])
    x = torch.empty(xs, dtype=torch.float32, device=dev)
    ch.synth_fill(x, sx, ch.KIND_UNIFORM01)
    fan = synth.fan_in(cfg["w"])
    w = torch.empty(cfg["w"], dtype=torch.float32, device=dev)
    ch.synth_fill(w, sw, ch.KIND_SYMMETRIC, bound=synth.symmetric_bound(fan))
    b = None
    if cfg["bias"]:
        b = torch.empty((cfg["w"][0],), dtype=torch.float32, device=dev)
        ch.synth_fill(b, sb, ch.KIND_SYMMETRIC, bound=synth.symmetric_bound(fan))
    return cfg, x, w, b


def time_workload(name, steps, warmup, torch, ch, synth, flush=None, warm_s=WARM_S):
    base, cl, mode = split_name(name)
    # Switches read by the library at every call.
    var = {"generic": ("CONVHIP_TAP", "0"), "valu": ("CONVHIP_VALU", "1")}.get(mode)
    saved = os.environ.get(var[0]) if var else None
    if var:
        os.environ[var[0]] = var[1]
    try:
        return _time_workload(name, base, cl, steps, warmup, torch, ch, synth, flush, warm_s)
    finally:
        if var:
            if saved is None:
                del os.environ[var[0]]
            else:
                os.environ[var[0]] = saved


def _time_workload(name, base, cl, steps, warmup, torch, ch, synth, flush, warm_s):
    cfg, x, w, b = make_device_inputs(base, torch, ch, synth, channels_last=cl)
    out, macs, nbytes, conv_elems, y_elems = geometry(cfg)
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    md = cfg.get("min_dim", 2)
    if cl and cfg["fused"]:
        keep = [o for a, o in enumerate(out) if a != md - 2]
        y = torch.empty((cfg["x"][0], *keep, cfg["w"][0]), dtype=torch.float32, device=x.device)
        call = lambda: ch.conv3d_min_softmax_channels_last(x, w, b, *args, min_dim=md, out=y)
    elif cl:
        y = torch.empty((cfg["x"][0], *out, cfg["w"][0]), dtype=torch.float32, device=x.device)
        call = lambda: ch.conv_fwd_channels_last(x, w, b, *args, out=y)
    elif cfg["fused"]:
        keep = [o for a, o in enumerate(out) if a != md - 2]
        y = torch.empty((cfg["x"][0], cfg["w"][0], *keep), dtype=torch.float32, device=x.device)
        call = lambda: ch.conv3d_min_softmax(x, w, b, *args, min_dim=md, out=y)
    else:
        y = torch.empty((cfg["x"][0], cfg["w"][0], *out), dtype=torch.float32, device=x.device)
        call = lambda: ch.conv_fwd(x, w, b, *args, out=y)
    # Warm-up: at least `warmup` calls and WARM_S seconds of back-to-back calls, so
    # the GPU's clocks have left their idle state before the timed region.
    t_w = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_w < warm_s:
        for _ in range(8):
            call()
        done += 8
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # Per-launch durations of a few isolated launches, for the spread.
    singles = []
    for _ in range(min(steps, 10)):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        z.record(stream)
        torch.cuda.synchronize()
        singles.append(a.elapsed_time(z))
    # Cold caches: a 512 MiB write (more than L2 + MALL) before each timed launch.
    colds = []
    if flush is not None:
        for _ in range(min(steps, 10)):
            flush.fill_(1.0)
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            z.record(stream)
            torch.cuda.synchronize()
            colds.append(a.elapsed_time(z))
    tflops = 2.0 * macs / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    plan = ch.plan_describe(tuple(x.shape), cfg["w"], *args, fused=cfg["fused"], channels_last=cl, min_dim=md)
    rec = {
        "workload": name,
        "plan": plan,
        "ms": round(ms, 5),
        "ms_single_min": round(min(singles), 5),
        "ms_single_max": round(max(singles), 5),
        "ms_cold_median": round(float(np.median(colds)), 5) if colds else None,
        "tflops": round(tflops, 3),
        "gbs": round(gbs, 1),
        "frac_fp32_peak": round(tflops / PEAK_FP32_TFLOPS, 4),
        "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "macs": macs,
        "alg_bytes": nbytes,
        "wall_s": round(wall, 3),
        "roofline": roofline(round(tflops, 3), name, latency_bound=base == "tiny_conv3d"),
    }
    if cfg["fused"] and not cl:
        # Unfused chain: conv writes the 5-D result, min reads it and writes its
        # result, softmax reads and writes that (algorithmic bytes).
        unfused = 4 * (int(np.prod(cfg["x"])) + int(np.prod(cfg["w"])) + cfg["w"][0]
                       + 2 * conv_elems + 3 * y_elems)
        rec["unfused_alg_bytes"] = unfused
        rec["fused_traffic_ratio_alg"] = round(unfused / nbytes, 2)
    del x, w, b, y
    torch.cuda.empty_cache()
    return rec, macs


def calibrate(torch, ch, seconds=0.05):
    """Rates this chip reaches in practice: fp32 matrix-core and vector-FMA
    throughput from the library's probes (each launch sized to about `seconds`),
    and HBM bandwidth from a plain 1 GiB device-to-device copy (2 bytes moved per
    byte copied). Each is the best of 5 timed repetitions after 0.3 s of warm-up."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    out = {}

    def best_rate(run, work):
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.3:
            run()
            torch.cuda.synchronize()
        rates = []
        for _ in range(5):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            z.record(stream)
            torch.cuda.synchronize()
            rates.append(work / (a.elapsed_time(z) * 1e-3))
        return max(rates)

    for key, kind, guess in (("mfma_f32_tflops", ch.PROBE_MFMA_F32, PEAK_FP32_TFLOPS),
                             ("fma_f32_tflops", ch.PROBE_FMA_F32, PEAK_FP32_TFLOPS / 2)):
        # Size the launch from the published rate: about `seconds` of work.
        flop1 = ch.peak_probe(kind, 1, sink)
        iters = min(1 << 22, max(1, int(seconds * guess * 1e12 / flop1)))
        flop = flop1 * iters
        out[key] = round(best_rate(lambda: ch.peak_probe(kind, iters, sink), flop) / 1e12, 2)
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    out["hbm_copy_gbs"] = round(best_rate(lambda: dst.copy_(src), 2.0 * 4 * n) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def headline_slice_inputs(name, samples):
    """Host copies of the given batch samples of a workload's input (the same
    seeded stream the device generator fills), and its weights and bias."""
    import synth
    cfg = synth.WORKLOADS[name]
    sx = cfg["seeds"][0]
    per = int(np.prod(cfg["x"][1:]))
    x = np.concatenate([synth.uniform01(sx, (1, *cfg["x"][1:]), start=n * per) for n in samples])
    _, w, b = synth.make_inputs(name, n_samples=1)
    return cfg, x, w, b


def cpu_baseline(name, samples, seconds=10.0):
    """The fp64 oracle on a batch slice of the headline workload, timed on the
    host cores for about `seconds`; returns the record and the slice's result."""
    import oracle
    cfg, x, w, b = headline_slice_inputs(name, samples)
    _, macs_full, _, _, _ = geometry(cfg)
    macs = macs_full // cfg["x"][0] * len(samples)
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    oracle.conv(x[:1, :, :64], w, b, *args)  # load the library, start the threads
    reps = 0
    t0 = time.perf_counter()
    while reps < 1 or time.perf_counter() - t0 < seconds:
        ref = oracle.conv(x, w, b, *args)
        reps += 1
    t = (time.perf_counter() - t0) / reps
    return {"value": round(2.0 * macs / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{name} batch samples n in {list(samples)} of {cfg['x'][0]} (full length), "
                      f"{macs} MAC per pass, fp64 nested loops, {reps} pass(es), {t:.3f} s per pass; "
                      f"full workload extrapolated: {t * cfg['x'][0] / len(samples):.1f} s"}, x, ref


def headline_parity(name, samples, ref, torch, ch, synth):
    """The headline call at full size (input generated on the device) against
    the oracle's result on the batch slice."""
    cfg, x, w, b = make_device_inputs(name, torch, ch, synth)
    y = ch.conv_fwd(x, w, b, cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    torch.cuda.synchronize()
    err = 0.0
    for i, n in enumerate(samples):
        err = max(err, float(np.abs(y[n].cpu().numpy().astype(np.float64) - ref[i]).max()))
    tol = 1e-4 * math.sqrt(int(np.prod(cfg["w"][1:]))) * float(np.abs(ref).max())
    del x, w, b, y
    torch.cuda.empty_cache()
    return {"max_abs_err": err, "tol": tol, "pass": err <= tol, "compared": f"batch samples {list(samples)}"}


def cpu_baselines_per_workload(shapes, seconds=1.0):
    """The fp64 oracle on one sample of each workload (channels-first), timed on
    the host cores for about `seconds` each: its FLOP rate, the full workload's
    time extrapolated from it, and the GPU's speed-up over it."""
    import oracle
    import synth
    out = {}
    for name in ("tiny_conv3d", "general_conv3d", "conv3d_min_softmax", "asym_conv3d", "long_conv1d"):
        cfg = synth.WORKLOADS[name]
        x, w, b = synth.make_inputs(name, n_samples=1)
        _, macs_full, _, _, _ = geometry(cfg)
        macs = macs_full // cfg["x"][0]
        args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
        run = (lambda: oracle.conv3d_min_softmax(x, w, b, *args)) if cfg["fused"] else \
              (lambda: oracle.conv(x, w, b, *args))
        reps = 0
        t0 = time.perf_counter()
        while reps < 1 or time.perf_counter() - t0 < seconds:
            run()
            reps += 1
        t = (time.perf_counter() - t0) / reps
        full_s = t * cfg["x"][0]
        rec = {"tflops": round(2.0 * macs / t / 1e12, 6), "cores": oracle.num_threads(),
               "sample": f"sample 0 of {cfg['x'][0]}, {reps} pass(es), {1e3 * t:.4g} ms per pass",
               "full_s_extrapolated": float(f"{full_s:.4g}")}
        if name in shapes:
            rec["gpu_over_cpu"] = round(full_s / (shapes[name]["ms"] * 1e-3), 1)
        out[name] = rec
        del x, w, b
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=ORDER, default=None, help="time one workload only (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--warm-seconds", type=float, default=WARM_S,
                    help="minimum seconds of back-to-back warm-up calls per workload")
    ap.add_argument("--unfused-chain", action="store_true",
                    help="only run the fused workload as three separate launches (conv_fwd writing the 5-D "
                         "result, min_over_axis over depth, softmax_over_channels) and time the chain and each "
                         "step; for measuring the HBM traffic the fused kernel avoids")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes per step "
                         "(calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE against a known traffic)")
    ap.add_argument("--calibrate-only", action="store_true",
                    help="only run the calibration probes (matrix-core and vector-FMA throughput, copy bandwidth) "
                         "and print their rates; for collecting counters on the probes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the convolution "
              "would shard over the batch, each GPU computing its own samples with no exchange). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import implicit_gemm_convolution_direct_amd as ch
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ch.lib()

    if args.calibrate_only:
        print(json.dumps({"calibration": calibrate(torch, ch)}), flush=True)
        return
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "steps": args.warmup + args.steps}), flush=True)
        return

    if args.unfused_chain:
        name = "conv3d_min_softmax"
        cfg, x, w, b = make_device_inputs(name, torch, ch, synth)
        args4 = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
        y5 = ch.conv_fwd(x, w, b, *args4)
        m = ch.min_over_axis(y5, 2)
        sm = ch.softmax_over_channels(m)
        steps = {
            "conv_fwd": lambda: ch.conv_fwd(x, w, b, *args4, out=y5),
            "min_over_axis": lambda: ch.min_over_axis(y5, 2, out=m),
            "softmax_over_channels": lambda: ch.softmax_over_channels(m, out=sm),
        }

        def chain():
            for f in steps.values():
                f()

        fused = ch.conv3d_min_softmax(x, w, b, *args4)
        chain()
        err = float((sm - fused).abs().max())
        stream = torch.cuda.current_stream()

        def timed(f):
            for _ in range(args.warmup):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        nbytes = {"conv_fwd": 4 * (x.numel() + w.numel() + (b.numel() if b is not None else 0) + y5.numel()),
                  "min_over_axis": 4 * (y5.numel() + m.numel()),
                  "softmax_over_channels": 4 * 2 * m.numel()}
        per = {}
        for k, f in steps.items():
            ms = timed(f)
            per[k] = {"ms": round(ms, 5), "alg_bytes": nbytes[k], "gbs": round(nbytes[k] / ms / 1e6, 1)}
        print(json.dumps({"unfused_chain": name, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_chain": round(timed(chain), 5), "per_step": per,
                          "max_abs_diff_vs_fused": err}), flush=True)
        return

    names = [args.only] if args.only else ORDER
    shapes = {}
    head = None
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda:0")
    for name in names:
        print(f"[bench] timing {name}", file=sys.stderr, flush=True)
        rec, macs = time_workload(name, args.steps, args.warmup, torch, ch, synth, flush=flush,
                                  warm_s=args.warm_seconds)
        shapes[name] = rec
        print(f"[bench] {name}: {rec['ms']:.4f} ms  {rec['tflops']:.2f} TFLOP/s  "
              f"({100 * rec['frac_fp32_peak']:.1f}% of fp32 peak); cold caches {rec['ms_cold_median']} ms",
              file=sys.stderr, flush=True)
    if args.only:
        head = shapes[args.only]
        head_name = args.only
    else:
        head = shapes[HEADLINE]
        head_name = HEADLINE

    cpu = None
    cpu_all = None
    parity = None
    if not args.no_cpu and not args.only:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        cpu, _, ref = cpu_baseline(HEADLINE, HEADLINE_SLICE)
        # Parity of the headline launch against the oracle on the same seeded inputs.
        print("[bench] headline parity", file=sys.stderr, flush=True)
        parity = headline_parity(HEADLINE, HEADLINE_SLICE, ref, torch, ch, synth)
        del ref
        print("[bench] oracle CPU rate per workload (one sample each)", file=sys.stderr, flush=True)
        cpu_all = cpu_baselines_per_workload(shapes)

    # Achievable rates on this GPU, and each workload against them (the matrix
    # rate binds every workload here).
    achievable = None
    if not args.only:
        print("[bench] calibration probes", file=sys.stderr, flush=True)
        achievable = calibrate(torch, ch)
        for rec in shapes.values():
            rec["frac_achievable_mfma"] = round(rec["tflops"] / achievable["mfma_f32_tflops"], 4)
            rec["frac_achievable_hbm"] = round(rec["gbs"] / achievable["hbm_copy_gbs"], 4)

    cfgh = synth.config(split_name(head_name)[0])
    achieved = head["tflops"]
    line = {
        "metric": "conv fwd TFLOP/s (fp32) and % of MI355X FP32/HBM roofline per shape",
        "value": achieved,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "ms_per_step_cold": head["ms_cold_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64: x~U[0,1), w,b~U(+-1/sqrt(fan_in)))",
        "config": {"workload": head_name, "x": list(cfgh["x"]), "w": list(cfgh["w"]),
                   "stride": list(cfgh["stride"]), "padding": list(cfgh["padding"]),
                   "dilation": list(cfgh["dilation"]), "groups": cfgh["groups"], "bias": cfgh["bias"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "cpu_baseline_per_workload": cpu_all,
        "achievable": achievable,
        "parity": parity,
        "shapes": shapes,
        "kernel_src": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
