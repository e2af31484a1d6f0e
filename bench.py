#!/usr/bin/env python3
"""Benchmark of the fused NHWC conv2d hot path on one MI355X.

A step is one pass of the 640x640 YOLO layer stack (four 320x320x3 fp32
tiles mosaic-packed into a 640x640x3 bf16 canvas, then nine bf16 convs with
fused bias + Mish, N=1), captured once into a HIP graph and replayed. Each
3x3 layer that is followed by a 1x1 layer the library can fuse (L2+L3,
L5+L6) runs with it as one launch, so the graph has 8 nodes. All inputs,
weights and intermediate buffers are resident in device memory before the
timed region starts.

Prints ONE JSON line:
  value         TFLOP/s of the stack (26.5 GFLOP per step, every tap counted)
  ms_per_step   ms per 640x640 layer stack
  roofline      the dominant kernel (largest share of the step), timed with
                HIP events on the stream it runs on, against MI355X peaks
  cpu_baseline  the CPU oracle on the same stack: all host threads (median
                of 5 passes), with a 1-thread rung (median of 3)
  layers        per-node time and roofline fraction (a fused pair's bytes
                leave out the intermediate tensor it never stores)

  secondary     per-layer rates of the depthwise probe (vs the HBM peak) and
                of the N=16 YOLO sweep (vs the MFMA peak), measured after the
                step, each launch on its own buffer set (Infinity-Cache cold);
                the SPP, upsample+concat and residual kernels; the small
                stacks (digit classifier, keyword spotting, wake words) as
                microseconds per stack and per layer; the measured peaks
                (matrix-core probe, 1 GiB read+write stream)

Options: --gpus N (only 1 is supported), --steps K, --warmup W,
--workload NAME (another stack, for information), --no-cpu-baseline,
--no-secondary, --no-stacks (skip the small stacks of the secondary set),
--no-fuse (every layer its own launch),
--calib-copy MIB (run only a plain device copy of known size, for the
counter calibration of the traffic figure).
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

METRIC = "conv TFLOP/s (bf16) / TOPS (int8) + % MFMA or HBM peak; ms per 640² layer stack"
PEAK = {"bf16": 2500.0, "i8": 5000.0, "f32": 157.3}  # dense MFMA TFLOP/s (TOPS for int8)
HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="yolo640_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the depthwise-probe and N=16-sweep measurements")
    ap.add_argument("--no-stacks", action="store_true",
                    help="skip the small-stack timings of the secondary measurements")
    ap.add_argument("--no-fuse", action="store_true",
                    help="launch every layer on its own (no fused 3x3 + 1x1 pairs)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    """Digest of the HIP sources, to tell whether stored counter figures still
    describe the current kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_conv2d_nhwc_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_digest") != kernel_source_digest():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is a design note, not built)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calib_copy:
        from convolution_conv2d_nhwc_amd import _lib

        n = args.calib_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            _lib.probe_copy(a, b)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_kernel": "stream_copy_kernel", "calib_copy_bytes_read": n * 4,
                          "calib_copy_bytes_written": n * 4, "launches": 5}))
        return

    from convolution_conv2d_nhwc_amd import _lib
    from convolution_conv2d_nhwc_amd.data import workload
    from convolution_conv2d_nhwc_amd.stack import Stack

    wl = workload(args.workload)
    if not wl.chained:
        print("bench.py: the step is a chained stack; %s is not one" % wl.name, file=sys.stderr)
        sys.exit(2)

    # ---- resident inputs, weights and buffers; one step captured as a graph --
    # (a 3x3 layer and the 1x1 layer after it run as one fused launch)
    stack = Stack(wl, fuse=not args.no_fuse)
    convs, canvas = stack.convs, stack.canvas
    graph = stack.capture()

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: K graph replays ------------------------------------------
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    progress("%s: %.5f ms per step over %d graph replays" % (wl.name, ms_per_step, args.steps))

    # ---- per-kernel durations, inside the stack ----------------------------------
    dur_us, ev_gap_us = per_launch_us(stack.launches())

    layers = []
    j = 0
    if canvas is not None:
        m, th, tw, c = wl.mosaic
        # fp32 tiles read, the bf16 canvas written (padded to 8 channels for
        # the window stem kernel)
        mb = 4 * m * th * tw * c * 4 + m * 4 * th * tw * stack.canvas_c * 2
        layers.append({"name": "mosaic_pack", "kernel": stack.mosaic_kernel(), "us": dur_us[0],
                       "gflop": 0.0, "mbytes": mb / 1e6, "bound": "hbm",
                       "frac": (mb / (HBM_GBS * 1e9)) / (dur_us[0] * 1e-6)})
        j = 1
    for k, node in enumerate(stack.nodes()):
        us = dur_us[j + k]
        ls = [wl.layers[i] for i in node]
        fl = sum(l.flops() for l in ls)
        # a fused pair: the intermediate tensor is neither written nor read
        by = sum(l.bytes() for l in ls) - 2 * sum(l.n * l.ho * l.wo * l.cout * 2 for l in ls[:-1])
        name = "+".join(l.name for l in ls)
        if node == (0,) and stack.mosaic_fused:
            # the mosaic folded into the first layer: its input is the fp32
            # tiles, the canvas is never written
            m, th, tw, c = wl.mosaic
            l0 = ls[0]
            by += 4 * m * th * tw * c * 4 - l0.n * l0.h * l0.w * l0.cin * 2
            name = "mosaic_pack+" + name
        dt = ls[0].dtype
        t_mfma = fl / (PEAK[dt] * 1e12)
        t_hbm = by / (HBM_GBS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        desc = _lib.describe_fused(convs[node[0]], convs[node[1]]) if len(node) == 2 else convs[node[0]].describe()
        layers.append({"name": name, "kernel": stack.node_kernel(node),
                       "desc": desc, "us": us, "gflop": fl / 1e9, "mbytes": by / 1e6,
                       "tflops": fl / (us * 1e-6) / 1e12, "gbs": by / (us * 1e-6) / 1e9, "bound": bound,
                       "frac": max(t_mfma, t_hbm) / (us * 1e-6)})

    # dominant kernel = the kernel symbol with the largest time per step
    by_kernel = {}
    for L in layers:
        by_kernel.setdefault(L["kernel"], []).append(L)
    dom, dl = max(by_kernel.items(), key=lambda kv: sum(L["us"] for L in kv[1]))
    n_launch = len(dl)
    avg_us = sum(L["us"] for L in dl) / n_launch
    fl = sum(L["gflop"] for L in dl) * 1e9 / n_launch
    by = sum(L["mbytes"] for L in dl) * 1e6 / n_launch
    t_m = fl / (PEAK[wl.layers[0].dtype] * 1e12) if fl else 0.0
    t_h = by / (HBM_GBS * 1e9)
    if t_m >= t_h and fl:
        roof = {"bound": "mfma", "achieved": fl / (avg_us * 1e-6) / 1e12, "peak": PEAK[wl.layers[0].dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / (avg_us * 1e-6) / 1e9, "peak": HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(dom)
    roof["kernel"] = dom
    roof["launches_per_step"] = n_launch
    roof["avg_launch_us"] = avg_us
    roof["algorithmic_per_launch"] = {"flop": fl, "bytes": by}
    roof["event_gap_us"] = ev_gap_us
    # the same fraction against what this GPU measurably sustains (the
    # library's matrix-core probe and 1 GiB read+write stream)
    progress("measured peaks")
    peaks = measured_peaks()
    mp = peaks["copy"] if roof["bound"] == "hbm" else peaks["mfma_" + wl.layers[0].dtype]
    roof["measured_peak"] = dict(peaks, frac=roof["achieved"] / mp["value"])

    total_flop = wl.flops()
    value = total_flop / (ms_per_step * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        progress("CPU oracle ladder")
        cpu = cpu_baseline(wl)

    secondary = None if args.no_secondary else secondary_measurements(peaks, stacks=not args.no_stacks)

    dt = wl.layers[0].dtype
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s" if dt != "i8" else "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (wl.name, wl.description), "global_batch": wl.layers[0].n,
                   "input": "640x640x3 from 4x320x320x3" if wl.mosaic else "%dx%dx%d" % (
                       wl.layers[0].h, wl.layers[0].w, wl.layers[0].cin),
                   "gflop_per_step": total_flop / 1e9, "timing": "hipGraph replay, HIP events",
                   "graph_nodes": len(stack.launches()), "fused_pairs": ["+".join(wl.layers[i].name for i in n)
                                                                        for n in stack.nodes() if len(n) == 2],
                   "mosaic_folded_into_first_layer": stack.mosaic_fused,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in L.items() if k != "desc"}
                   for L in layers],
        "secondary": secondary,
        "wall_s_timed": round(wall, 4),
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


def per_launch_us(seq, T=20):
    """Average duration of each launch of `seq` (single-kernel closures run in
    order), over T eager passes with a timing event after every launch. A spin
    kernel first holds the stream while the host enqueues all of it, so the
    kernels run back to back as in the graph, each reading what the previous
    one just wrote, and the interval between consecutive events is one
    kernel's duration. An event between two kernels delays the second by a
    little; a pair of events with nothing between them measures that delay,
    which is taken off every interval. Returns (durations in us, that delay)."""
    import torch

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 2)] for _ in range(T)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for t in range(T):
        evs[t][0].record()
        evs[t][1].record()
        for k, fn in enumerate(seq):
            fn()
            evs[t][k + 2].record()
    torch.cuda.synchronize()
    ev_gap_us = sum(evs[t][0].elapsed_time(evs[t][1]) for t in range(T)) * 1000.0 / T
    dur_us = [sum(evs[t][k + 1].elapsed_time(evs[t][k + 2]) for t in range(T)) * 1000.0 / T - ev_gap_us
              for k in range(len(seq))]
    return dur_us, ev_gap_us


def graph_median_us(fn_list, reps=200, warmup=20):
    """Microseconds of one replay of `fn_list` captured as one graph, after
    `warmup` replays: the median over `reps` replays each between its own pair
    of events (one stack's latency), and the mean over `reps` replays back to
    back (its rate when the host keeps the queue full)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fn_list:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fn_list:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) * 1000.0 for e0, e1 in evs)
    # the same replays back to back with no events between them
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return ts[len(ts) // 2], a.elapsed_time(b) * 1000.0 / reps


def stack_measurements():
    """The small stacks (single fp32 layer of the 28x28 digit classifier,
    keyword-spotting int8 DS-CNN, visual-wake-words bf16 MobileNet) and the
    640x640 stack with and without its mosaic: microseconds per stack as the
    median of 200 graph replays after 20 warm-ups, and per layer. Their ideal
    work is far below a microsecond, so launch latency bounds them and a
    roofline fraction says nothing about them."""
    import torch

    from convolution_conv2d_nhwc_amd.data import workload
    from convolution_conv2d_nhwc_amd.stack import Stack

    out = {}
    for name in ("mnist_f32", "kws_int8", "vww_bf16", "yolo640_bf16"):
        wl = workload(name)
        st = Stack(wl, fuse=True)
        seq = st.launches()
        st.step()
        torch.cuda.synchronize()
        med, thr = graph_median_us(seq)
        durs, _ = per_launch_us(seq)
        names = (["mosaic_pack"] if st.canvas is not None else []) + [
            "+".join(wl.layers[i].name for i in n) for n in st.nodes()]
        kern = ([st.mosaic_kernel()] if st.canvas is not None else []) + [st.node_kernel(n) for n in st.nodes()]
        row = {"us_per_stack_median": round(med, 2), "us_per_stack_back_to_back": round(thr, 2),
               "replays": 200, "warmup": 20, "nodes": len(seq),
               "gflop": round(wl.flops() / 1e9, 5),
               "layers": [{"name": n, "kernel": k, "us": round(u, 2)} for n, k, u in zip(names, kern, durs)],
               "roofline": "not meaningful: launch-latency bound" if name != "yolo640_bf16" else "see the main line"}
        if st.canvas is not None:
            med1, thr1 = graph_median_us(seq[1:])
            row["us_per_stack_median_without_mosaic"] = round(med1, 2)
            row["us_per_stack_back_to_back_without_mosaic"] = round(thr1, 2)
        out[name] = row
        st.close()
        del st
        torch.cuda.empty_cache()
    return out


def measured_peaks():
    """What this GPU measurably sustains, beside the spec peaks: the library's
    matrix-core probe (bf16 and int8, back-to-back independent MFMAs on every
    SIMD) and its read+write stream over 1 GiB. Best of 5 timed launches after
    2 warm-ups each."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib

    def best_us(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0
            best = us if best is None else min(best, us)
        return best

    out = {}
    buf = torch.empty(4 * _lib.PROBE_MFMA_WORKGROUPS, dtype=torch.float32, device="cuda")
    for dt, unit in (("bf16", "TFLOP/s"), ("i8", "TOPS")):
        ops = _lib.probe_mfma(dt, 4000, buf)
        us = best_us(lambda dt=dt: _lib.probe_mfma(dt, 4000, buf))
        out["mfma_" + dt] = {"value": round(ops / (us * 1e-6) / 1e12, 1), "unit": unit,
                             "spec": PEAK[dt], "what": "conv_probe_mfma, %d workgroups x 4 waves" %
                             _lib.PROBE_MFMA_WORKGROUPS}
    n = 2 ** 30 // 16
    src = torch.ones(n * 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    moved = _lib.probe_copy(src, dst)
    us = best_us(lambda: _lib.probe_copy(src, dst))
    out["copy"] = {"value": round(moved / (us * 1e-6) / 1e9, 1), "unit": "GB/s", "spec": HBM_GBS,
                   "what": "conv_probe_copy over 1 GiB, read + write"}
    del src, dst
    torch.cuda.empty_cache()
    return out


def secondary_measurements(peaks, stacks=True):
    """Per-layer rates of the depthwise probe (against the HBM peak) and of the
    N=16 YOLO sweep (against the MFMA peak), outside the step's timed region.
    Inputs are seeded device tensors of each layer's shape and value law;
    every launch reads a different buffer set, with the sets together larger
    than 768 MB, so repeated launches cannot be served from the 256 MB
    Infinity Cache."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib
    from convolution_conv2d_nhwc_amd.data import workload

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)

    def draw(layer, shape, what):
        if layer.dtype == "i8":
            if what == "b":
                return torch.randint(-16129, 16130, shape, generator=gen, device="cuda", dtype=torch.int32)
            return torch.randint(-127, 128, shape, generator=gen, device="cuda", dtype=torch.int8)
        if what == "b":
            return (torch.rand(shape, generator=gen, device="cuda") * 0.2 - 0.1).float()
        fan_in = (layer.cin // layer.groups) * layer.kh * layer.kw
        sd = 0.5 if what == "x" else (2.0 / fan_in) ** 0.5
        return (torch.randn(shape, generator=gen, device="cuda") * sd).to(torch.bfloat16)

    out = {}
    # (label, workload, weight format): the bf16 sweep once more with its
    # weights in bfp8 blocks (16 values per shared exponent)
    for label, name, wfmt in (("dw_probe_bf16", "dw_probe_bf16", "plain"), ("dw_probe_int8", "dw_probe_int8", "plain"),
                              ("yolo_sweep_bf16", "yolo_sweep_bf16", "plain"),
                              ("yolo_sweep_int8", "yolo_sweep_int8", "plain"),
                              ("yolo_sweep_bf16_bfp8w", "yolo_sweep_bf16", "bfp8")):
        progress(label)
        rows = []
        tot_flop = tot_us = 0.0
        for layer in workload(name).layers:
            conv = _lib.Conv2d.from_layer(layer, w_format=wfmt)
            w = draw(layer, (layer.cout, layer.kh, layer.kw, layer.cin // layer.groups), "w")
            wbytes_plain = w.numel() * w.element_size()
            if wfmt == "bfp8":
                w = _lib.pack_bfp8(w)
            b = draw(layer, (layer.cout,), "b")
            if layer.dtype == "i8":
                s_ = torch.rand(layer.cout, generator=gen, device="cuda") * 0.009 + 0.001
                b = _lib.pack_bias_scale(b, s_)
            xy_bytes = layer.bytes() - wbytes_plain + w.numel() * w.element_size()
            nsets = max(2, min(32, -(-768 * 2 ** 20 // xy_bytes)))
            xs = [draw(layer, (layer.n, layer.h, layer.w, layer.cin), "x") for _ in range(nsets)]
            ys = [conv.empty_output() for _ in range(nsets)]
            for i in range(nsets):
                conv.run(xs[i], w, b, ys[i])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(nsets):
                    conv.run(xs[i], w, b, ys[i])
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / (reps * nsets)
            fl, by = layer.flops(), xy_bytes
            peak = PEAK[layer.dtype]
            t_roof = max(fl / (peak * 1e12), by / (HBM_GBS * 1e9))
            rows.append({"layer": layer.name, "kernel": conv.describe().split("kernel=")[-1], "us": round(us, 2),
                         "tflops": round(fl / (us * 1e-6) / 1e12, 2), "gbs": round(by / (us * 1e-6) / 1e9, 1),
                         "bound": "mfma" if fl / (peak * 1e12) >= by / (HBM_GBS * 1e9) else "hbm",
                         "roof_frac": round(t_roof / (us * 1e-6), 4),
                         "frac_mfma_peak": round(fl / (us * 1e-6) / 1e12 / peak, 4),
                         "frac_hbm_peak": round(by / (us * 1e-6) / 1e9 / HBM_GBS, 4),
                         "frac_measured_mfma": round(fl / (us * 1e-6) / 1e12 / peaks["mfma_" + layer.dtype]["value"],
                                                     4),
                         "dtype": layer.dtype, "buffer_sets": nsets})
            if layer.depthwise:
                # the same bytes moved by the library's read+write stream, same
                # buffer rotation and back-to-back launches: what a pure copy of
                # this size reaches on this GPU (launch gaps and ramp included)
                half = (xy_bytes // 2) // 16 * 16
                cs = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
                cd = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
                cus = _time_graph([lambda i=i: _lib.probe_copy(cs[i], cd[i]) for i in range(nsets)])
                rows[-1]["copy_same_bytes_us"] = round(cus, 2)
                rows[-1]["frac_copy_same_bytes"] = round(cus / us, 4)
                del cs, cd
            tot_flop += fl
            tot_us += us
            del xs, ys, g
            torch.cuda.empty_cache()
        out[label] = {"layers": rows, "total_us": round(tot_us, 2),
                     "tflops": round(tot_flop / (tot_us * 1e-6) / 1e12, 2)}
    progress("spp, upsample+concat, residual")
    out["spp_bf16"] = spp_measurements(gen)
    out["upcat_bf16"] = upcat_measurements(gen)
    out["upcat_conv_bf16"] = upcat_conv_measurements(gen)
    out["residual_bf16"] = residual_measurements(gen)
    copy = peaks["copy"]["value"]
    for sec in out.values():
        for row in sec.get("layers", []) if isinstance(sec, dict) else []:
            if "gbs" in row:
                row["frac_measured_copy"] = round(row["gbs"] / copy, 4)
    if stacks:
        progress("small stacks")
        out["stacks"] = stack_measurements()
    out["measured_peaks"] = peaks
    return out


def residual_measurements(gen):
    """The residual-add epilogue on a CSPDarknet ResBlock tail of the 640-pixel
    network (3x3, 64 -> 64 channels, Mish, 320x320, N=1 and N=16): the same
    layer through conv_run and through conv_run_residual. Cold buffer sets;
    the residual adds one read of y's size."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib
    from convolution_conv2d_nhwc_amd.data import Layer

    rows = []
    for n in (1, 16):
        layer = Layer("resblock_3x3_64", n, 320, 320, 64, 64, 3, 3, 1, 1, 1, 1, 1, "bf16", "bf16", "mish", 320, 320)
        conv = _lib.Conv2d.from_layer(layer)
        w = (torch.randn((64, 3, 3, 64), generator=gen, device="cuda") * (2.0 / 576) ** 0.5).to(torch.bfloat16)
        b = (torch.rand(64, generator=gen, device="cuda") * 0.2 - 0.1).float()
        xy = layer.bytes()
        nsets = max(2, min(32, -(-768 * 2 ** 20 // (xy + 2 * n * 320 * 320 * 64))))
        xs = [(torch.randn((n, 320, 320, 64), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
              for _ in range(nsets)]
        rs = [(torch.randn((n, 320, 320, 64), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
              for _ in range(nsets)]
        ys = [conv.empty_output() for _ in range(nsets)]
        plain = _time_graph([lambda i=i: conv.run(xs[i], w, b, ys[i]) for i in range(nsets)])
        fused = _time_graph([lambda i=i: conv.run(xs[i], w, b, ys[i], residual=rs[i]) for i in range(nsets)])
        rows.append({"layer": "%dx320x320x64 3x3 -> 64, Mish" % n, "kernel": conv.describe().split("kernel=")[-1],
                     "us_plain": round(plain, 2), "us_residual": round(fused, 2),
                     "extra_mb": round(2 * n * 320 * 320 * 64 / 1e6, 2), "buffer_sets": nsets})
        del xs, rs, ys
        conv.close()
        torch.cuda.empty_cache()
    return {"layers": rows}


def _time_graph(fn_list):
    """Average microseconds per call of a list of launches captured once and
    replayed 10 times."""
    import torch

    for f in fn_list:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fn_list:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (reps * len(fn_list))


def upcat_measurements(gen):
    """Upsample x2 + concat at YOLOv4's two neck joins for a 640-pixel input
    (20x20x256 upsampled beside 40x40x256; 40x40x128 beside 80x80x128), N=1
    and N=16. Cold buffer sets; bytes = both sources read once + y written."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib

    rows = []
    for n, (hs, cs) in [(1, (20, 256)), (1, (40, 128)), (16, (20, 256)), (16, (40, 128))]:
        a_shape, b_shape = (n, hs, hs, cs), (n, 2 * hs, 2 * hs, cs)
        by = 2 * (n * hs * hs * cs + 2 * n * 4 * hs * hs * cs)
        nsets = max(2, min(64, -(-768 * 2 ** 20 // by)))
        srcs = [((torch.randn(a_shape, generator=gen, device="cuda")).to(torch.bfloat16),
                 (torch.randn(b_shape, generator=gen, device="cuda")).to(torch.bfloat16)) for _ in range(nsets)]
        ys = [torch.empty((n, 2 * hs, 2 * hs, 2 * cs), dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]
        us = _time_graph([lambda i=i: _lib.upsample_concat(srcs[i][0], 1, srcs[i][1], 0, ys[i]) for i in range(nsets)])
        rows.append({"shape": "%dx%dx%dx%d up + %dx%dx%dx%d" % (a_shape + b_shape), "kernel": "upcat_kernel",
                     "us": round(us, 2), "gbs": round(by / (us * 1e-6) / 1e9, 1), "bound": "hbm",
                     "frac_hbm_peak": round(by / (us * 1e-6) / 1e9 / HBM_GBS, 4), "buffer_sets": nsets})
        del srcs, ys
        torch.cuda.empty_cache()
    return {"layers": rows}


def upcat_conv_measurements(gen):
    """The neck joins of upcat_measurements followed by their 1x1 convolution
    (2c -> c channels, Mish): the two-step path (conv_upsample_concat, then
    conv_run) against conv_run_upcat, which reads both maps itself and never
    writes the joined map. Same plan, cold buffer sets; bytes_saved = the
    joined map's write and read."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib
    from convolution_conv2d_nhwc_amd.data import Layer

    rows = []
    for n, (hs, cs) in [(1, (20, 256)), (1, (40, 128)), (16, (20, 256)), (16, (40, 128))]:
        h = 2 * hs
        layer = Layer("join_1x1", n, h, h, 2 * cs, cs, 1, 1, 1, 1, 0, 0, 1, "bf16", "bf16", "mish", h, h)
        conv = _lib.Conv2d.from_layer(layer)
        w = (torch.randn((cs, 1, 1, 2 * cs), generator=gen, device="cuda") * (1.0 / cs) ** 0.5).to(torch.bfloat16)
        b = (torch.rand(cs, generator=gen, device="cuda") * 0.2 - 0.1).float()
        joined = 2 * n * h * h * 2 * cs
        by = 2 * (n * hs * hs * cs + n * h * h * cs) + w.numel() * 2 + 2 * n * h * h * cs
        nsets = max(2, min(64, -(-768 * 2 ** 20 // (by + joined))))
        srcs = [((torch.randn((n, hs, hs, cs), generator=gen, device="cuda")).to(torch.bfloat16),
                 (torch.randn((n, h, h, cs), generator=gen, device="cuda")).to(torch.bfloat16)) for _ in range(nsets)]
        xs = [torch.empty((n, h, h, 2 * cs), dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]
        ys = [conv.empty_output() for _ in range(nsets)]

        def two_step(i):
            _lib.upsample_concat(srcs[i][0], 1, srcs[i][1], 0, xs[i])
            conv.run(xs[i], w, b, ys[i])

        us2 = _time_graph([lambda i=i: two_step(i) for i in range(nsets)])
        usf = _time_graph([lambda i=i: _lib.run_upcat(conv, srcs[i][0], 1, srcs[i][1], 0, w, b, ys[i])
                           for i in range(nsets)])
        rows.append({"shape": "%dx%dx%dx%d up + %dx%dx%dx%d -> 1x1 %d" % (n, hs, hs, cs, n, h, h, cs, cs),
                     "plan": conv.describe().split(" kernel=")[0], "us_two_step": round(us2, 2),
                     "us_fused": round(usf, 2), "bytes_saved": joined, "buffer_sets": nsets,
                     "fused_gbs": round(by / (usf * 1e-6) / 1e9, 1)})
        conv.close()
        del srcs, xs, ys
        torch.cuda.empty_cache()
    return {"layers": rows}


def spp_measurements(gen):
    """The SPP max-pool block (5/9/13 windows + the map) on YOLOv4's SPP maps:
    10x10x512 (320-pixel input, the size of the pages' isolated benchmark),
    20x20x512 (640-pixel input) and the N=16 batch of the latter. Cold buffer
    sets as above; bytes = x read once + y (4x) written once."""
    import torch

    from convolution_conv2d_nhwc_amd import _lib

    rows = []
    for shape in ((1, 10, 10, 512), (1, 20, 20, 512), (16, 20, 20, 512)):
        xb = 2 * shape[0] * shape[1] * shape[2] * shape[3]
        nsets = max(2, min(64, -(-768 * 2 ** 20 // (5 * xb))))
        xs = [(torch.randn(shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16) for _ in range(nsets)]
        ys = [torch.empty(shape[:3] + (4 * shape[3],), dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]
        for i in range(nsets):
            _lib.spp_maxpool(xs[i], ys[i])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nsets):
                _lib.spp_maxpool(xs[i], ys[i])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / (reps * nsets)
        by = 5 * xb
        rows.append({"shape": "x".join(map(str, shape)), "kernel": "spp_kernel<1, %d>" % (2 if 4 * xb >= 8 << 20 else 0), "us": round(us, 2),
                     "gbs": round(by / (us * 1e-6) / 1e9, 1), "bound": "hbm",
                     "frac_hbm_peak": round(by / (us * 1e-6) / 1e9 / HBM_GBS, 4), "buffer_sets": nsets})
        del xs, ys, g
        torch.cuda.empty_cache()
    return {"layers": rows}


def progress(msg: str):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def _oracle_stack_seconds(wl, threads):
    """One pass of the oracle over the stack (mosaic + every layer, each
    output rounded to the layer's output type as the next layer reads it)."""
    import numpy as np
    import torch

    from convolution_conv2d_nhwc_amd.data import layer_params, network_input
    from oracle import oracle

    x0 = network_input(wl)
    ps = [layer_params(wl, i) for i in range(len(wl.layers))]
    t = time.perf_counter()
    if wl.mosaic is not None:
        bits = oracle.mosaic(x0.numpy(), out="bf16")
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    else:
        x = x0.float().numpy()
    for layer, p in zip(wl.layers, ps):
        r, _ = oracle.conv_float(x, p["w"].float().numpy(), p["b"].numpy(), (layer.sh, layer.sw),
                                 (layer.ph, layer.pw), layer.groups, layer.act, want_abs=False, threads=threads)
        x = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).float().numpy() if layer.out == "bf16" \
            else r.astype(np.float32)
    return time.perf_counter() - t


def cpu_baseline(wl):
    """The oracle, untuned, on the same stack, as a ladder: every host thread
    (median of 5 passes; the reported value) and one thread (median of 3
    passes, ~10 s each)."""
    from oracle import oracle

    threads = oracle.num_threads(0)
    all_t = sorted(_oracle_stack_seconds(wl, threads) for _ in range(5))[2]
    one_t = sorted(_oracle_stack_seconds(wl, 1) for _ in range(3))[1]
    gf = wl.flops() / 1e9
    return {"value": round(gf / all_t / 1e3, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "the whole %s stack (%.2f GFLOP): median of 5 passes on %d threads (%.3f s); "
                      "ladder also at 1 thread, median of 3" % (wl.name, gf, threads, all_t),
            "ms_per_step": round(all_t * 1e3, 1),
            "ladder": [{"threads": 1, "ms_per_step": round(one_t * 1e3, 1), "runs": 3,
                        "value": round(gf / one_t / 1e3, 6)},
                       {"threads": threads, "ms_per_step": round(all_t * 1e3, 1), "runs": 5,
                        "value": round(gf / all_t / 1e3, 6)}],
            "host_cpus": os.cpu_count(), "cpu": _cpu_name()}


def _cpu_name():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
