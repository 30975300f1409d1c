"""Benchmark: conv2d forward / backward-data / backward-filter on one MI355X.

One step = one pass of the whole hot path over one batch of the workload:
forward, backward-data and backward-filter (for the deconvolution workload:
its forward, backward-data and backward-weights passes, which run the
backward-data, forward and backward-filter kernels).  value = 3 * 2*N*K*P*Q*C*R*S / step time, in TFLOP/s.
The passes run in order on one stream.  With --streams 2 the two backward
passes, which depend only on the step's inputs, run concurrently on two
streams after the forward, each with its own workspace, and value is that
schedule's step rate.  Otherwise each buffer set's in-order step is recorded
once into a HIP graph (the library only launches kernels on the caller's
stream) and value is the rate of replaying those graphs (--no-graph: of the
launches from Python).  The in-order run launched from Python ("serial") is
always timed too, and the per-pass times and the roofline entry come from its
events.

The headline workload (default: deep3x3 in bf16, N=256 C=K=512 14x14 3x3, the largest
configuration) gives value; every other configuration (the tiny, resnet3x3, 1x1 projection,
7x7 stem and deconvolution workloads, in each dtype they are defined for) is then measured the
same way, with fewer steps, and reported under "configs" with its own per-pass times and
roofline entry (--no-extra skips them).

Inputs are synthetic (seeded, the workload's value distributions) and resident
in HBM before timing starts.  Buffer sets are rotated so that the per-step
footprint cycles through more than 1 GB and the 256 MB Infinity Cache cannot
hold the working set ("cold" timing).  Each pass is bracketed by HIP events on
the stream the library launches on; the dominant pass's kernel time gives the
roofline entry.  The CPU baseline is the fp64 oracle (test infrastructure,
never tuned) timed on the host on one step of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype bf16|f32]
                       [--streams 1|2] [--epilogue [--bf16-out]] [--no-extra] [--no-cpu-baseline]
Prints one JSON line on stdout.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
METRIC = "conv2d fwd/bwd-data/bwd-filter TFLOP/s (2NKPQCRS) and % of MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before each timed phase: the pass times settle over a few dozen steps
    # (deep3x3 bf16 on one box: 950 TFLOP/s after 5 warm-up steps, 974 after 60)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="deep3x3")
    ap.add_argument("--dtype", default="bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the headline workload (not the other configurations)")
    ap.add_argument("--hot", action="store_true", help="reuse one buffer set (cache-resident)")
    ap.add_argument("--passes", default=None, help="comma list, default: the workload's passes")
    ap.add_argument("--epilogue", action="store_true",
                    help="run the forward pass as conv2d_fwd_ex with a per-channel bias and ReLU")
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2),
                    help="1: every pass in order on one stream; 2: after the forward, backward-data and "
                         "backward-filter run concurrently on two streams (separate workspaces)")
    ap.add_argument("--no-graph", action="store_true",
                    help="value from the in-order run launched from Python instead of from replays of each "
                         "buffer set's step recorded into a HIP graph")
    ap.add_argument("--bf16-out", action="store_true",
                    help="with --epilogue: the forward writes y in bf16 (fp32 accumulation)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def source_hash():
    """Hash of the HIP sources; stored traffic counts are valid only for these kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_implicit_gemm_nchw_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, dtype, pass_id):
    """HBM bytes per launch of the pass's main kernel from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (profiles/traffic.json), or None if absent or taken on other kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get("entries", {}).get(f"{workload}/{dtype}/{pass_id}")
    if not e or e.get("source_hash") != source_hash():
        return None
    return e["bytes_per_launch"]


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))


def alg_bytes(s, pass_id, es):
    """Algorithmic HBM bytes: every touched input element read once, the filter once,
    every output element written once (fp32)."""
    nchw = s.N * s.C * s.H * s.W
    nkpq = s.N * s.K * s.P * s.Q
    kcrs = s.K * s.C * s.R * s.S
    # x elements a forward window touches (a 1x1 stride-2 filter reads 1/4 of x)
    rows = len({p * s.stride[0] - s.pad[0] + r for p in range(s.P) for r in range(s.R)
                if 0 <= p * s.stride[0] - s.pad[0] + r < s.H})
    cols = len({q * s.stride[1] - s.pad[1] + c for q in range(s.Q) for c in range(s.S)
                if 0 <= q * s.stride[1] - s.pad[1] + c < s.W})
    x_touched = s.N * s.C * rows * cols
    if pass_id == "fwd":
        return x_touched * es + kcrs * es + nkpq * 4
    if pass_id in ("bwd_data", "deconv_fwd"):
        return nkpq * es + kcrs * es + nchw * 4
    if pass_id == "deconv_bwd_data":   # convolution forward over the whole deconvolution output
        return nchw * es + kcrs * es + nkpq * 4
    if pass_id == "deconv_bwd_filter":
        return nchw * es + nkpq * es + kcrs * 4
    return x_touched * es + nkpq * es + kcrs * 4


# Every other configuration, measured in the same run after the headline one and reported
# under "configs": the five workloads of the target list (the tiny one is launch-bound), plus
# the 1x1 projection in bf16, where the HBM roofline binds.
EXTRA_CONFIGS = [("tiny", "f32"), ("resnet3x3", "bf16"), ("resnet3x3", "f32"), ("proj1x1", "f32"),
                 ("proj1x1", "bf16"), ("stem7x7", "f32"), ("deconv4x4", "f32"), ("deconv4x4", "bf16")]


def measure(args, name, dt, steps, warmup, graph_on=True):
    """Times `steps` steps of every pass of one workload on cuda:0 (after `warmup` steps) and
    returns the step rate, per-pass times and the roofline entry of the slowest pass."""
    import numpy as np
    import torch

    import convolution_implicit_gemm_nchw_amd as mc
    from workloads import WORKLOADS, inputs

    wl = WORKLOADS[name]
    s = wl.shape
    passes = args.passes.split(",") if args.passes and name == args.workload else list(wl.passes)
    es = 2 if dt == "bf16" else 4
    dev = torch.device("cuda:0")
    code = mc.BF16 if dt == "bf16" else mc.F32
    bf16_out = args.bf16_out and name == args.workload
    epilogue = args.epilogue and name == args.workload

    host = inputs(wl, dt)
    a13 = s.args13()

    def pass_bytes(p):
        """Algorithmic bytes of a pass (a bf16 y writes 2 bytes per output)."""
        return alg_bytes(s, p, es) - (s.N * s.K * s.P * s.Q * 2 if p == "fwd" and bf16_out else 0)

    pid = {"fwd": mc.FWD, "bwd_data": mc.BWD_DATA, "bwd_filter": mc.BWD_FILTER, "deconv_fwd": mc.DECONV_FWD,
           "deconv_bwd_data": mc.DECONV_BWD_DATA, "deconv_bwd_filter": mc.DECONV_BWD_FILTER}
    deconv13 = (s.N, s.K, s.P, s.Q, s.C, s.R, s.S, s.pad[0], s.pad[1], s.stride[0], s.stride[1], s.H, s.W)

    def sizes(p):
        return deconv13 if p.startswith("deconv") else a13

    ws_need = 0
    for p in passes:
        ws_need = max(ws_need, mc.workspace_size(pid[p], code, sizes(p)))

    # with two streams the two backward passes overlap; each has its own workspace
    bwd_pair = [p for p in passes[1:] if p.endswith("bwd_data")], [p for p in passes[1:] if p.endswith("bwd_filter")]
    concurrent = (args.streams == 2 and name == args.workload and len(passes) == 3 and len(bwd_pair[0]) == 1
                  and len(bwd_pair[1]) == 1)

    # one buffer set = inputs + outputs of every pass + workspace(s)
    def make_set():
        d = {k: v.to(dev) for k, v in host.items()}
        if wl.deconv:
            d["out"] = torch.empty(s.x_shape, dtype=torch.float32, device=dev)
            d["din"] = torch.empty(s.y_shape, dtype=torch.float32, device=dev)
            d["dwd"] = torch.empty(s.w_shape, dtype=torch.float32, device=dev)
        else:
            d["y"] = torch.empty(s.y_shape, dtype=torch.bfloat16 if bf16_out else torch.float32, device=dev)
            d["dx"] = torch.empty(s.x_shape, dtype=torch.float32, device=dev)
            d["dw"] = torch.empty(s.w_shape, dtype=torch.float32, device=dev)
        d["ws"] = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
        if concurrent:
            d["ws2"] = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
        if epilogue:
            d["bias"] = torch.linspace(-0.5, 0.5, s.K, dtype=torch.float32, device=dev)
        return d

    first = make_set()
    footprint = sum(t.numel() * t.element_size() for t in first.values())
    # cold: rotate sets through > 1 GB (the tiny workload is launch-bound and cache-resident anyway)
    hot = args.hot or footprint < (1 << 20)
    n_sets = 1 if hot else min(64, max(1, math.ceil(1.0e9 / footprint)))
    sets = [first] + [make_set() for _ in range(n_sets - 1)]
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev) if concurrent else None   # default priority

    def run_pass(p, d, stream=stream, ws="ws"):
        if p == "fwd" and epilogue:
            mc.conv2d_fwd_ex(d["x"], d["w"], s.pad, s.stride, bias=d["bias"], relu=True, y=d["y"],
                             workspace=d[ws], stream=stream)
        elif p == "fwd":
            mc.conv2d_fwd(d["x"], d["w"], s.pad, s.stride, y=d["y"], workspace=d[ws], stream=stream)
        elif p == "bwd_data":
            mc.conv2d_bwd_data(d["dy"], d["w"], (s.H, s.W), s.pad, s.stride, dx=d["dx"],
                               workspace=d[ws], stream=stream)
        elif p == "bwd_filter":
            mc.conv2d_bwd_filter(d["x"], d["dy"], (s.R, s.S), s.pad, s.stride, dw=d["dw"],
                                 workspace=d[ws], stream=stream)
        elif p == "deconv_fwd":
            mc.deconv2d_fwd(d["x_in"], d["w"], (s.H, s.W), s.pad, s.stride, y=d["out"],
                            workspace=d[ws], stream=stream)
        elif p == "deconv_bwd_data":
            mc.deconv2d_bwd_data(d["dout"], d["w"], (s.P, s.Q), s.pad, s.stride, dx=d["din"],
                                 workspace=d[ws], stream=stream)
        else:
            mc.deconv2d_bwd_filter(d["x_in"], d["dout"], (s.R, s.S), s.pad, s.stride, dw=d["dwd"],
                                   workspace=d[ws], stream=stream)

    for i in range(warmup):
        for p in passes:
            run_pass(p, sets[i % n_sets])
    torch.cuda.synchronize()

    # in-order run launched from Python; HIP events on the library's stream bracket each pass
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(passes) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        d = sets[i % n_sets]
        ev[i][0].record(stream)
        for j, p in enumerate(passes):
            run_pass(p, d)
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_serial = elapsed * 1e3 / steps
    flops_pass = s.flops()
    total_flops = flops_pass * len(passes)
    value_serial = total_flops / (ms_serial * 1e-3) / 1e12

    ms_step, value = ms_serial, value_serial
    if concurrent:
        fwd_done = torch.cuda.Event()
        side_done = torch.cuda.Event()

        def step2(d):
            run_pass(passes[0], d)
            fwd_done.record(stream)
            side.wait_event(fwd_done)
            run_pass(bwd_pair[1][0], d, stream=side, ws="ws2")
            run_pass(bwd_pair[0][0], d)
            side_done.record(side)
            stream.wait_event(side_done)

        for i in range(warmup):
            step2(sets[i % n_sets])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step2(sets[i % n_sets])
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        value = total_flops / (ms_step * 1e-3) / 1e12
    graph = None
    if graph_on and not concurrent:
        cap = torch.cuda.Stream(device=dev)   # default priority
        graphs = []
        for d in sets:
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):   # one eager step on the capture stream first
                for p in passes:
                    run_pass(p, d, stream=cap)
            stream.wait_stream(cap)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for p in passes:
                    run_pass(p, d, stream=cap)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        ms_graph = (time.perf_counter() - t0) * 1e3 / steps
        graph = {"value": round(total_flops / (ms_graph * 1e-3) / 1e12, 3), "ms_per_step": round(ms_graph, 5),
                 "note": "one HIP graph per buffer set holding the step's library calls, replayed in turn"}
        ms_step, value = ms_graph, total_flops / (ms_graph * 1e-3) / 1e12
        del graphs
    pass_ms = {p: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
               for j, p in enumerate(passes)}
    per_pass = {}
    for p, ms in pass_ms.items():
        b = pass_bytes(p)
        per_pass[p] = {"ms": round(ms, 5), "tflops": round(flops_pass / (ms * 1e-3) / 1e12, 2),
                       "mfma_frac": round(flops_pass / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[dt], 4),
                       "alg_bytes": b, "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "plan": mc.plan_describe(pid[p], code, sizes(p), ws_need)}
    dom = max(pass_ms, key=pass_ms.get)
    dm = pass_ms[dom]
    t_flop = flops_pass / (PEAK_TFLOPS[dt] * 1e12)
    t_hbm = pass_bytes(dom) / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_flop:
        achieved = pass_bytes(dom) / (dm * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = flops_pass / (dm * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = stored_traffic(wl.name, dt, dom)
    plan = dict(kv.split("=", 1) for kv in per_pass[dom]["plan"].split() if "=" in kv)
    tinyc = "few-channel MFMA kernel" if plan.get("form") == "mfma" else "few-channel vector kernel"
    parts = [{"patch": "LDS-patch kernel", "tinyc": tinyc,
              "pointwise": "pointwise kernel"}.get(plan.get("algo"), "implicit-GEMM kernel")]
    if int(plan.get("splits", "1")) > 1:
        parts.append("split-K reduce")
    roof["kernel"] = f"{dom} pass: " + " + ".join(parts) + " (time between the pass's events)"
    roof["ms_per_launch"] = round(dm, 5)
    res = {"workload": f"{wl.name}: N={s.N} C={s.C} H={s.H} W={s.W} K={s.K} R={s.R} S={s.S} "
                       f"pad={s.pad[0]} stride={s.stride[0]} P={s.P} Q={s.Q}",
           "passes": passes, "value": value, "ms_per_step": ms_step, "value_serial": value_serial,
           "ms_serial": ms_serial, "graph": graph, "concurrent": concurrent, "per_pass": per_pass,
           "roofline": roof, "n_sets": n_sets, "hot": hot, "total_flops": total_flops}
    del sets, first
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, dt, passes):
    """The oracle (fp64 direct loops, never tuned) on one full step of the workload."""
    import oracle
    from workloads import WORKLOADS, inputs
    wl = WORKLOADS[name]
    s = wl.shape
    host = inputs(wl, dt)
    f = {k: v.float().numpy() for k, v in host.items()}
    t1 = time.perf_counter()
    for p in passes:
        if p == "fwd":
            oracle.conv2d_fwd(f["x"], f["w"], s.pad, s.stride)
        elif p == "bwd_data":
            oracle.conv2d_bwd_data(f["dy"], f["w"], (s.H, s.W), s.pad, s.stride)
        elif p == "bwd_filter":
            oracle.conv2d_bwd_filter(f["x"], f["dy"], (s.R, s.S), s.pad, s.stride)
        elif p == "deconv_fwd":
            oracle.deconv2d_fwd(f["x_in"], f["w"], (s.H, s.W), s.pad, s.stride)
        elif p == "deconv_bwd_data":
            oracle.deconv2d_bwd_data(f["dout"], f["w"], (s.P, s.Q), s.pad, s.stride)
        else:
            oracle.deconv2d_bwd_filter(f["x_in"], f["dout"], (s.R, s.S), s.pad, s.stride)
    tc = time.perf_counter() - t1
    total = s.flops() * len(passes)
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(total / tc / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": model,
            "sample": f"one full step ({'+'.join(passes)}) of {wl.name}, fp64 direct loops",
            "seconds": round(tc, 3)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.bf16_out and not args.epilogue:
        sys.exit("--bf16-out needs --epilogue")
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only: the path shards over images (N) with one "
                                   "all-reduce of dW per step, which is not built", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    torch.cuda.set_device(torch.device("cuda:0"))

    head = measure(args, args.workload, args.dtype, args.steps, args.warmup, graph_on=not args.no_graph)
    dt = args.dtype
    extra = {}
    if not args.no_extra:
        for name, edt in EXTRA_CONFIGS:
            if (name, edt) == (args.workload, dt):
                continue
            r = measure(args, name, edt, min(args.steps, 20), min(args.warmup, 20), graph_on=not args.no_graph)
            extra[f"{name}/{edt}"] = {
                "workload": r["workload"], "dtype": edt, "passes": r["passes"], "value": round(r["value"], 3),
                "unit": "TFLOP/s", "ms_per_step": round(r["ms_per_step"], 5),
                "mfma_frac_of_step": round(r["value"] / PEAK_TFLOPS[edt], 4), "cold": not r["hot"],
                "per_pass": {p: {k: v for k, v in pp.items() if k != "plan"} for p, pp in r["per_pass"].items()},
                "roofline": r["roofline"]}
            print(f"[bench] {name}/{edt}: {r['value']:.1f} TFLOP/s, slowest pass "
                  f"{r['roofline']['kernel'].split(':')[0]} {r['roofline']['frac']:.3f} of {r['roofline']['bound']}",
                  file=sys.stderr, flush=True)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, dt, head["passes"])
    from workloads import WORKLOADS
    wl = WORKLOADS[args.workload]
    out = {
        "metric": METRIC, "value": round(head["value"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded; the workload's value distributions)",
        "config": {"workload": head["workload"],
                   "passes": head["passes"], "input_dtype": dt, "accum_out": "f32",
                   "forward_epilogue": ("bias+relu (fused)" if args.epilogue else "none") +
                                       (", bf16 y" if args.bf16_out else ""),
                   "cold": not head["hot"], "buffer_sets": head["n_sets"],
                   "schedule": ("forward, then backward-data and backward-filter concurrently on two streams "
                                "(separate workspaces)") if head["concurrent"] else (
                       "every pass in order on one stream, replayed from a HIP graph" if head["graph"]
                       else "every pass in order on one stream"),
                   "mfma_frac_of_step": round(head["value"] / PEAK_TFLOPS[dt], 4)},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "per_pass": head["per_pass"],
        **({"graph": head["graph"]} if head["graph"] else {}),
        "serial": {"value": round(head["value_serial"], 3), "ms_per_step": round(head["ms_serial"], 5),
                   "note": "the same passes in order on one stream; per-pass times and the roofline come "
                           "from this run"},
        "configs": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
