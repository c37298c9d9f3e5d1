"""Benchmark: quantized Winograd F(6,3) conv layer on one MI355X.

Workload: the ResNet-18-shaped 3x3 layer (N=32, Cin=Cout=64, 56x56, pad 1,
group 64, seeded exp(U(-1/2,1/2)) transform scales), synthetic seeded inputs.
A step is one whole forward (input transform + int8 Hadamard GEMMs + output
transform) with inputs and prepared weights resident in HBM; the weight
transform is done once before timing.

Prints one JSON line: direct-conv-equivalent int8 TOPS, the per-kernel
roofline of the dominant kernel (HIP events around each stage's kernel on the
stream it runs on), and the CPU oracle timed on the host for comparison.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_convolution_amd as q  # noqa: E402
from quantized_convolution_amd import workloads as WL  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POP/s)
KERNEL_SRC = os.path.join(ROOT, "quantized_convolution_amd", "csrc", "wq8_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# name of each stage's kernel in a rocprofv3 trace (template prefix)
KERNEL_NAMES = {"stage1": ("wq8::k_stage1<",), "stage2": ("wq8::k_stage2<",),
                "stage3": ("wq8::k_stage3<",),
                "stage23": ("wq8::k_fused23<", "wq8::k_fused23w<")}


def kernel_source_sha():
    """Hash of the kernel source's code: comments and whitespace are dropped,
    so only a change to the code itself marks recorded counters stale."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def recorded_traffic(layer, kernel):
    """HBM bytes per launch of `kernel` on `layer` from the committed counter
    summary, or None when there is none or the kernel source has changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    k = rec.get("layers", {}).get(layer, {}).get(kernel)
    return None if k is None else k["bytes_per_launch"]


# position of the integer-input-stage flag among k_stage1's template arguments
# <M, G, TPB, BMASK, VEC, XT, IQ, RH>
STAGE1_IQ_ARG = 6


def stage_of(kernel_name):
    """Stage key of a kernel in a rocprofv3 trace, or None. The stage-1
    kernel with the integer input stage (template argument IQ true) is
    "stage1_int"."""
    for stage, prefixes in KERNEL_NAMES.items():
        for prefix in prefixes:
            i = kernel_name.find(prefix)
            if i >= 0:
                if stage == "stage1":
                    args = kernel_name[i + len(prefix):].split(">")[0].split(",")
                    if len(args) > STAGE1_IQ_ARG and args[STAGE1_IQ_ARG].strip() == "true":
                        return "stage1_int"
                return stage
    return None


def _pmc_rows(d, counter):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV run."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_summary(layer, fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib):
    """Turn two counter passes over bench.py (FETCH_SIZE, WRITE_SIZE, KiB per
    dispatch) and the same two over the copy probe into bytes per launch of
    each stage kernel. The copy probe reads and writes copy_mib MiB per
    launch; the counters are scaled by known / counted on it."""
    known = copy_mib * 2 ** 20

    def copy_factor(d, counter):
        vals = [v for _, v in _pmc_rows(d, counter)]
        return known / (statistics.median(vals) * 1024.0)

    fr, wr = copy_factor(cfetch_dir, "FETCH_SIZE"), copy_factor(cwrite_dir, "WRITE_SIZE")
    out = {"kernel_source_sha": kernel_source_sha(), "copy_probe_mib": copy_mib,
           "fetch_factor": round(fr, 4), "write_factor": round(wr, 4), "layers": {layer: {}}}
    fetch, write = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")
    lines = ["| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (scaled) |",
             "|---|---|---|---|---|"]
    for stage in list(KERNEL_NAMES) + ["stage1_int"]:
        f = [v for k, v in fetch if stage_of(k) == stage]
        w = [v for k, v in write if stage_of(k) == stage]
        if not f or not w:
            continue
        fk, wk = statistics.median(f), statistics.median(w)
        b = int(round(fk * 1024 * fr + wk * 1024 * wr))
        out["layers"][layer][stage] = {"fetch_kib": fk, "write_kib": wk, "bytes_per_launch": b}
        lines.append(f"| {stage} | {len(f)} | {fk:.1f} | {wk:.1f} | {b} |")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(f"copy probe {copy_mib} MiB: fetch factor {fr:.4f}, write factor {wr:.4f}")
    print("\n".join(lines))


def copy_probe(mib, steps, dev):
    """A plain copy kernel of known size (read mib MiB, write mib MiB per
    launch) for calibrating the HBM byte counters."""
    n = mib * 2 ** 20 // 4
    src = torch.empty(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "launches": steps}), flush=True)


def stage_bytes(L, plan):
    """Algorithmic HBM bytes of each kernel per launch (each operand read or
    written once)."""
    n2, T, ng = plan.n ** 2, plan.T, plan.ng
    xb = L.N * L.Cin * L.H * L.W * 4
    yb = L.N * L.Cout * L.Ho * L.Wo * 4
    vq, sv = n2 * T * L.Cin, n2 * T * ng * 4
    uq, su = n2 * L.Cout * L.Cin, n2 * L.Cout * ng * 4
    mb = n2 * T * L.Cout * 4
    return {"stage1": xb + vq + sv, "stage2": vq + sv + uq + su + mb, "stage3": mb + yb,
            "stage23": vq + sv + uq + su + yb}


def time_events(fn, iters, stream):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def time_each(fn, iters, stream, before=None):
    """Per-call times (ms) from an event pair around each call; `before` runs
    between the calls, outside the timed pairs."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(L, d, min_seconds=10.0):
    """The plain CPU oracle (as it stands) on the host cores, over the full
    workload (fp32 quantized pipeline, weight transform excluded like on the
    GPU), repeated until about `min_seconds` of CPU work; then one run on a
    single thread, and the fp64 direct convolution (the accuracy reference,
    timed separately; it is not the competitor)."""
    import oracle
    from oracle import transforms as T

    Bt, Gm, At = T.transforms_f32(L.m, list(d["points"]), d["s_b"], d["s_g"])
    Uq, sU = oracle.weights(L.m, d["w"], L.G, Gm)

    def fwd():
        t0 = time.perf_counter()
        Vq, sV = oracle.stage1(L.m, d["x"], L.pad, L.G, Bt)
        M = oracle.stage2(Vq, sV, Uq, sU, L.G)
        oracle.stage3(L.m, M, L.N, L.H, L.W, L.pad, At)
        return time.perf_counter() - t0

    cores = oracle.num_threads()
    times = []
    t_end = time.perf_counter() + min_seconds
    while len(times) < 3 or time.perf_counter() < t_end:
        times.append(fwd())
        if len(times) >= 200:
            break
    t = statistics.median(times)
    oracle.set_num_threads(1)
    try:
        t1 = fwd()
    finally:
        oracle.set_num_threads(cores)
    t0 = time.perf_counter()
    oracle.direct_conv_f64(d["x"], d["w"], L.pad)
    td = time.perf_counter() - t0
    return {"value": round(L.direct_ops() / t / 1e12, 5), "unit": "TOPS",
            "cores": cores, "kind": "oracle",
            "sample": f"full workload (N={L.N}), forward only (fp32 quantized pipeline), median of "
                      f"{len(times)} runs, {t * 1e3:.1f} ms each",
            "value_1thread": round(L.direct_ops() / t1 / 1e12, 5),
            "direct_f64_ms": round(td * 1e3, 1)}


def accuracy(L, d, dev, images=4):
    """Output SQNR (dB) of the GPU forward against a float64 CPU convolution
    (torch), on the first `images` images, for the timed scales, standard
    scales (S = I) and equalising scales."""
    from quantized_convolution_amd import scales as S

    n = L.m + 2
    x = torch.from_numpy(d["x"][:images]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ref = torch.nn.functional.conv2d(torch.from_numpy(d["x"][:images]).double(),
                                     torch.from_numpy(d["w"]).double(), padding=L.pad)
    out = {}
    for iq in ("fp32", "int_tensor", "int_row"):
        row = {}
        for name, (b, g) in {"timed_scales": (d["s_b"], d["s_g"]), "standard_S_I": ([1.0] * n, [1.0] * n),
                             "equalizing": S.equalizing_scales(L.m, list(d["points"]))}.items():
            plan = q.Plan(L.m, images, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=b,
                          s_G=g, in_quant=iq)
            Uq, sU = q.wq8_weights_prepare(plan, w)
            y = q.wq8_conv_forward(plan, x, Uq, sU).double().cpu()
            row[name] = round(float(10 * torch.log10(torch.sum(ref ** 2) / torch.sum((y - ref) ** 2))), 2)
        out[iq + "_input"] = row
    return {"sqnr_db": out, "reference": "float64 direct convolution (torch, CPU)",
            "sample": f"images 0..{images - 1} of the timed workload",
            "input_stage": "fp32: fp32 input transform; int_tensor / int_row: B^T (one scale / one per "
                           "row) and input patches quantized, integer transform"}


def run_layer(L, algo, steps, warmup, dev):
    d = WL.make(L)
    plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"],
                  s_B=d["s_b"], s_G=d["s_g"], algo=algo)
    x = torch.from_numpy(d["x"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    Uq, sU = q.wq8_weights_prepare(plan, w)
    y = plan.empty_output(dev)
    ws = plan.empty_workspace(dev)
    stream = torch.cuda.current_stream()

    def step():
        q.wq8_conv_forward(plan, x, Uq, sU, y=y, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-step distribution, caches warm, and cold: a 512 MiB fill before each
    # step evicts the 256 MB Infinity Cache (and the L2s)
    hot = time_each(step, min(steps, 100), stream)
    flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    cold = time_each(step, 20, stream, before=lambda: flush.fill_(1.0))
    del flush

    # per-kernel durations: each stage entry point launches exactly the kernel
    # the forward launches, with the same grid, on the same stream
    n2 = plan.n ** 2
    Vq = torch.empty((n2, plan.T, L.Cin), dtype=torch.int8, device=dev)
    sV = torch.empty((n2, plan.T, plan.ng), dtype=torch.float32, device=dev)
    iters = max(20, steps // 2)
    k_ms = {"stage1": time_events(lambda: q.wq8_stage1(plan, x, Vq, sV), iters, stream)}
    if plan.fused:
        k_ms["stage23"] = time_events(lambda: q.wq8_stage23(plan, Vq, sV, Uq, sU, y), iters, stream)
    else:
        M = torch.empty((n2, plan.T, L.Cout), dtype=torch.float32, device=dev)
        k_ms["stage2"] = time_events(lambda: q.wq8_stage2(plan, Vq, sV, Uq, sU, M), iters, stream)
        k_ms["stage3"] = time_events(lambda: q.wq8_stage3(plan, M, y), iters, stream)
    nbytes = stage_bytes(L, plan)
    hop = 2 * n2 * plan.T * L.Cin * L.Cout
    stages = {}
    for k, v in k_ms.items():
        gbs = nbytes[k] / (v * 1e-3) / 1e9
        stages[k] = {"us": round(v * 1e3, 2), "GB_s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if k in ("stage2", "stage23"):
            stages[k]["int8_TOPS"] = round(hop / (v * 1e-3) / 1e12, 2)
            stages[k]["mfma_frac"] = round(hop / (v * 1e-3) / 1e12 / INT8_PEAK_TOPS, 5)
    # the literal input stage (quantized B^T and input patch, integer
    # transform): its stage-1 kernel and whole forward on the same workload
    lit = {}
    for iq in ("int_tensor", "int_row"):
        pl = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                    s_G=d["s_g"], algo=algo, in_quant=iq)
        s1 = time_events(lambda: q.wq8_stage1(pl, x, Vq, sV), iters, stream)
        fw = time_events(lambda: q.wq8_conv_forward(pl, x, Uq, sU, y=y, workspace=ws), iters, stream)
        lit[iq] = {"stage1_us": round(s1 * 1e3, 2),
                   "stage1_hbm_frac": round(nbytes["stage1"] / (s1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "forward_us": round(fw * 1e3, 2),
                   "TOPS": round(L.direct_ops() / (fw * 1e-3) / 1e12, 2)}
    # the non-Winograd baseline on the same layer: group-wise W8A8 direct conv
    Wq, sW = q.wq8_direct_weights_prepare(plan, w)
    dws = torch.empty(plan.direct_workspace_bytes, dtype=torch.uint8, device=dev)
    for _ in range(3):
        q.wq8_direct_forward(plan, x, Wq, sW, y=y, workspace=dws)
    d_ms = time_events(lambda: q.wq8_direct_forward(plan, x, Wq, sW, y=y, workspace=dws), iters, stream)
    Xq, sX = q.wq8_direct_quantize_x(plan, x)
    dq_ms = time_events(lambda: q.wq8_direct_quantize_x(plan, x, Xq, sX), iters, stream)
    dc_ms = time_events(lambda: q.wq8_direct_conv(plan, Xq, sX, Wq, sW, y=y), iters, stream)
    direct = {"us": round(d_ms * 1e3, 2), "quantize_x_us": round(dq_ms * 1e3, 2),
              "conv_us": round(dc_ms * 1e3, 2), "TOPS": round(L.direct_ops() / (d_ms * 1e-3) / 1e12, 2),
              "winograd_speedup": round(d_ms / ms, 3)}
    del dws, Xq, sX

    dom = max(k_ms, key=k_ms.get)
    achieved = nbytes[dom] / (k_ms[dom] * 1e-3) / 1e9
    return dict(plan=plan, d=d, ms=ms, wall=wall, stages=stages, dom=dom, achieved=achieved,
                nbytes=nbytes, tops=L.direct_ops() / (ms * 1e-3) / 1e12, direct=direct, literal=lit,
                hot=(statistics.median(hot), min(hot)), cold=(statistics.median(cold), min(cold)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layer", default=WL.BENCH_LAYER, choices=sorted(WL.LAYERS))
    ap.add_argument("--algo", default="auto", choices=["auto", "staged", "fused"])
    ap.add_argument("--sweep", action="store_true",
                    help="one line per layer and schedule (for tuning; no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a copy kernel of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="rocprofv3 --pmc output dirs (bench FETCH_SIZE, bench WRITE_SIZE, copy "
                         "probe FETCH_SIZE, copy probe WRITE_SIZE): write profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.layer, *args.traffic_summary, args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is not "
              "sharded across GPUs in this build", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps, dev)
        return

    if args.sweep:
        for name, L in WL.LAYERS.items():
            for algo in ("staged", "fused"):
                r = run_layer(L, algo, args.steps, args.warmup, dev)
                print(json.dumps({"layer": name, "algo": algo, "us": round(r["ms"] * 1e3, 2),
                                  "TOPS": round(r["tops"], 2), "stages": r["stages"],
                                  "direct_w8a8": r["direct"], "literal_input_stage": r["literal"]}),
                      flush=True)
        return

    L = WL.LAYERS[args.layer]
    r = run_layer(L, args.algo, args.steps, args.warmup, dev)
    plan, dom = r["plan"], r["dom"]
    out = {
        "metric": "direct-conv-equiv int8 TOPS per layer, F(6,3); % MFMA int8 peak + HBM GB/s",
        "value": round(r["tops"], 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": L.name, "m": L.m, "N": L.N, "Cin": L.Cin, "Cout": L.Cout,
                   "H": L.H, "W": L.W, "pad": L.pad, "group": L.G, "scales": L.scales,
                   "x_dtype": "f32", "tiles": plan.T,
                   "schedule": "fused" if plan.fused else "staged"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(r["achieved"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(L.name, dom),
                     "bytes_per_launch": r["nbytes"][dom]},
        "stages": r["stages"],
        "baseline_direct_w8a8": r["direct"],
        "literal_input_stage": r["literal"],
        "accuracy": accuracy(L, r["d"], dev),
        "per_step_ms": {"median": round(r["hot"][0], 5), "min": round(r["hot"][1], 5),
                        "cold_median": round(r["cold"][0], 5), "cold_min": round(r["cold"][1], 5),
                        "cold_TOPS": round(L.direct_ops() / (r["cold"][0] * 1e-3) / 1e12, 3)},
        "wall_s": round(r["wall"], 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, r["d"])
        out["cpu_baseline"]["gpu_speedup_vs_oracle"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
