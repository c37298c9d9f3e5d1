"""Benchmark: quantized Winograd F(m,3) conv layers on one MI355X.

Workload (the headline): the largest configuration, a deep UNet-shaped 3x3
layer, F(6,3), N=8, Cin=Cout=1280, 16x16, pad 1, group 32, Student-t(3)
activations with 1 % of the channels x20, N(0, 0.02^2) weights, seeded
exp(U(-1/2,1/2)) transform scales; synthetic seeded inputs. A step is one
whole forward (input transform + int8 Hadamard GEMMs + output transform) with
inputs and prepared weights resident in HBM; the weight transform is done
once before timing. K steps are captured in one HIP graph and replayed
between two HIP events on the launch stream.

Prints one JSON line: direct-conv-equivalent int8 TOPS, the roofline of the
dominant kernel (each kernel's own launches, captured and replayed the same
way), per-layer records for every configuration, SQNR per scale set, and the
CPU oracle timed on the host for comparison.
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

HEADLINE = "c5_f6_n8_c1280_16x16_g32"  # the largest configuration (bytes moved per layer)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POP/s)
KERNEL_SRCS = [os.path.join(ROOT, "quantized_convolution_amd", "csrc", f)
               for f in ("wq8_kernels.hip", "wq8_hgemm.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# name of each stage's kernel in a rocprofv3 trace (template prefix)
KERNEL_NAMES = {"stage1": ("wq8::k_stage1<",), "stage2": ("wq8::k_stage2<", "wq8::k_hgemm<"),
                "stage3": ("wq8::k_stage3<",),
                "stage23": ("wq8::k_fused23<", "wq8::k_fused23w<")}


def kernel_source_sha():
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so only a change to the code itself marks recorded counters stale."""
    src = ""
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            src += f.read() + "\n"
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
           "fetch_factor": round(fr, 4), "write_factor": round(wr, 4), "layers": {}}
    try:
        with open(TRAFFIC_FILE) as f:
            old = json.load(f)
        if old.get("kernel_source_sha") == out["kernel_source_sha"]:
            out["layers"] = old.get("layers", {})  # other layers taken on the same code
    except (OSError, ValueError):
        pass
    out["layers"][layer] = {}
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
    """Average ms per call of `iters` eagerly launched calls (each call goes
    through the Python binding, so short kernels measure the host instead)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def capture(fn, reps):
    """A HIP graph of `reps` calls of fn (every kernel the calls launch, in
    order, on the capture stream; nothing else is recorded)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first call outside the graph: per-device lookups happen here
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def warm_graph(g, min_seconds=0.025):
    """Untimed replays of g until it has kept the GPU busy for at least
    `min_seconds` of wall time: a short warm-up after the idle capture would
    leave the timed replay to start below steady clocks (a timed graph of 20
    forwards of the 1280-channel layer measured 10 % slower after a single
    warm replay)."""
    t_end = time.perf_counter() + min_seconds
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


def time_graph(g, reps, stream, replays=1):
    """ms per call: `replays` replays of a graph of `reps` calls between two
    events on `stream`; the kernels run back to back with no host launch in
    between."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / (reps * replays)


def time_cold(g, n, stream, flush):
    """ms of each of n replays of a one-call graph, each after a read pass
    over a 512 MiB buffer (written once beforehand): the read evicts the 256
    MB Infinity Cache and the L2s and leaves only clean lines, so the replay
    finds its operands in HBM and no other data waiting to be written back
    (the read also keeps the GPU busy while the replay is enqueued)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    sink = torch.empty((), dtype=torch.float32, device=flush.device)
    for a, b in evs:
        torch.sum(flush, dim=0, out=sink)
        a.record(stream)
        g.replay()
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


def scale_sets(L, d):
    """Transform scales the accuracy report covers: the timed workload's
    (seeded exp(U(-1/2, 1/2)) or identity), standard (S = I), the data-free
    equalizing set, and the learned set for this m when one is recorded."""
    from quantized_convolution_amd import scales as S

    n = L.m + 2
    sets = {"timed_scales": (d["s_b"], d["s_g"]), "standard_S_I": ([1.0] * n, [1.0] * n),
            "equalizing": S.equalizing_scales(L.m, list(d["points"]))}
    learned = S.recorded_learned_scales(L.m)
    if learned is not None:
        sets["learned"] = learned
    return sets


def accuracy(L, d, dev, images):
    """Output SQNR (dB) of the GPU forward against a float64 CPU convolution
    (torch), on the first `images` images, for each scale set; the literal
    input-stage readings for the timed and equalizing scales."""
    x = torch.from_numpy(d["x"][:images]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ref = torch.nn.functional.conv2d(torch.from_numpy(d["x"][:images]).double(),
                                     torch.from_numpy(d["w"]).double(), padding=L.pad)
    out = {}
    for iq in ("fp32", "int_tensor", "int_row"):
        row = {}
        for name, (b, g) in scale_sets(L, d).items():
            if iq != "fp32" and name not in ("timed_scales", "equalizing"):
                continue
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


def mfma_report(L, plan, us, bytes_):
    """int8 Hadamard work of a stage-2 (or fused) launch against the MFMA
    peak, and the ceiling its arithmetic intensity allows from HBM:
    min(1, AI * BW / peak)."""
    hop = 2 * plan.n ** 2 * plan.T * L.Cin * L.Cout
    tops = hop / (us * 1e-6) / 1e12
    ceiling = min(1.0, hop / bytes_ * HBM_PEAK_GBS * 1e9 / (INT8_PEAK_TOPS * 1e12))
    frac = tops / INT8_PEAK_TOPS
    return {"int8_TOPS": round(tops, 2), "mfma_frac": round(frac, 5),
            "mfma_ceiling": round(ceiling, 5), "of_ceiling": round(frac / ceiling, 4)}


def make_plan(L, d, algo="auto", **kw):
    return q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"],
                  s_B=d["s_b"], s_G=d["s_g"], algo=algo, **kw)


def run_layer(L, algo, steps, warmup, dev, d=None, cold_reps=20, extras=False, direct=False):
    """One layer: the forward (K steps captured in one HIP graph and
    replayed between two events; the same K steps eagerly launched for
    comparison), each kernel on its own (its stage entry point captured
    `iters` times), warm and after a cache flush. extras: the literal input
    stage and the W8A8 direct baseline on the same workload; direct: the
    W8A8 direct baseline only."""
    d = WL.make(L) if d is None else d
    plan = make_plan(L, d, algo)
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
    g = capture(step, steps)
    warm_graph(g)
    t0 = time.perf_counter()
    ms = time_graph(g, steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager = time_events(step, steps, stream)
    del g
    flush = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g1 = capture(step, 1)
    cold = time_cold(g1, cold_reps, stream, flush)
    del g1

    # per-kernel durations: each stage entry point launches exactly the kernel
    # the forward launches, with the same grid
    calls = stage_calls(plan, x, Uq, sU, y, dev)
    iters = max(20, steps // 2)
    k_ms, k_cold = {}, {}
    for k, fn in calls.items():
        gk = capture(fn, iters)
        gk.replay()
        k_ms[k] = time_graph(gk, iters, stream)
        del gk
        gk = capture(fn, 1)
        k_cold[k] = statistics.median(time_cold(gk, cold_reps, stream, flush))
        del gk
    del flush
    nbytes = stage_bytes(L, plan)
    stages = {}
    for k, v in k_ms.items():
        gbs = nbytes[k] / (v * 1e-3) / 1e9
        cgbs = nbytes[k] / (k_cold[k] * 1e-3) / 1e9
        stages[k] = {"us": round(v * 1e3, 2), "cold_us": round(k_cold[k] * 1e3, 2),
                     "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "cold_hbm_frac": round(cgbs / HBM_PEAK_GBS, 4), "bytes": nbytes[k]}
        if k in ("stage2", "stage23"):
            stages[k]["mfma"] = mfma_report(L, plan, v * 1e3, nbytes[k])
            stages[k]["mfma_cold"] = mfma_report(L, plan, k_cold[k] * 1e3, nbytes[k])
    out = dict(plan=plan, d=d, ms=ms, eager_ms=eager, wall=wall, stages=stages, k_ms=k_ms,
               nbytes=nbytes, tops=L.direct_ops() / (ms * 1e-3) / 1e12,
               cold=(statistics.median(cold), min(cold)))
    if not extras:
        if direct:
            out["direct"] = time_direct(L, plan, x, w, y, ms, max(5, iters // 4), dev)
        return out
    # the literal input stage (quantized B^T and input patch, integer
    # transform): its stage-1 kernel and whole forward on the same workload
    lit = {}
    Vq = torch.empty(plan.vq_shape, dtype=torch.int8, device=dev)
    sV = torch.empty(plan.sv_shape, dtype=torch.float32, device=dev)
    for iq in ("int_tensor", "int_row"):
        pl = make_plan(L, d, algo, in_quant=iq)
        gs = capture(lambda: q.wq8_stage1(pl, x, Vq, sV), iters)
        s1 = time_graph(gs, iters, stream)
        del gs
        gf = capture(lambda: q.wq8_conv_forward(pl, x, Uq, sU, y=y, workspace=ws), iters)
        fw = time_graph(gf, iters, stream)
        del gf
        lit[iq] = {"stage1_us": round(s1 * 1e3, 2),
                   "stage1_hbm_frac": round(nbytes["stage1"] / (s1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "forward_us": round(fw * 1e3, 2),
                   "TOPS": round(L.direct_ops() / (fw * 1e-3) / 1e12, 2)}
    out["literal"] = lit
    out["direct"] = time_direct(L, plan, x, w, y, ms, max(5, iters // 4), dev)
    return out


def time_direct(L, plan, x, w, y, wino_ms, reps, dev):
    """The non-Winograd baseline on the same layer and inputs: the group-wise
    W8A8 direct convolution (activation quantization + convolution), each
    part and the whole forward captured `reps` times in a HIP graph."""
    stream = torch.cuda.current_stream()
    Wq, sW = q.wq8_direct_weights_prepare(plan, w)
    dws = torch.empty(plan.direct_workspace_bytes, dtype=torch.uint8, device=dev)
    Xq, sX = q.wq8_direct_quantize_x(plan, x)
    res = {}
    for key, fn in (("forward", lambda: q.wq8_direct_forward(plan, x, Wq, sW, y=y, workspace=dws)),
                    ("quantize_x", lambda: q.wq8_direct_quantize_x(plan, x, Xq, sX)),
                    ("conv", lambda: q.wq8_direct_conv(plan, Xq, sX, Wq, sW, y=y))):
        gd = capture(fn, reps)
        res[key] = time_graph(gd, reps, stream)
        del gd
    return {"us": round(res["forward"] * 1e3, 2), "quantize_x_us": round(res["quantize_x"] * 1e3, 2),
            "conv_us": round(res["conv"] * 1e3, 2),
            "TOPS": round(L.direct_ops() / (res["forward"] * 1e-3) / 1e12, 2),
            "winograd_speedup": round(res["forward"] / wino_ms, 3)}


def layer_entry(L, r):
    """Per-layer record: forward time and throughput, each kernel warm and
    cold against HBM, the Hadamard stage against int8 MFMA, and (when timed)
    the W8A8 direct baseline with the Winograd speedup over it."""
    e = {"schedule": "fused" if r["plan"].fused else "staged", "tiles": r["plan"].T,
         "forward_us": round(r["ms"] * 1e3, 2), "TOPS": round(r["tops"], 2),
         "cold_forward_us": round(r["cold"][0] * 1e3, 2),
         "cold_TOPS": round(L.direct_ops() / (r["cold"][0] * 1e-3) / 1e12, 2),
         "eager_forward_us": round(r["eager_ms"] * 1e3, 2), "stages": r["stages"]}
    if "direct" in r:
        e["direct_w8a8_us"] = r["direct"]["us"]
        e["winograd_speedup"] = r["direct"]["winograd_speedup"]
    return e


def stage_calls(plan, x, Uq, sU, y, dev):
    """Each kernel of the forward through its stage entry point (the same
    kernel and grid), on buffers of its own: the calls whose durations the
    per-stage records and the roofline report."""
    Vq = torch.empty(plan.vq_shape, dtype=torch.int8, device=dev)
    sV = torch.empty(plan.sv_shape, dtype=torch.float32, device=dev)
    q.wq8_stage1(plan, x, Vq, sV)
    calls = {"stage1": lambda: q.wq8_stage1(plan, x, Vq, sV)}
    if plan.fused:
        calls["stage23"] = lambda: q.wq8_stage23(plan, Vq, sV, Uq, sU, y)
    else:
        M = torch.empty(plan.m_shape, dtype=torch.float32, device=dev)
        calls["stage2"] = lambda: q.wq8_stage2(plan, Vq, sV, Uq, sU, M)
        calls["stage3"] = lambda: q.wq8_stage3(plan, M, y)
    return calls


def profile_run(L, algo, steps, dev, stages=False):
    """The command rocprofv3 traces or counts for the summaries under
    profiles/ (one process): only the forward of one layer, `steps` times
    (eager launches); or, with `stages`, each kernel as the per-stage timing
    runs it (a HIP graph of `steps` back-to-back calls of its stage entry
    point, replayed once, after one call outside the graph)."""
    d = WL.make(L)
    plan = make_plan(L, d, algo)
    x = torch.from_numpy(d["x"]).to(dev)
    Uq, sU = q.wq8_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    y = plan.empty_output(dev)
    ws = plan.empty_workspace(dev)
    torch.cuda.synchronize()
    if stages:
        for fn in stage_calls(plan, x, Uq, sU, y, dev).values():
            g = capture(fn, steps)
            g.replay()
            torch.cuda.synchronize()
            del g
    else:
        for _ in range(steps):
            q.wq8_conv_forward(plan, x, Uq, sU, y=y, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": L.name, "schedule": "fused" if plan.fused else "staged",
                      "what": "stage graphs" if stages else "forwards", "calls": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layer", default=HEADLINE, choices=sorted(WL.LAYERS))
    ap.add_argument("--algo", default="auto", choices=["auto", "staged", "fused"])
    ap.add_argument("--sweep", action="store_true",
                    help="one line per layer and schedule (for tuning; no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layers", action="store_true", help="skip the per-layer records")
    ap.add_argument("--profile-run", action="store_true",
                    help="only run --steps forwards of --layer (for rocprofv3)")
    ap.add_argument("--profile-stages", action="store_true",
                    help="with --profile-run: each kernel as the per-stage timing runs it (a graph of "
                         "--steps calls of its stage entry point)")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a copy kernel of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="rocprofv3 --pmc output dirs (FETCH_SIZE and WRITE_SIZE over --profile-run "
                         "of --layer, then over the copy probe): record the layer in "
                         "profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.layer, *args.traffic_summary, args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library does "
              "not shard a layer across GPUs", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps, dev)
        return
    if args.profile_run:
        profile_run(WL.LAYERS[args.layer], args.algo, args.steps, dev, stages=args.profile_stages)
        return

    if args.sweep:
        for name, L in WL.LAYERS.items():
            for algo in ("staged", "fused"):
                r = run_layer(L, algo, args.steps, args.warmup, dev)
                print(json.dumps({"layer": name, "algo": algo, **layer_entry(L, r)}), flush=True)
        return

    L = WL.LAYERS[args.layer]
    r = run_layer(L, args.algo, args.steps, args.warmup, dev, extras=True)
    plan = r["plan"]
    dom = max(r["k_ms"], key=r["k_ms"].get)
    st = r["stages"][dom]
    out = {
        "metric": "direct-conv-equiv int8 TOPS per layer, F(6,3); % MFMA int8 peak + HBM GB/s",
        "value": round(r["tops"], 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": L.name, "m": L.m, "N": L.N, "Cin": L.Cin, "Cout": L.Cout,
                   "H": L.H, "W": L.W, "pad": L.pad, "group": L.G, "scales": L.scales,
                   "x_dtype": "f32", "tiles": plan.T,
                   "schedule": "fused" if plan.fused else "staged",
                   "timing": "K forwards captured in one HIP graph, replayed between two HIP events"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": st["GB_s"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": st["hbm_frac"],
                     "cold_frac": st["cold_hbm_frac"],
                     "traffic": recorded_traffic(L.name, dom),
                     "bytes_per_launch": r["nbytes"][dom], "avg_launch_us": st["us"]},
        "stages": r["stages"],
        "per_step_ms": {"graph": round(r["ms"], 5), "eager": round(r["eager_ms"], 5),
                        "cold_median": round(r["cold"][0], 5), "cold_min": round(r["cold"][1], 5),
                        "cold_TOPS": round(L.direct_ops() / (r["cold"][0] * 1e-3) / 1e12, 3)},
        "baseline_direct_w8a8": r["direct"],
        "literal_input_stage": r["literal"],
        "wall_s": round(r["wall"], 4),
    }
    if "mfma" in st:
        out["roofline"]["mfma"] = st["mfma"]
    if not args.no_layers:
        layers = {}
        for name, Lx in WL.LAYERS.items():
            if name == L.name:
                layers[name] = layer_entry(L, r)
                continue
            layers[name] = layer_entry(Lx, run_layer(Lx, "auto", min(args.steps, 100),
                                                     min(args.warmup, 10), dev, direct=True))
        out["layers"] = layers
    out["accuracy"] = accuracy(L, r["d"], dev, images=min(L.N, 4 if L.N >= 32 else 2))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, r["d"])
        out["cpu_baseline"]["gpu_speedup_vs_oracle"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
