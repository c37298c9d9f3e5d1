"""A plan is immutable and may be used from several host threads on
different streams at once, each call with its own workspace: forwards
launched concurrently from two threads on two streams give the outputs of the
same forwards run one after the other, bit for bit, for one shared plan and
for two plans of different schedules."""
import threading

import pytest
import torch

import quantized_convolution_amd as q
from quantized_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    return torch.device("cuda:0")


def _setup(L, algo, dev, seed):
    d = WL.make(L)
    plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], algo=algo)
    Uq, sU = q.wq8_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn(plan.x_shape, generator=g).to(dev) for _ in range(3)]
    return plan, Uq, sU, xs


def _run_threads(jobs, dev):
    """jobs: list of (plan, Uq, sU, xs); each runs its forwards on its own
    stream from its own host thread; returns the outputs per job."""
    outs = [None] * len(jobs)
    errors = []
    start = threading.Barrier(len(jobs))

    def work(k, plan, Uq, sU, xs):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream()
            ws = plan.empty_workspace(dev)
            ys = [plan.empty_output(dev) for _ in xs]
            torch.cuda.synchronize()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(5):  # repeated so that the streams overlap in time
                    for x, y in zip(xs, ys):
                        q.wq8_conv_forward(plan, x, Uq, sU, y=y, workspace=ws)
            s.synchronize()
            outs[k] = [y.cpu() for y in ys]
        except Exception as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=work, args=(k, *job)) for k, job in enumerate(jobs)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    return outs


@pytest.mark.parametrize("pair", ["one plan", "two plans"])
def test_concurrent_streams_match_serial(dev, pair):
    La = WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g32"], N=2, H=16, W=16, Cin=256, Cout=64)
    Lb = WL.small(WL.LAYERS["c2_f6_n32_c64_56x56_g64"], N=2, H=30, W=26, Cin=64, Cout=40)
    print(f"\n[case] concurrent streams, {pair}", flush=True)
    a = _setup(La, "staged", dev, 1)
    if pair == "one plan":
        b = (a[0], a[1], a[2], [x.flip(0).contiguous() for x in a[3]])
    else:
        b = _setup(Lb, "fused", dev, 2)
    serial = []
    for plan, Uq, sU, xs in (a, b):
        ws = plan.empty_workspace(dev)
        serial.append([q.wq8_conv_forward(plan, x, Uq, sU, workspace=ws).cpu() for x in xs])
    torch.cuda.synchronize()
    conc = _run_threads([a, b], dev)
    for k in range(2):
        for i, (want, got) in enumerate(zip(serial[k], conc[k])):
            assert torch.equal(want.view(torch.int32), got.view(torch.int32)), f"job {k}, input {i}"
