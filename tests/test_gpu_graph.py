"""The forward captured in a HIP graph (how the benchmark times it) gives the
eager forward's output bit for bit on every replay, with eager work and
synchronisations between the replays. The library records only kernel
launches (no memset or copy nodes)."""
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


@pytest.mark.parametrize("name,algo", [
    ("c2_f6_n32_c64_56x56_g64", "auto"),          # fused schedule
    ("c5_f6_n8_c1280_16x16_g32", "auto"),         # staged schedule
    ("c4_f4_n2_c320_64x64_g64_pert", "fused"),
])
def test_graph_replays_match_eager(dev, name, algo):
    L = WL.LAYERS[name]
    print(f"\n[case] graph {name} ({algo})", flush=True)
    d = WL.make(L)
    plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], algo=algo)
    x = torch.from_numpy(d["x"]).to(dev)
    Uq, sU = q.wq8_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    ws = plan.empty_workspace(dev)
    want = q.wq8_conv_forward(plan, x, Uq, sU, workspace=ws).clone()
    y = plan.empty_output(dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.wq8_conv_forward(plan, x, Uq, sU, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.wq8_conv_forward(plan, x, Uq, sU, y=y, workspace=ws)
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0x5A)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), f"replay {rep} differs"
    # the no-allocation entry point is capturable the same way
    if plan.workspace_bytes > q.binding.NOALLOC_MAX_WORKSPACE:
        return
    q.binding.wq8_conv_forward_noalloc(plan, x, Uq, sU, y)  # per-device lookup outside the graph
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        q.binding.wq8_conv_forward_noalloc(plan, x, Uq, sU, y)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), f"no-alloc replay {rep} differs"
