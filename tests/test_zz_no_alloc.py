"""wq8_conv_forward_noalloc (the forward on the library's built-in workspace)
against wq8_conv_forward (caller's workspace): the same kernels on the same
inputs, so the outputs must agree bit for bit. Two calls in a row, the second
on a smaller layer, so the second reuses the array the first left behind; a
plan whose workspace exceeds the array is refused before any launch."""
import numpy as np
import pytest
import torch

import quantized_convolution_amd as q
from quantized_convolution_amd import binding as B
from quantized_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    return torch.device("cuda:0")


def _run(L, dev, algo):
    d = WL.make(L)
    plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], algo=algo)
    x = torch.from_numpy(d["x"]).to(dev)
    Uq, sU = q.wq8_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    want = q.wq8_conv_forward(plan, x, Uq, sU)
    got = torch.full_like(want, float("nan"))
    B.wq8_conv_forward_noalloc(plan, x, Uq, sU, got)
    torch.cuda.synchronize()
    return plan, got, want


@pytest.mark.parametrize("first,second", [
    # the largest workspace the array holds (staged ResNet-18 layer, 66.4 MB),
    # then a small fused layer
    (("c2_f6_n32_c64_56x56_g64", "staged"), ("c3c_f6_n32_c512_7x7_g64", "auto")),
    # the deep staged layer, then a small ragged one with groups of 16
    (("c5_f6_n8_c1280_16x16_g32", "auto"), ("c1_f4_n1_c16_16x16_g16", "auto")),
])
def test_noalloc_matches_forward(dev, first, second):
    (n1, a1), (n2, a2) = first, second
    print(f"\n[case] noalloc {n1} ({a1}) then {n2} ({a2})", flush=True)
    p1, g1, w1 = _run(WL.LAYERS[n1], dev, a1)
    assert p1.workspace_bytes <= B.NOALLOC_MAX_WORKSPACE
    assert torch.equal(g1.view(torch.int32), w1.view(torch.int32)), f"{n1}: outputs differ"
    p2, g2, w2 = _run(WL.LAYERS[n2], dev, a2)
    assert p2.workspace_bytes < p1.workspace_bytes
    assert torch.equal(g2.view(torch.int32), w2.view(torch.int32)), f"{n2}: outputs differ"


def test_noalloc_refuses_oversized_plan(dev):
    # N = 64 of the ResNet-18 layer, staged: 132.7 MB of workspace
    plan = q.Plan(6, 64, 64, 64, 56, 56, 1, 64, algo="staged")
    assert plan.workspace_bytes > B.NOALLOC_MAX_WORKSPACE
    x = torch.zeros(plan.x_shape, device=dev)
    Uq, sU = plan.empty_weights(dev)
    y = torch.full(plan.y_shape, 7.0, device=dev)
    with pytest.raises(q.Wq8Error) as e:
        B.wq8_conv_forward_noalloc(plan, x, Uq, sU, y)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "nothing may be launched"
