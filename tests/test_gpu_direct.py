"""GPU parity of the group-wise W8A8 direct convolution (the non-Winograd
baseline) against the CPU oracle, through the C ABI.

Bar: activation and weight codes and scales bit-exact; outputs bit-exact as
well (both sides evaluate the same fp32 fma chain, in the same order, on the
same codes; no rounding decision follows). Cases span the group sizes,
padding 0..2, pixel blocks that split a wide row or span several narrow rows
and images, with a ragged tail, channel counts that are not multiples of 64, bf16 in and out, and the
full ResNet-18 layer.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_convolution_amd as q
from quantized_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    return torch.device("cuda:0")


def plan_for(L, xdt=torch.float32, ydt=None):
    return q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, x_dtype=xdt, y_dtype=ydt)


CASES = [
    WL.small(WL.LAYERS["c2_f6_n32_c64_56x56_g64"], N=2, H=9, W=70, Cin=64, Cout=72),
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], N=1, H=7, W=5, Cin=32, Cout=5),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], N=1, H=6, W=13, Cin=96, Cout=20).replace(pad=0, name="g32pad0"),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g128"], N=1, H=5, W=6, Cin=256, Cout=9).replace(pad=2, name="g128pad2"),
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], N=1, H=4, W=3, Cin=256, Cout=3).replace(G=256, name="g256"),
    WL.small(WL.LAYERS["c4_f4_n2_c320_64x64_g64_pert"], N=1, H=3, W=130, Cin=192, Cout=65),
    # rows narrower than a 64-pixel block: blocks span rows and images, ragged pixel tail
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g32"], N=3, H=5, W=7, Cin=96, Cout=40),
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], N=2, H=16, W=16, Cin=256, Cout=70),
    # either side of the switch between the two block forms (rows of 32 and 33 pixels)
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], N=2, H=5, W=32, Cin=64, Cout=36),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], N=2, H=5, W=33, Cin=64, Cout=36),
]


@pytest.mark.parametrize("L", CASES, ids=[L.name for L in CASES])
def test_direct_matches_oracle(dev, L):
    print(f"\n[case] direct W8A8 {L.name} N={L.N} C={L.Cin}->{L.Cout} {L.H}x{L.W} pad={L.pad} G={L.G}",
          flush=True)
    d = WL.make(L)
    ref = oracle.direct_w8a8(d["x"], d["w"], L.pad, L.G, keep=True)
    plan = plan_for(L)
    Wq, sW = q.wq8_direct_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    x = torch.from_numpy(d["x"]).to(dev)
    Xq, sX = q.wq8_direct_quantize_x(plan, x)
    y = q.wq8_direct_forward(plan, x, Wq, sW)
    y2 = q.wq8_direct_conv(plan, Xq, sX, Wq, sW)
    torch.cuda.synchronize()
    assert np.array_equal(Wq.cpu().numpy(), ref["wq"]) and np.array_equal(sW.cpu().numpy(), ref["sw"])
    assert np.array_equal(Xq.cpu().numpy(), ref["xq"]) and np.array_equal(sX.cpu().numpy(), ref["sx"])
    assert np.array_equal(y.cpu().numpy(), ref["y"])
    assert np.array_equal(y2.cpu().numpy(), ref["y"])


def test_direct_full_resnet_layer(dev):
    """The full ResNet-18 layer (N=32, 64 -> 64, 56x56, G=64) in the launch
    configuration bench.py times."""
    L = WL.LAYERS["c2_f6_n32_c64_56x56_g64"]
    print(f"\n[case] direct W8A8 full {L.name}", flush=True)
    d = WL.make(L)
    ref = oracle.direct_w8a8(d["x"], d["w"], L.pad, L.G)
    plan = plan_for(L)
    Wq, sW = q.wq8_direct_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    y = q.wq8_direct_forward(plan, torch.from_numpy(d["x"]).to(dev), Wq, sW)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), ref)


# W = 11: blocks of consecutive pixels across rows; W = 40: row blocks
@pytest.mark.parametrize("W", [11, 40])
@pytest.mark.parametrize("xdt,ydt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16)])
def test_direct_bf16(dev, xdt, ydt, W):
    L = WL.small(WL.LAYERS["c2_f6_n32_c64_56x56_g64"], N=1, H=8, W=W, Cin=64, Cout=24)
    print(f"\n[case] direct W8A8 bf16 {xdt} -> {ydt} W={W}", flush=True)
    d = WL.make(L)
    xt = torch.from_numpy(d["x"]).to(xdt)
    x_ref = d["x"] if xdt == torch.float32 else oracle.bf16_bits_to_f32(
        xt.view(torch.int16).numpy().view(np.uint16))
    ref = oracle.direct_w8a8(x_ref, d["w"], L.pad, L.G)
    plan = plan_for(L, xdt, ydt)
    Wq, sW = q.wq8_direct_weights_prepare(plan, torch.from_numpy(d["w"]).to(dev))
    y = q.wq8_direct_forward(plan, xt.to(dev), Wq, sW)
    torch.cuda.synchronize()
    bits = y.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, oracle.f32_to_bf16_bits(ref))


def test_direct_rejects_small_workspace(dev):
    L = WL.small(WL.LAYERS["c2_f6_n32_c64_56x56_g64"], N=1, H=8, W=8, Cin=64, Cout=8)
    plan = plan_for(L)
    x = torch.zeros((L.N, L.Cin, L.H, L.W), device=dev)
    Wq, sW = q.wq8_direct_weights_prepare(plan, torch.zeros((L.Cout, L.Cin, 3, 3), device=dev))
    ws = torch.empty(plan.direct_workspace_bytes - 256, dtype=torch.uint8, device=dev)
    y = plan.empty_output(dev)
    # the binding refuses before calling the library ...
    with pytest.raises(ValueError, match="workspace"):
        q.wq8_direct_forward(plan, x, Wq, sW, y=y, workspace=ws)
    # ... and so does the library itself, called directly through the C ABI
    import ctypes as C
    from quantized_convolution_amd import binding as B
    st = B.load().wq8_direct_forward(plan.handle, C.c_void_p(x.data_ptr()), C.c_void_p(Wq.data_ptr()),
                                     C.c_void_p(sW.data_ptr()), C.c_void_p(y.data_ptr()),
                                     C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel()),
                                     C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -4
