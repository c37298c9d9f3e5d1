"""GPU parity of the literal input stage (B^T and the input patch quantized,
integer transform; the review page's "sqB sqB sqx" factor of Eqs. 14-16)
against the CPU oracle, through the C ABI.

Bars: Vq and sV bit-exact (the transform is exact integer arithmetic and the
scale products are the same fp32 operations in the same order on both sides,
so no rounding decision can differ); forward outputs within the pipeline's
output tolerance (1e-3 of the oracle output's RMS) on both schedules.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import transforms as TR
import quantized_convolution_amd as q
from quantized_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    return torch.device("cuda:0")


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def plan_for(L, d, iq, algo="auto", xdt=torch.float32):
    return q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], algo=algo, in_quant=iq, x_dtype=xdt)


CASES = [WL.small(L) for L in WL.LAYERS.values()] + [
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=3, W=70, Cin=64, Cout=13),           # wide, W % 4 != 0
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=12, W=12).replace(pad=0, name="pad0"),
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=5, W=9).replace(pad=2, name="pad2"),
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], H=1, W=1),                   # 1x1 image
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], Cin=256, Cout=40).replace(G=256, name="g256"),
]
IQ = ["int_tensor", "int_row"]


@pytest.mark.parametrize("iq", IQ)
@pytest.mark.parametrize("L", CASES, ids=[L.name for L in CASES])
def test_literal_stage1_and_forward(dev, L, iq):
    print(f"\n[case] literal {iq} {L.name} F({L.m},3) N={L.N} C={L.Cin}->{L.Cout} {L.H}x{L.W} "
          f"pad={L.pad} G={L.G}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True, in_quant=iq)
    plan = plan_for(L, d, iq)
    Bq, sq = q.wq8_plan_bt_codes(plan)
    oBq, osq = oracle.quant_bt(ref["Bt"], iq == "int_row")
    assert np.array_equal(Bq, oBq) and np.array_equal(sq, osq)
    x = to_dev(d["x"], dev)
    Vq, sV = q.wq8_stage1(plan, x)
    torch.cuda.synchronize()
    assert np.array_equal(Vq.cpu().numpy(), ref["Vq"])
    assert np.array_equal(sV.cpu().numpy(), ref["sV"])
    for algo in ("staged", "fused"):
        p2 = plan_for(L, d, iq, algo=algo)
        Uq, sU = q.wq8_weights_prepare(p2, to_dev(d["w"], dev))
        y = q.wq8_conv_forward(p2, x, Uq, sU)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(y.cpu().numpy().astype(np.float64) - ref["y"])))
        assert err <= OUT_TOL * rms(ref["y"]) or err == 0.0, f"{algo}: {err:.3e}"


@pytest.mark.parametrize("iq", IQ)
def test_literal_bf16_input(dev, iq):
    L = WL.small(WL.LAYERS[WL.BENCH_LAYER], N=2, H=9, W=13, Cin=64, Cout=16)
    print(f"\n[case] literal {iq} bf16 input {L.name}", flush=True)
    d = WL.make(L)
    xb = torch.from_numpy(d["x"]).to(torch.bfloat16)
    x_ref = oracle.bf16_bits_to_f32(xb.view(torch.int16).numpy().view(np.uint16))
    Bt = TR.transforms_f32(L.m, list(d["points"]), d["s_b"], d["s_g"])[0]
    oBq, osq = oracle.quant_bt(Bt, iq == "int_row")
    oVq, osV = oracle.stage1_int(L.m, x_ref, L.pad, L.G, oBq, osq)
    plan = plan_for(L, d, iq, xdt=torch.bfloat16)
    Vq, sV = q.wq8_stage1(plan, xb.to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(Vq.cpu().numpy(), oVq) and np.array_equal(sV.cpu().numpy(), osV)


@pytest.mark.parametrize("iq", IQ)
def test_literal_full_bench_layer(dev, iq):
    """The full ResNet-18 layer (N=32, 64 -> 64, 56x56, G=64, F(6,3)) in the
    launch configuration of the forward: every V code and scale."""
    L = WL.LAYERS[WL.BENCH_LAYER]
    print(f"\n[case] literal {iq} full {L.name}", flush=True)
    d = WL.make(L)
    plan = plan_for(L, d, iq)
    Bt = TR.transforms_f32(L.m, list(d["points"]), d["s_b"], d["s_g"])[0]
    oBq, osq = oracle.quant_bt(Bt, iq == "int_row")
    oVq, osV = oracle.stage1_int(L.m, d["x"], L.pad, L.G, oBq, osq)
    Vq, sV = q.wq8_stage1(plan, to_dev(d["x"], dev))
    torch.cuda.synchronize()
    assert np.array_equal(Vq.cpu().numpy(), oVq) and np.array_equal(sV.cpu().numpy(), osV)
