"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (floating point decides the int8 codes, so both sides take those
decisions in fp32 with the same operation order):
  * int8 codes (Uq, Vq, Yq): mismatches in at most 1e-4 of the values, each at
    most one step (a rounding tie); in practice they are identical;
  * int32 Hadamard partials given identical codes: bit-exact;
  * group and tile scales: identical wherever the codes agree;
  * outputs: max |gpu - oracle| <= 1e-3 * RMS(oracle output).
Inputs come from quantized_convolution_amd.workloads (seeded) and the oracle
only ever sees those inputs, never a GPU result.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_convolution_amd as q
from quantized_convolution_amd import workloads as WL

pytestmark = pytest.mark.gpu

CODE_MISMATCH_MAX = 1e-4
OUT_TOL = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    return torch.device("cuda:0")


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def assert_codes(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, what
    bad = got != ref
    frac = float(bad.mean()) if bad.size else 0.0
    if bad.any():
        step = np.abs(got.astype(np.int32) - ref.astype(np.int32))[bad].max()
        assert step <= 1, f"{what}: code differs by {step}"
    assert frac <= CODE_MISMATCH_MAX, f"{what}: {frac:.2e} of codes differ"
    return frac


def assert_out(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= OUT_TOL * rms(ref) or err == 0.0, f"{what}: max err {err:.3e}, rms {rms(ref):.3e}"
    return err


def make_plan(L, d, xdt=torch.float32, ydt=None, algo="auto", **shape):
    return q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], x_dtype=xdt, y_dtype=ydt, algo=algo, **shape)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


# ------------------------------------------------------------ small sizes
SMALL = [WL.small(L) for L in WL.LAYERS.values()]
EDGE = [
    WL.LAYERS["c1_f4_n1_c16_16x16_g16"],                                      # full c1
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], H=1, W=1),                  # 1x1 image
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=3, W=70, Cin=64, Cout=13),          # odd Cout, wide
    WL.small(WL.LAYERS[WL.BENCH_LAYER], N=3, H=7, W=6, Cin=64, Cout=1),       # Cout = 1
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=12, W=12).replace(pad=0, name="pad0"),
    WL.small(WL.LAYERS[WL.BENCH_LAYER], H=5, W=9).replace(pad=2, name="pad2"),
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], Cin=256, Cout=40).replace(G=256, name="g256"),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], Cin=96, Cout=20, H=14, W=14),  # 3 groups
    WL.small(WL.LAYERS["c4_f4_n2_c320_64x64_g64_pert"], N=2, Cin=192, Cout=70, H=21, W=19),
    # stage-2 K chunks: 8 groups of 16 per 128-byte chunk; 4 groups of 32 per chunk
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], N=2, H=9, W=11, Cin=128, Cout=72),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], Cin=128, Cout=80, H=13, W=14),
    # 16-byte chunks over three groups of 16; Cout above one 64-channel block
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], N=1, H=6, W=7, Cin=48, Cout=130),
]


def ids(Ls):
    return [L.name for L in Ls]


@pytest.mark.parametrize("L", SMALL + EDGE, ids=ids(SMALL + EDGE))
def test_stages_and_forward(dev, L):
    print(f"\n[case] {L.name} F({L.m},3) N={L.N} C={L.Cin}->{L.Cout} {L.H}x{L.W} pad={L.pad} "
          f"G={L.G}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True)
    plan = make_plan(L, d)
    # matrices
    Bt, Gm, At = q.wq8_plan_matrices(plan)
    assert np.array_equal(Bt, ref["Bt"]) and np.array_equal(Gm, ref["G"])
    assert np.array_equal(At, ref["At"])
    # weights
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    torch.cuda.synchronize()
    assert_codes(Uq.cpu().numpy(), ref["Uq"], "Uq")
    assert np.array_equal(sU.cpu().numpy(), ref["sU"])
    # stage 1
    Vq, sV = q.wq8_stage1(plan, to_dev(d["x"], dev))
    torch.cuda.synchronize()
    assert_codes(Vq.cpu().numpy(), ref["Vq"], "Vq")
    assert np.array_equal(sV.cpu().numpy(), ref["sV"])
    # stage 2 from the oracle's codes: int32 partials exact, M exact
    oVq, oUq = to_dev(ref["Vq"], dev), to_dev(ref["Uq"], dev)
    P = q.wq8_stage2_i32(plan, oVq, oUq)
    M = q.wq8_stage2(plan, oVq, to_dev(ref["sV"], dev), oUq, to_dev(ref["sU"], dev))
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.stage2_i32(ref["Vq"], ref["Uq"], L.G))
    assert np.array_equal(M.cpu().numpy(), ref["M"])
    # stage 3 from the oracle's M
    y3, Yq, sY = q.wq8_stage3(plan, to_dev(ref["M"], dev), want_codes=True)
    torch.cuda.synchronize()
    assert_codes(Yq.cpu().numpy(), ref["Yq"], "Yq")
    assert np.array_equal(sY.cpu().numpy(), ref["sY"])
    assert_out(y3.cpu().numpy(), ref["y"], "stage-3 output")
    # fused stages 2 + 3 from the oracle's codes
    y23 = q.wq8_stage23(plan, oVq, to_dev(ref["sV"], dev), oUq, to_dev(ref["sU"], dev))
    torch.cuda.synchronize()
    assert_out(y23.cpu().numpy(), ref["y"], "fused stage-2+3 output")
    # whole forward, both schedules
    for algo in ("staged", "fused"):
        p2 = make_plan(L, d, algo=algo)
        y = q.wq8_conv_forward(p2, to_dev(d["x"], dev), Uq, sU)
        torch.cuda.synchronize()
        err = assert_out(y.cpu().numpy(), ref["y"], f"forward ({algo})")
        print(f"[case] {L.name}: {algo} forward max err {err:.3e} (rms {rms(ref['y']):.3e})",
              flush=True)


@pytest.mark.parametrize("algo", ["staged", "fused"])
@pytest.mark.parametrize("xdt,ydt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32)])
def test_bf16_activations(dev, xdt, ydt, algo):
    """bf16 input is widened exactly; bf16 output is the nearest-even rounding
    of the fp32 result. The staged output transform is the oracle's fp32 fma
    chain, so its bf16 bits match exactly; the fused one evaluates A^T Yq A on
    fp16 MFMA parts, so each bf16 value must be a correct rounding of some
    value within the output tolerance of the oracle's."""
    L = WL.small(WL.LAYERS[WL.BENCH_LAYER], N=2, H=15, W=13, Cin=64, Cout=24)
    print(f"\n[case] bf16 {xdt} -> {ydt} {algo} {L.name}", flush=True)
    d = WL.make(L)
    xt = torch.from_numpy(d["x"]).to(xdt)
    x_ref = d["x"] if xdt == torch.float32 else oracle.bf16_bits_to_f32(
        xt.view(torch.int16).numpy().view(np.uint16))
    ref = oracle.forward(L.m, x_ref, d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"])
    plan = make_plan(L, d, xdt, ydt, algo=algo)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    y = q.wq8_conv_forward(plan, xt.to(dev), Uq, sU)
    torch.cuda.synchronize()
    if ydt == torch.bfloat16:
        bits = y.cpu().view(torch.int16).numpy().view(np.uint16)
        want = oracle.f32_to_bf16_bits(ref)
        if algo == "staged":
            assert np.array_equal(bits, want)
        else:
            got = oracle.bf16_bits_to_f32(bits).astype(np.float64)
            r64 = ref.astype(np.float64)
            half_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(got), np.abs(r64)))[1] - 9)
            slack = half_ulp + OUT_TOL * rms(ref)
            assert np.all(np.abs(got - r64) <= slack), "bf16 output off by more than rounding + tolerance"
            print(f"[case] bf16 bits differing from the oracle's rounding: "
                  f"{int(np.sum(bits != want))} of {bits.size}", flush=True)
    else:
        assert_out(y.cpu().numpy(), ref, "bf16-in forward")


def test_zero_input_gives_zero_scales(dev):
    L = WL.small(WL.LAYERS[WL.BENCH_LAYER], N=1, H=9, W=9, Cin=64, Cout=16)
    d = WL.make(L)
    plan = make_plan(L, d)
    x = torch.zeros((L.N, L.Cin, L.H, L.W), device=dev)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    Vq, sV = q.wq8_stage1(plan, x)
    y = q.wq8_conv_forward(plan, x, Uq, sU)
    torch.cuda.synchronize()
    assert not Vq.any() and not sV.any() and not y.any()


def test_forward_is_deterministic(dev):
    L = WL.LAYERS["c3a_f6_n32_c128_28x28_g64"]
    d = WL.make(L)
    plan = make_plan(L, d)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    x = to_dev(d["x"], dev)
    ws = plan.empty_workspace(dev)
    a = q.wq8_conv_forward(plan, x, Uq, sU, workspace=ws).clone()
    ws.fill_(0x5A)
    b = q.wq8_conv_forward(plan, x, Uq, sU, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ------------------------------------------------------------- full sizes
FULL = list(WL.LAYERS.values())


def equalizing(m):
    """Data-free equalizing scales written by tests/golden/make_equalized_scales.py
    (which calls only oracle/)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "equalized_scales.json")) as f:
        e = json.load(f)[f"F({m},3)"]
    return np.array(e["s_B"], np.float32), np.array(e["s_G"], np.float32)


def scale_set(L, which):
    n = L.m + 2
    if which == "config":
        return WL.make_scales(L)
    if which == "standard":
        return np.ones(n, np.float32), np.ones(n, np.float32)
    if which == "equalizing":
        return equalizing(L.m)
    if which == "learned":
        from quantized_convolution_amd import scales as S
        sb, sg = S.recorded_learned_scales(L.m)
        return np.array(sb, np.float32), np.array(sg, np.float32)
    raise ValueError(which)


def check_full(L, d, dev, schedules, stages=True):
    """Every element of a full-size layer against the oracle, launched as
    the benchmark launches it (wq8_conv_forward with a plan-sized
    workspace): Uq, sU, Vq, sV in full; M (int8 GEMMs from the oracle's
    codes) bit-exact; Yq, sY and the stage-3 output from the oracle's M;
    the fused stages 2+3 from the oracle's codes; the whole forward for
    each schedule in `schedules` against the oracle output at 1e-3 of its
    RMS. Returns {schedule: max error / RMS}."""
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True)
    r = rms(ref["y"])
    plan = make_plan(L, d)
    x = to_dev(d["x"], dev)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    Vq, sV = q.wq8_stage1(plan, x)
    torch.cuda.synchronize()
    fu = assert_codes(Uq.cpu().numpy(), ref["Uq"], "Uq")
    fv = assert_codes(Vq.cpu().numpy(), ref["Vq"], "Vq")
    if fu == 0:
        assert np.array_equal(sU.cpu().numpy(), ref["sU"]), "sU"
    if fv == 0:
        assert np.array_equal(sV.cpu().numpy(), ref["sV"]), "sV"
    if stages:
        oVq, osV = to_dev(ref["Vq"], dev), to_dev(ref["sV"], dev)
        oUq, osU = to_dev(ref["Uq"], dev), to_dev(ref["sU"], dev)
        ps = make_plan(L, d, algo="staged")
        M = q.wq8_stage2(ps, oVq, osV, oUq, osU)
        torch.cuda.synchronize()
        assert np.array_equal(M.cpu().numpy(), ref["M"]), "M"
        del M
        y3, Yq, sY = q.wq8_stage3(ps, to_dev(ref["M"], dev), want_codes=True)
        torch.cuda.synchronize()
        assert_codes(Yq.cpu().numpy(), ref["Yq"], "Yq")
        assert np.array_equal(sY.cpu().numpy(), ref["sY"]), "sY"
        assert_out(y3.cpu().numpy(), ref["y"], "stage-3 output")
        del y3, Yq, sY
        y23 = q.wq8_stage23(make_plan(L, d, algo="fused"), oVq, osV, oUq, osU)
        torch.cuda.synchronize()
        assert_out(y23.cpu().numpy(), ref["y"], "fused stage-2+3 output")
        del y23, oVq, osV, oUq, osU
    errs, outs = {}, {}
    for algo in schedules:
        p2 = make_plan(L, d, algo=algo)
        y = q.wq8_conv_forward(p2, x, Uq, sU, workspace=p2.empty_workspace(dev))
        torch.cuda.synchronize()
        outs[algo] = y.cpu().numpy()
        errs[algo] = assert_out(outs[algo], ref["y"], f"forward ({algo})") / r
    if "staged" in outs and "fused" in outs:
        # identical codes; only the fp16 evaluation of A^T Yq A differs
        diff = float(np.max(np.abs(outs["staged"].astype(np.float64) - outs["fused"])))
        assert diff <= 2e-5 * r, f"fused vs staged forward: {diff / r:.2e} rms"
    return errs


@pytest.mark.parametrize("L", FULL, ids=ids(FULL))
def test_full_size_elementwise(dev, L):
    """Full configuration with its own scales, every element, both schedules
    and the schedule the plan picks."""
    print(f"\n[case] full {L.name} ({L.scales} scales)", flush=True)
    d = WL.make(L)
    errs = check_full(L, d, dev, ("staged", "fused", "auto"))
    print(f"[case] full {L.name}: max err / rms " +
          ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


@pytest.mark.parametrize("which", ["standard", "equalizing", "learned"])
@pytest.mark.parametrize("L", FULL, ids=ids(FULL))
def test_full_size_scale_sets(dev, L, which):
    """Full configuration under the standard scales (S = I), the equalizing
    scales (F(6,3) s_B spans 0.13 to 24.8) and the learned ones
    (quantized_convolution_amd/data/learned_scales.json): codes and scales of
    every stage, and the forward the plan picks, element by element."""
    sb, sg = scale_set(L, which)
    print(f"\n[case] full {L.name} ({which} scales)", flush=True)
    d = dict(WL.make(L), s_b=sb, s_g=sg)
    errs = check_full(L, d, dev, ("auto",))
    print(f"[case] full {L.name} ({which}): max err / rms {errs['auto']:.2e}", flush=True)


@pytest.mark.parametrize("name", ["c2_f6_n32_c64_56x56_g64", "c4_f4_n2_c320_64x64_g64_pert",
                                  "c5_f6_n8_c640_32x32_g32"])
def test_fused_output_transform_precision(dev, name):
    """The fused kernel evaluates A^T Yq A on fp16 matrix cores with the
    Kronecker matrix split into two fp16 parts; on identical codes it must
    agree with the staged fp32 chain to a few 1e-6 of the output RMS (far
    inside the 1e-3 output tolerance)."""
    L = WL.small(WL.LAYERS[name], N=2, H=23, W=21, Cin=64, Cout=48)
    print(f"\n[case] fused-vs-staged precision {L.name}", flush=True)
    d = WL.make(L)
    ys = {}
    for algo in ("staged", "fused"):
        plan = make_plan(L, d, algo=algo)
        Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
        ys[algo] = q.wq8_conv_forward(plan, to_dev(d["x"], dev), Uq, sU).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    err = float(np.max(np.abs(ys["fused"] - ys["staged"])))
    r = rms(ys["staged"])
    print(f"[case] max |fused - staged| = {err:.3e} = {err / r:.2e} rms", flush=True)
    assert err <= 2e-5 * r


@pytest.mark.parametrize("rows", ["full", "half"])
@pytest.mark.parametrize("L", [
    WL.small(WL.LAYERS[WL.BENCH_LAYER], N=2, H=13, W=30, Cin=128, Cout=8),
    WL.small(WL.LAYERS[WL.BENCH_LAYER], N=1, H=9, W=17, Cin=64, Cout=8).replace(pad=2, name="pad2w17"),
    WL.small(WL.LAYERS["c4_f4_n2_c320_64x64_g64_pert"], N=1, H=11, W=21, Cin=64, Cout=8),
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], N=2, H=9, W=11, Cin=48, Cout=8),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g128"], N=1, H=10, W=12, Cin=256, Cout=8),
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], N=1, H=7, W=26, Cin=96, Cout=8),
], ids=lambda L: L.name)
def test_stage1_window_rows(dev, rows, L):
    """Stage 1 holds all n window rows in LDS, or half of them at a time
    (the launch picks by how many strips the GPU can hold; the plan's
    stage1_rows forces one): both give the oracle's codes and scales bit for
    bit."""
    print(f"\n[case] stage-1 {rows} rows {L.name}", flush=True)
    d = WL.make(L)
    from oracle import transforms as T
    Bt = T.transforms_f32(L.m, list(d["points"]), d["s_b"], d["s_g"])[0]
    oVq, osV = oracle.stage1(L.m, d["x"], L.pad, L.G, Bt)
    plan = make_plan(L, d, stage1_rows={"full": 1, "half": 2}[rows])
    Vq, sV = q.wq8_stage1(plan, to_dev(d["x"], dev))
    torch.cuda.synchronize()
    assert np.array_equal(Vq.cpu().numpy(), oVq) and np.array_equal(sV.cpu().numpy(), osV)


@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("name,kw", [
    ("c2_f6_n32_c64_56x56_g64", dict(N=2, H=30, W=26, Cin=64, Cout=40)),
    ("c3c_f6_n32_c512_7x7_g64", dict(N=3, H=7, W=7, Cin=192, Cout=24)),
    ("c5_f6_n8_c640_32x32_g32", dict(N=1, H=13, W=17, Cin=96, Cout=20)),
    ("c5_f6_n8_c1280_16x16_g128", dict(N=1, H=9, W=11, Cin=256, Cout=17)),
])
def test_fused_block_shapes(dev, waves, name, kw):
    """The fused kernel splits a block's taps over 4, 8 or 16 waves (the
    launch picks by block count; the plan's fused_waves forces one): every
    shape gives the oracle's result, for one and several quantization
    groups."""
    L = WL.small(WL.LAYERS[name], **kw)
    print(f"\n[case] fused waves={waves} {L.name} C={L.Cin}->{L.Cout} {L.H}x{L.W} G={L.G}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"])
    plan = make_plan(L, d, algo="fused", fused_waves=waves, fused_block=1)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    y = q.wq8_conv_forward(plan, to_dev(d["x"], dev), Uq, sU)
    torch.cuda.synchronize()
    assert_out(y.cpu().numpy(), ref, f"fused forward, {waves} waves")


@pytest.mark.parametrize("name,kw", [
    ("c2_f6_n32_c64_56x56_g64", dict(N=2, H=30, W=26, Cin=64, Cout=40)),
    ("c5_f6_n8_c640_32x32_g32", dict(N=1, H=13, W=17, Cin=96, Cout=20)),
])
def test_fused_wave_counts_agree(dev, name, kw):
    """16 x 16 fused blocks of 4, 8 and 16 waves split the same per-pair work
    differently: their outputs agree bit for bit."""
    L = WL.small(WL.LAYERS[name], **kw)
    print(f"\n[case] fused wave counts {L.name}", flush=True)
    d = WL.make(L)
    x, w = to_dev(d["x"], dev), to_dev(d["w"], dev)
    outs = {}
    for waves in ("4", "8", "16"):
        plan = make_plan(L, d, algo="fused", fused_waves=int(waves), fused_block=1)
        Uq, sU = q.wq8_weights_prepare(plan, w)
        outs[waves] = q.wq8_conv_forward(plan, x, Uq, sU)
        torch.cuda.synchronize()
    assert torch.equal(outs["4"], outs["8"]) and torch.equal(outs["4"], outs["16"])


@pytest.mark.parametrize("pad", [None, 0, 2])
@pytest.mark.parametrize("name,kw,G,ydt", [
    # tiles and channels not multiples of 32
    ("c2_f6_n32_c64_56x56_g64", dict(N=2, H=30, W=26, Cin=64, Cout=40), None, None),
    # three groups of 32 (the group loop and its cross-group prefetch)
    ("c5_f6_n8_c640_32x32_g32", dict(N=1, H=13, W=17, Cin=96, Cout=20), None, None),
    # groups of 16 (half of each K slot is zero), several groups of 64
    ("c2_f6_n32_c64_56x56_g64", dict(N=1, H=19, W=14, Cin=64, Cout=33), 16, None),
    ("c3c_f6_n32_c512_7x7_g64", dict(N=3, H=7, W=7, Cin=192, Cout=72), None, None),
    # bf16 output
    ("c2_f6_n32_c64_56x56_g64", dict(N=2, H=30, W=26, Cin=64, Cout=40), None, torch.bfloat16),
    # two tiles in all (blocks almost all padding), one output channel past a block
    ("c2_f6_n32_c64_56x56_g64", dict(N=1, H=5, W=9, Cin=64, Cout=33), None, None),
])
def test_fused_wide_blocks(dev, name, kw, G, ydt, pad):
    """Wide fused blocks (32 x 32, 32 tiles x 16 channels, 16 tiles x 32
    channels; each tap's operands feed two or four MFMAs): the oracle's
    result, and bit for bit the output of the 16 x 16 blocks, whose per-pair
    arithmetic they repeat."""
    L = WL.small(WL.LAYERS[name], **kw)
    if G is not None:
        L = L.replace(G=G, name=L.name + f"_g{G}")
    if pad is not None:
        L = L.replace(pad=pad, name=L.name + f"_pad{pad}")
    print(f"\n[case] fused wide {L.name} C={L.Cin}->{L.Cout} {L.H}x{L.W} G={L.G} y={ydt}", flush=True)
    d = WL.make(L)
    x, w = to_dev(d["x"], dev), to_dev(d["w"], dev)
    outs = {}
    for wide in ("0", "1", "2", "3"):
        plan = make_plan(L, d, ydt=ydt, algo="fused", fused_block=int(wide) + 1)
        Uq, sU = q.wq8_weights_prepare(plan, w)
        outs[wide] = q.wq8_conv_forward(plan, x, Uq, sU)
        torch.cuda.synchronize()
    for wide in ("1", "2", "3"):
        assert torch.equal(outs["0"], outs[wide]), f"wide blocks ({wide}) and 16 x 16 blocks differ"
    if ydt is None:
        ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                             s_g=d["s_g"])
        assert_out(outs["1"].cpu().numpy(), ref, "fused forward, wide blocks")


@pytest.mark.parametrize("name,kw", [
    ("c2_f6_n32_c64_56x56_g64", dict(N=2, H=17, W=23, Cin=64, Cout=24)),
    ("c4_f4_n2_c320_64x64_g64_pert", dict(N=1, H=13, W=9, Cin=128, Cout=20)),
])
def test_per_row_y_scales(dev, name, kw):
    """One Y scale per row of taps (staged schedule): Y codes and scales
    bit-exact from the oracle's M; forward output within tolerance; the
    fused entry point refuses the plan."""
    L = WL.small(WL.LAYERS[name], **kw)
    print(f"\n[case] per-row Y {L.name}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True, y_group="row")
    plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                  s_G=d["s_g"], y_group="row")
    assert not plan.fused
    y3, Yq, sY = q.wq8_stage3(plan, to_dev(ref["M"], dev), want_codes=True)
    Uq, sU = q.wq8_weights_prepare(plan, to_dev(d["w"], dev))
    y = q.wq8_conv_forward(plan, to_dev(d["x"], dev), Uq, sU)
    torch.cuda.synchronize()
    assert np.array_equal(Yq.cpu().numpy(), ref["Yq"]) and np.array_equal(sY.cpu().numpy(), ref["sY"])
    assert_out(y3.cpu().numpy(), ref["y"], "per-row stage 3")
    assert_out(y.cpu().numpy(), ref["y"], "per-row forward")
    with pytest.raises(q.Wq8Error) as e:
        q.wq8_stage23(plan, *q.wq8_stage1(plan, to_dev(d["x"], dev)), Uq, sU)
    assert e.value.status == -2


@pytest.mark.parametrize("y_group", ["tile", "row"])
@pytest.mark.parametrize("name,kw,ydt", [
    ("c5_f6_n8_c1280_16x16_g32", dict(N=2, H=16, W=16, Cin=64, Cout=50), torch.float32),   # 18 tiles
    ("c4_f4_n2_c320_64x64_g64_pert", dict(N=1, H=13, W=22, Cin=64, Cout=33), torch.float32),
    ("c5_f6_n8_c640_32x32_g128", dict(N=1, H=20, W=14, Cin=128, Cout=40), torch.bfloat16),
    ("c3c_f6_n32_c512_7x7_g64", dict(N=3, H=7, W=7, Cin=64, Cout=70), torch.float32),       # odd W, 12 tiles
])
def test_stage3_lanes(dev, name, kw, ydt, y_group):
    """The output transform with one lane per (tile, channel) pair and with
    two (each holding half the columns of taps; the launch takes two on
    layers with few pairs; stage3_lanes forces either): Y codes and scales
    bit-exact from the oracle's M for both, and the two outputs bit-identical
    (the same fma chains), within tolerance of the oracle."""
    L = WL.small(WL.LAYERS[name], **kw)
    print(f"\n[case] stage-3 lanes {L.name} {ydt} y_group={y_group}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True, y_group=y_group)
    M = to_dev(ref["M"], dev)
    outs = {}
    for lanes in (1, 2):
        plan = q.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, points=d["points"], s_B=d["s_b"],
                      s_G=d["s_g"], y_dtype=ydt, algo="staged", y_group=y_group, stage3_lanes=lanes)
        y3, Yq, sY = q.wq8_stage3(plan, M, want_codes=True)
        torch.cuda.synchronize()
        assert np.array_equal(Yq.cpu().numpy(), ref["Yq"]), f"Yq, {lanes} lane(s)"
        assert np.array_equal(sY.cpu().numpy(), ref["sY"]), f"sY, {lanes} lane(s)"
        outs[lanes] = y3.cpu()
    assert torch.equal(outs[1].view(torch.int16 if ydt == torch.bfloat16 else torch.int32),
                       outs[2].view(torch.int16 if ydt == torch.bfloat16 else torch.int32))
    if ydt == torch.float32:
        assert_out(outs[2].numpy(), ref["y"], "stage-3 output")


# every block shape of the register-streamed Hadamard kernel (stage2_rows
# 4/5/6/8 x channel tiles 1/2 x 2/4 waves) and the LDS-pipelined one (1),
# on layers with partial chunks (odd group counts), ragged tiles and
# channels, and each group size
HGEMM_SHAPES = [(1, 0, 0)] + [(r, c, w) for r in (4, 5, 6, 8) for c in (1, 2) for w in (2, 4)
                              if not (c == 2 and r > 5)]
HGEMM_LAYERS = [
    WL.small(WL.LAYERS["c1_f4_n1_c16_16x16_g16"], N=2, H=15, W=13, Cin=80, Cout=37),     # G=16, 5 groups
    WL.small(WL.LAYERS["c5_f6_n8_c640_32x32_g32"], N=1, H=29, W=31, Cin=160, Cout=70),   # G=32, 5 groups
    WL.small(WL.LAYERS["c4_f6_n2_c320_64x64_g64_pert"], N=1, H=20, W=9, Cin=192, Cout=19),  # G=64, 3 groups
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], N=2, H=11, W=16, Cin=384, Cout=33),  # G=128
    WL.small(WL.LAYERS["c5_f6_n8_c1280_16x16_g128"], N=1, H=9, W=9, Cin=512, Cout=20).replace(G=256, name="h256"),
]


@pytest.mark.parametrize("L", HGEMM_LAYERS, ids=ids(HGEMM_LAYERS))
def test_hgemm_block_shapes(dev, L):
    """int32 partials and M bit-exact for every block shape of both Hadamard
    kernels, from the oracle's codes."""
    print(f"\n[case] hgemm shapes {L.name} G={L.G} Cin={L.Cin} Cout={L.Cout}", flush=True)
    d = WL.make(L)
    ref = oracle.forward(L.m, d["x"], d["w"], L.pad, L.G, points=list(d["points"]), s_b=d["s_b"],
                         s_g=d["s_g"], keep=True)
    P_ref = oracle.stage2_i32(ref["Vq"], ref["Uq"], L.G)
    oVq, osV = to_dev(ref["Vq"], dev), to_dev(ref["sV"], dev)
    oUq, osU = to_dev(ref["Uq"], dev), to_dev(ref["sU"], dev)
    for rows, cols, waves in HGEMM_SHAPES:
        plan = make_plan(L, d, algo="staged", stage2_rows=rows, stage2_cols=cols, stage2_waves=waves)
        P = q.wq8_stage2_i32(plan, oVq, oUq)
        M = q.wq8_stage2(plan, oVq, osV, oUq, osU)
        torch.cuda.synchronize()
        assert np.array_equal(P.cpu().numpy(), P_ref), f"P, shape {(rows, cols, waves)}"
        assert np.array_equal(M.cpu().numpy(), ref["M"]), f"M, shape {(rows, cols, waves)}"
