"""Host-side checks of the HIP library: it loads, exports every entry point the
header declares, validates descriptors, and builds the same fp32 transform
matrices as the oracle's exact construction. No kernel is launched."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest
import torch

from oracle import transforms as T
from quantized_convolution_amd import binding as B
from quantized_convolution_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAS_GPU = torch.cuda.is_available()


def header_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(wq8_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    declared = header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTS)


def _create(**kw):
    base = dict(m=6, points=None, s_B=None, s_G=None, group=64, N=1, Cin=64, Cout=64, H=16, W=16,
                pad=1, x_dtype=0, y_dtype=0, algo=0, y_group=0, in_quant=0, stage1_rows=0,
                fused_waves=0, fused_block=0, stage2_rows=0, stage2_cols=0,
                stage2_waves=0, stage3_lanes=0)
    base.update(kw)
    keep = []

    def arr(v, ct, dt):
        if v is None:
            return None
        a = np.ascontiguousarray(v, dtype=dt)
        keep.append(a)
        return a.ctypes.data_as(C.POINTER(ct))

    d = B.wq8_desc(base["m"], arr(base["points"], C.c_double, np.float64),
                   arr(base["s_B"], C.c_float, np.float32), arr(base["s_G"], C.c_float, np.float32),
                   base["group"], base["N"], base["Cin"], base["Cout"], base["H"], base["W"],
                   base["pad"], base["x_dtype"], base["y_dtype"], base["algo"], base["y_group"],
                   base["in_quant"], base["stage1_rows"], base["fused_waves"], base["fused_block"],
                   base["stage2_rows"], base["stage2_cols"], base["stage2_waves"], base["stage3_lanes"])
    h = C.c_void_p()
    st = B.wq8_plan_create(d, h)
    if st == 0:
        B.load().wq8_plan_destroy(h)
    return st


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    (dict(m=4), 0),
    (dict(m=5), -2), (dict(m=2), -2),
    (dict(group=48), -2), (dict(group=8), -2),
    (dict(Cin=96, group=64), -1), (dict(Cin=96, group=32), 0),
    (dict(pad=3), -1), (dict(pad=-1), -1),
    (dict(H=1, W=1, pad=0), -1), (dict(H=1, W=1, pad=1), 0),
    (dict(N=0), -1), (dict(Cout=0), -1),
    (dict(x_dtype=7), -1), (dict(algo=3), -1), (dict(algo=1), 0), (dict(algo=2), 0),
    (dict(y_group=1), 0), (dict(y_group=2), -1), (dict(y_group=1, algo=2), -2),
    (dict(y_group=1, algo=1), 0),
    (dict(in_quant=1), 0), (dict(in_quant=2, algo=2), 0), (dict(in_quant=3), -1),
    (dict(in_quant=-1), -1),
    (dict(points=[0, 1, -1, 2, 2, .5, -.5, math.inf]), -3),
    (dict(points=[0, 1, -1, 2, -2, .5, math.inf, math.inf]), -3),
    (dict(points=[0, 1, -1, 2, -2, .5, -.5, math.nan]), -1),
    (dict(s_B=[1, 1, 0, 1, 1, 1, 1, 1]), -1),
    (dict(s_G=[1, 1, 1, 1, math.inf, 1, 1, 1]), -1),
    (dict(s_B=[3e38] * 8, s_G=[1e-3] * 8), -1),
    (dict(N=4096, Cin=1024, Cout=1024, H=512, W=512, group=64), -2),
    # kernel-shape fields: 0 = chosen at launch; out of range -1; not built -2
    (dict(stage1_rows=1), 0), (dict(stage1_rows=2), 0), (dict(stage1_rows=3), -1),
    (dict(stage1_rows=-1), -1), (dict(stage1_rows=2, in_quant=1), -2),
    (dict(fused_waves=4), 0), (dict(fused_waves=8), 0), (dict(fused_waves=16), 0),
    (dict(fused_waves=6), -1), (dict(fused_waves=8, m=4), -2), (dict(fused_waves=4, m=4), 0),
    (dict(fused_block=1), 0), (dict(fused_block=4), 0), (dict(fused_block=5), -1),
    (dict(fused_block=-1), -1), (dict(fused_block=2, m=4), -2),
    (dict(fused_block=3, group=128, Cin=128), -2), (dict(fused_block=1, group=128, Cin=128), 0),
    (dict(stage2_rows=1), 0), (dict(stage2_rows=5), 0), (dict(stage2_rows=3), -1), (dict(stage2_rows=7), -1),
    (dict(stage2_cols=2, stage2_rows=5), 0), (dict(stage2_cols=2, stage2_rows=6), -2),
    (dict(stage2_cols=3), -1), (dict(stage2_waves=2), 0), (dict(stage2_waves=3), -1),
    (dict(stage3_lanes=1), 0), (dict(stage3_lanes=2), 0), (dict(stage3_lanes=3), -1), (dict(stage3_lanes=-1), -1),
])
def test_plan_validation(kw, status):
    assert _create(**kw) == status


def test_last_error_names_the_problem():
    assert _create(group=48) == -2
    assert b"group" in B.load().wq8_last_error()
    assert B.load().wq8_status_string(-4) == b"workspace too small"


def _scale_sets():
    sets = [("identity", np.ones(8, np.float32), np.ones(8, np.float32))]
    for name, L in WL.LAYERS.items():
        if L.m == 6 and L.scales == "perturbed":
            sb, sg = WL.make_scales(L)
            sets.append((name, sb, sg))
    r = np.random.default_rng(77)
    for k in range(20):
        sets.append((f"rand{k}", np.exp(r.uniform(-2, 2, 8)).astype(np.float32) * r.choice([-1, 1], 8),
                     np.exp(r.uniform(-2, 2, 8)).astype(np.float32)))
    return sets


@pytest.mark.parametrize("m", [4, 6])
def test_plan_matrices_equal_exactly_rounded(m):
    n = m + 2
    for name, sb, sg in _scale_sets():
        sb, sg = sb[:n], sg[:n]
        plan = B.Plan(m, 1, 16, 16, 9, 9, 1, 16, s_B=sb, s_G=sg)
        Bt, Gm, At = B.wq8_plan_matrices(plan)
        rb, rg, ra = T.transforms_f32(m, T.standard_points(m), sb, sg)
        assert np.array_equal(Bt, rb), name
        assert np.array_equal(Gm, rg), name
        assert np.array_equal(At, ra), name


@pytest.mark.parametrize("m", [4, 6])
@pytest.mark.parametrize("iq", ["int_tensor", "int_row"])
def test_plan_bt_codes_match_oracle(m, iq):
    """The host's B^T quantization for the integer input stage equals the
    oracle's (same fp32 absmax quantizer, per matrix or per row)."""
    import oracle
    n = m + 2
    for name, sb, sg in _scale_sets():
        sb, sg = sb[:n], sg[:n]
        plan = B.Plan(m, 1, 16, 16, 9, 9, 1, 16, s_B=sb, s_G=sg, in_quant=iq)
        Bq, sq = B.wq8_plan_bt_codes(plan)
        Bt, _, _ = B.wq8_plan_matrices(plan)
        rq, rs = oracle.quant_bt(Bt, iq == "int_row")
        assert np.array_equal(Bq, rq), name
        assert np.array_equal(sq, rs), name


def test_plan_bt_codes_rejects_fp32_plan():
    plan = B.Plan(6, 1, 16, 16, 9, 9, 1, 16)
    with pytest.raises(B.Wq8Error) as e:
        B.wq8_plan_bt_codes(plan)
    assert e.value.status == -1


def test_plan_query_sizes():
    L = WL.LAYERS[WL.BENCH_LAYER]
    plan = B.Plan(L.m, L.N, L.Cin, L.Cout, L.H, L.W, L.pad, L.G, algo="staged")
    n2 = L.n ** 2
    assert plan.T == L.tiles == 3200
    assert plan.u_code_bytes == n2 * L.Cout * L.Cin
    assert plan.u_scale_bytes == n2 * L.Cout * (L.Cin // L.G) * 4
    assert plan.workspace_bytes >= n2 * plan.T * (L.Cin + 4 * (L.Cin // L.G) + 4 * L.Cout)


@pytest.mark.skipif(HAS_GPU, reason="host-only argument checks; uses fake device pointers")
def test_forward_rejects_bad_arguments_before_launch():
    lib = B.load()
    plan = B.Plan(6, 1, 64, 64, 16, 16, 1, 64, algo="staged")
    h = plan.handle
    good = C.c_void_p(0x10000)
    ws = plan.workspace_bytes
    f = lib.wq8_conv_forward
    assert f(None, good, good, good, C.c_void_p(0x20000), good, ws, None) == -1
    assert f(h, None, good, good, C.c_void_p(0x20000), good, ws, None) == -1
    assert f(h, C.c_void_p(0x10004), good, good, C.c_void_p(0x20000), good, ws, None) == -5
    assert f(h, good, good, good, C.c_void_p(0x20000), good, ws - 1, None) == -4
    assert f(h, good, good, good, good, C.c_void_p(0x30000), ws, None) == -1   # x == y
    assert lib.wq8_stage3(h, good, None, None, None, None) == -1
    assert lib.wq8_stage3(h, good, good, C.c_void_p(0x40008), None, None) == -5


def test_plan_reports_schedule():
    small = B.Plan(6, 32, 64, 64, 56, 56, 1, 64)                 # 256 KB of weights: fused
    big = B.Plan(6, 8, 1280, 1280, 16, 16, 1, 32)                # 105 MB of weights: staged
    assert small.fused and not big.fused
    assert B.Plan(6, 8, 1280, 1280, 16, 16, 1, 32, algo="fused").fused
    assert not B.Plan(6, 32, 64, 64, 56, 56, 1, 64, algo="staged").fused
    st = B.Plan(6, 32, 64, 64, 56, 56, 1, 64, algo="staged")
    assert small.workspace_bytes < st.workspace_bytes            # no M buffer when fused


def test_no_environment_reads_in_library_sources():
    """Kernel shapes come from the descriptor only: the library reads no
    process environment."""
    csrc = os.path.join(ROOT, "quantized_convolution_amd", "csrc")
    for f in os.listdir(csrc):
        src = open(os.path.join(csrc, f)).read()
        assert "getenv" not in src, f


def _tiny_plan(**kw):
    return B.Plan(6, 1, 64, 16, 9, 9, 1, 64, algo="staged", **kw)


def _cases(plan):
    """(callable, what) pairs, each with one bad buffer; all others are good
    CPU tensors (so the only failure a correct check can report before the
    device check is the planted one)."""
    f32, i8 = torch.float32, torch.int8
    x = torch.zeros(plan.x_shape)
    Uq, sU = torch.zeros(plan.uq_shape, dtype=i8), torch.zeros(plan.su_shape)
    Vq, sV = torch.zeros(plan.vq_shape, dtype=i8), torch.zeros(plan.sv_shape)
    M = torch.zeros(plan.m_shape)
    y = torch.zeros(plan.y_shape)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    return [
        (lambda: B.wq8_conv_forward(plan, x.double(), Uq, sU, y, ws), "x must be"),
        (lambda: B.wq8_conv_forward(plan, x[:, :, :8], Uq, sU, y, ws), "x must have shape"),
        (lambda: B.wq8_conv_forward(plan, x, Uq[:, :8], sU, y, ws), "Uq must have shape"),
        (lambda: B.wq8_conv_forward(plan, x, Uq.to(torch.uint8), sU, y, ws), "Uq must be"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU.double(), y, ws), "sU must be"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU, y.to(torch.bfloat16), ws), "y must be"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU, y[:, :, :1], ws), "y must have shape"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU, y, ws[:-1]), "workspace holds"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU, y, ws), "must be on a GPU"),
        (lambda: B.wq8_stage1(plan, x, Vq[:, :1], sV), "Vq must have shape"),
        (lambda: B.wq8_stage1(plan, x, Vq, sV.to(f32)[:, :, :0]), "sV must have shape"),
        (lambda: B.wq8_stage2(plan, Vq, sV, Uq, sU, M.double()), "M must be"),
        (lambda: B.wq8_stage2(plan, Vq, sV, Uq, sU, M[:1]), "M must have shape"),
        (lambda: B.wq8_stage2_i32(plan, Vq, Uq, torch.zeros(1, dtype=torch.int32)), "P must have shape"),
        (lambda: B.wq8_stage3(plan, M[:, :1], y), "M must have shape"),
        (lambda: B.wq8_stage3(plan, M, y, Yq=torch.zeros(1, dtype=i8),
                              sY=torch.zeros((plan.T, plan.Cout))), "Yq must have shape"),
        (lambda: B.wq8_stage23(plan, Vq, sV, Uq, sU, y.t() if y.dim() == 2 else y[:, :, :, :1]),
         "y must have shape"),
        (lambda: B.wq8_stage23(plan, Vq, sV, Uq, sU, torch.zeros(plan.y_shape).transpose(2, 3)),
         "y must be contiguous"),
        (lambda: B.wq8_weights_prepare(plan, torch.zeros((16, 64, 3, 3)), Uq, sU[..., :0]), "sU must have shape"),
        (lambda: B.wq8_direct_conv(plan, torch.zeros((1, 9, 9, 64), dtype=i8), torch.zeros((1, 9, 9, 1)),
                                   torch.zeros((9, 16, 64), dtype=i8), torch.zeros((9, 16, 2)), y),
         "sW must have shape"),
        (lambda: B.wq8_direct_forward(plan, x, torch.zeros((9, 16, 64), dtype=i8), torch.zeros((9, 16, 1)), y,
                                      torch.zeros(8, dtype=torch.uint8)), "workspace holds"),
        (lambda: B.wq8_conv_forward(plan, x, Uq, sU, "not a tensor", ws), "y must be a torch tensor"),
    ]


@pytest.mark.parametrize("k", range(22))
def test_binding_rejects_bad_buffers_before_launch(k):
    """Every wrapper checks dtype, shape, contiguity and device of every
    buffer against the plan and raises ValueError before any call into the
    library (the kernels size their accesses from the plan, not from the
    tensors)."""
    plan = _tiny_plan()
    cases = _cases(plan)
    assert len(cases) == 22
    fn, what = cases[k]
    with pytest.raises(ValueError, match=what):
        fn()


@pytest.mark.skipif(not HAS_GPU, reason="needs two kinds of device")
def test_binding_rejects_mixed_devices():
    plan = _tiny_plan()
    x = torch.zeros(plan.x_shape, device="cuda")
    Uq = torch.zeros(plan.uq_shape, dtype=torch.int8)
    sU = torch.zeros(plan.su_shape, device="cuda")
    with pytest.raises(ValueError, match="must be on a GPU"):
        B.wq8_conv_forward(plan, x, Uq, sU)
