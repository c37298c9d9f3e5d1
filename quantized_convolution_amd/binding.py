"""ctypes binding for libwino_q8_conv.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: torch supplies device memory and the current HIP
stream, the HIP kernels do the work. If the shared library is missing the
import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwino_q8_conv.so")

WQ8_F32, WQ8_BF16 = 0, 1
ALGOS = {"auto": 0, "staged": 1, "fused": 2}
YGROUPS = {"tile": 0, "row": 1}
IN_QUANTS = {"fp32": 0, "int_tensor": 1, "int_row": 2}
_DT = {torch.float32: WQ8_F32, torch.bfloat16: WQ8_BF16}


class Wq8Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class wq8_desc(C.Structure):
    _fields_ = [("m", C.c_int), ("points", C.POINTER(C.c_double)),
                ("s_B", C.POINTER(C.c_float)), ("s_G", C.POINTER(C.c_float)),
                ("group", C.c_int), ("N", C.c_int), ("Cin", C.c_int), ("Cout", C.c_int),
                ("H", C.c_int), ("W", C.c_int), ("pad", C.c_int),
                ("x_dtype", C.c_int), ("y_dtype", C.c_int), ("algo", C.c_int), ("y_group", C.c_int),
                ("in_quant", C.c_int)]


EXPORTS = ("wq8_plan_create", "wq8_plan_destroy", "wq8_plan_query", "wq8_plan_matrices",
           "wq8_plan_bt_codes",
           "wq8_weights_prepare", "wq8_conv_forward", "wq8_stage1", "wq8_stage2",
           "wq8_stage2_i32", "wq8_stage3", "wq8_stage23", "wq8_direct_query",
           "wq8_direct_weights_prepare", "wq8_direct_quantize_x", "wq8_direct_conv",
           "wq8_direct_forward", "wq8_status_string", "wq8_last_error")

_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = C.CDLL(path)
    P, S, i = C.c_void_p, C.c_size_t, C.c_int
    lib.wq8_plan_create.argtypes = [C.POINTER(wq8_desc), C.POINTER(P)]
    lib.wq8_plan_destroy.argtypes = [P]
    lib.wq8_plan_destroy.restype = None
    lib.wq8_plan_query.argtypes = [P, C.POINTER(S), C.POINTER(S), C.POINTER(S), C.POINTER(C.c_int64),
                                   C.POINTER(C.c_int)]
    lib.wq8_plan_matrices.argtypes = [P, P, P, P]
    lib.wq8_plan_bt_codes.argtypes = [P, P, P]
    lib.wq8_weights_prepare.argtypes = [P, P, P, P, P]
    lib.wq8_conv_forward.argtypes = [P, P, P, P, P, P, S, P]
    lib.wq8_stage1.argtypes = [P, P, P, P, P]
    lib.wq8_stage2.argtypes = [P, P, P, P, P, P, P]
    lib.wq8_stage2_i32.argtypes = [P, P, P, P, P]
    lib.wq8_stage3.argtypes = [P, P, P, P, P, P]
    lib.wq8_stage23.argtypes = [P, P, P, P, P, P, P]
    lib.wq8_direct_query.argtypes = [P, C.POINTER(S), C.POINTER(S), C.POINTER(S)]
    lib.wq8_direct_weights_prepare.argtypes = [P, P, P, P, P]
    lib.wq8_direct_quantize_x.argtypes = [P, P, P, P, P]
    lib.wq8_direct_conv.argtypes = [P, P, P, P, P, P, P]
    lib.wq8_direct_forward.argtypes = [P, P, P, P, P, P, S, P]
    lib.wq8_status_string.argtypes = [i]
    lib.wq8_status_string.restype = C.c_char_p
    lib.wq8_last_error.argtypes = []
    lib.wq8_last_error.restype = C.c_char_p
    for name in EXPORTS:
        if name not in ("wq8_plan_destroy", "wq8_status_string", "wq8_last_error"):
            getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        lib = load()
        raise Wq8Error(st, f"{lib.wq8_status_string(st).decode()}: {lib.wq8_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("device buffers must be torch tensors")
    if not t.is_contiguous():
        raise ValueError("device buffers must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


class Plan:
    """Owns a wq8_plan handle and the geometry needed to size buffers."""

    def __init__(self, m, N, Cin, Cout, H, W, pad=1, group=64, points=None, s_B=None, s_G=None,
                 x_dtype=torch.float32, y_dtype=None, algo="auto", y_group="tile",
                 in_quant="fp32"):
        lib = load()
        n = m + 2
        self.m, self.n, self.N, self.Cin, self.Cout, self.H, self.W = m, n, N, Cin, Cout, H, W
        self.pad, self.group, self.algo, self.y_group = pad, group, algo, y_group
        self.in_quant = in_quant
        self.x_dtype = x_dtype
        self.y_dtype = x_dtype if y_dtype is None else y_dtype
        self.Ho, self.Wo = H + 2 * pad - 2, W + 2 * pad - 2
        keep = []

        def arr(v, ct, npdt):
            if v is None:
                return None
            a = np.ascontiguousarray(np.asarray(v, dtype=npdt))
            if a.shape != (n,):
                raise ValueError(f"expected {n} values, got shape {a.shape}")
            keep.append(a)
            return a.ctypes.data_as(C.POINTER(ct))

        d = wq8_desc(m, arr(points, C.c_double, np.float64), arr(s_B, C.c_float, np.float32),
                     arr(s_G, C.c_float, np.float32), group, N, Cin, Cout, H, W, pad,
                     _DT[self.x_dtype], _DT[self.y_dtype], ALGOS[algo], YGROUPS[y_group],
                     IN_QUANTS[in_quant])
        h = C.c_void_p()
        self._h = None
        _check(wq8_plan_create(d, h))
        self._h = h
        ws, uc, us, t, al = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_int64(), C.c_int()
        _check(lib.wq8_plan_query(h, C.byref(ws), C.byref(uc), C.byref(us), C.byref(t),
                                  C.byref(al)))
        self.workspace_bytes, self.u_code_bytes, self.u_scale_bytes = ws.value, uc.value, us.value
        self.T = t.value
        self.ng = Cin // group
        self.fused = al.value == ALGOS["fused"]
        dws, dwc, dws_ = C.c_size_t(), C.c_size_t(), C.c_size_t()
        _check(lib.wq8_direct_query(h, C.byref(dws), C.byref(dwc), C.byref(dws_)))
        self.direct_workspace_bytes, self.direct_w_code_bytes = dws.value, dwc.value
        self.direct_w_scale_bytes = dws_.value

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.wq8_plan_destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def direct_ops(self) -> int:
        return 2 * self.N * self.Cin * self.Cout * self.Ho * self.Wo * 9

    # ---- buffers (torch is the allocator) ----
    def empty_weights(self, device="cuda"):
        n2 = self.n * self.n
        return (torch.empty((n2, self.Cout, self.Cin), dtype=torch.int8, device=device),
                torch.empty((n2, self.Cout, self.ng), dtype=torch.float32, device=device))

    def empty_workspace(self, device="cuda"):
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def empty_output(self, device="cuda"):
        return torch.empty((self.N, self.Cout, self.Ho, self.Wo), dtype=self.y_dtype, device=device)


def wq8_plan_create(desc: wq8_desc, out: C.c_void_p) -> int:
    return load().wq8_plan_create(C.byref(desc), C.byref(out))


def wq8_plan_matrices(plan: Plan):
    n, m = plan.n, plan.m
    Bt = np.zeros((n, n), np.float32)
    Gm = np.zeros((n, 3), np.float32)
    At = np.zeros((m, n), np.float32)
    _check(load().wq8_plan_matrices(plan.handle, Bt.ctypes.data_as(C.c_void_p),
                                    Gm.ctypes.data_as(C.c_void_p), At.ctypes.data_as(C.c_void_p)))
    return Bt, Gm, At


def wq8_plan_bt_codes(plan: Plan):
    """Bq [n][n] int8 and row scales sq [n] of an integer-input-stage plan."""
    n = plan.n
    Bq = np.zeros((n, n), np.int8)
    sq = np.zeros(n, np.float32)
    _check(load().wq8_plan_bt_codes(plan.handle, Bq.ctypes.data_as(C.c_void_p),
                                    sq.ctypes.data_as(C.c_void_p)))
    return Bq, sq


def wq8_weights_prepare(plan: Plan, w, Uq=None, sU=None, stream=None):
    if w.dtype != torch.float32 or tuple(w.shape) != (plan.Cout, plan.Cin, 3, 3):
        raise ValueError("w must be float32 [Cout][Cin][3][3]")
    if Uq is None:
        Uq, sU = plan.empty_weights(w.device)
    _check(load().wq8_weights_prepare(plan.handle, _ptr(w), _ptr(Uq), _ptr(sU), _stream(stream)))
    return Uq, sU


def _check_x(plan, x):
    if x.dtype != plan.x_dtype or tuple(x.shape) != (plan.N, plan.Cin, plan.H, plan.W):
        raise ValueError(f"x must be {plan.x_dtype} {(plan.N, plan.Cin, plan.H, plan.W)}")


def wq8_conv_forward(plan: Plan, x, Uq, sU, y=None, workspace=None, stream=None):
    _check_x(plan, x)
    if y is None:
        y = plan.empty_output(x.device)
    if workspace is None:
        workspace = plan.empty_workspace(x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().wq8_conv_forward(plan.handle, _ptr(x), _ptr(Uq), _ptr(sU), _ptr(y),
                                   _ptr(workspace), nbytes, _stream(stream)))
    return y


def wq8_stage1(plan: Plan, x, Vq=None, sV=None, stream=None):
    _check_x(plan, x)
    n2 = plan.n * plan.n
    if Vq is None:
        Vq = torch.empty((n2, plan.T, plan.Cin), dtype=torch.int8, device=x.device)
        sV = torch.empty((n2, plan.T, plan.ng), dtype=torch.float32, device=x.device)
    _check(load().wq8_stage1(plan.handle, _ptr(x), _ptr(Vq), _ptr(sV), _stream(stream)))
    return Vq, sV


def wq8_stage2(plan: Plan, Vq, sV, Uq, sU, M=None, stream=None):
    if M is None:
        M = torch.empty((plan.n * plan.n, plan.T, plan.Cout), dtype=torch.float32, device=Vq.device)
    _check(load().wq8_stage2(plan.handle, _ptr(Vq), _ptr(sV), _ptr(Uq), _ptr(sU), _ptr(M),
                             _stream(stream)))
    return M


def wq8_stage2_i32(plan: Plan, Vq, Uq, P=None, stream=None):
    if P is None:
        P = torch.empty((plan.n * plan.n, plan.ng, plan.T, plan.Cout), dtype=torch.int32,
                        device=Vq.device)
    _check(load().wq8_stage2_i32(plan.handle, _ptr(Vq), _ptr(Uq), _ptr(P), _stream(stream)))
    return P


def wq8_stage3(plan: Plan, M, y=None, Yq=None, sY=None, want_codes=False, stream=None):
    if y is None:
        y = plan.empty_output(M.device)
    if want_codes and Yq is None:
        Yq = torch.empty((plan.T, plan.Cout, plan.n * plan.n), dtype=torch.int8, device=M.device)
        sshape = (plan.T, plan.Cout, plan.n) if plan.y_group == "row" else (plan.T, plan.Cout)
        sY = torch.empty(sshape, dtype=torch.float32, device=M.device)
    _check(load().wq8_stage3(plan.handle, _ptr(M), _ptr(y), _ptr(Yq), _ptr(sY), _stream(stream)))
    return (y, Yq, sY) if want_codes else y


def wq8_stage23(plan: Plan, Vq, sV, Uq, sU, y=None, stream=None):
    if y is None:
        y = plan.empty_output(Vq.device)
    _check(load().wq8_stage23(plan.handle, _ptr(Vq), _ptr(sV), _ptr(Uq), _ptr(sU), _ptr(y),
                              _stream(stream)))
    return y


def tiles(m, N, H, W, pad):
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    return N * math.ceil(Ho / m) * math.ceil(Wo / m)


# ---- group-wise W8A8 direct convolution (the non-Winograd baseline)
def wq8_direct_weights_prepare(plan: Plan, w, Wq=None, sW=None, stream=None):
    if w.dtype != torch.float32 or tuple(w.shape) != (plan.Cout, plan.Cin, 3, 3):
        raise ValueError("w must be float32 [Cout][Cin][3][3]")
    if Wq is None:
        Wq = torch.empty((9, plan.Cout, plan.Cin), dtype=torch.int8, device=w.device)
        sW = torch.empty((9, plan.Cout, plan.ng), dtype=torch.float32, device=w.device)
    _check(load().wq8_direct_weights_prepare(plan.handle, _ptr(w), _ptr(Wq), _ptr(sW), _stream(stream)))
    return Wq, sW


def wq8_direct_quantize_x(plan: Plan, x, Xq=None, sX=None, stream=None):
    _check_x(plan, x)
    if Xq is None:
        Xq = torch.empty((plan.N, plan.H, plan.W, plan.Cin), dtype=torch.int8, device=x.device)
        sX = torch.empty((plan.N, plan.H, plan.W, plan.ng), dtype=torch.float32, device=x.device)
    _check(load().wq8_direct_quantize_x(plan.handle, _ptr(x), _ptr(Xq), _ptr(sX), _stream(stream)))
    return Xq, sX


def wq8_direct_conv(plan: Plan, Xq, sX, Wq, sW, y=None, stream=None):
    if y is None:
        y = plan.empty_output(Xq.device)
    _check(load().wq8_direct_conv(plan.handle, _ptr(Xq), _ptr(sX), _ptr(Wq), _ptr(sW), _ptr(y),
                                  _stream(stream)))
    return y


def wq8_direct_forward(plan: Plan, x, Wq, sW, y=None, workspace=None, stream=None):
    _check_x(plan, x)
    if y is None:
        y = plan.empty_output(x.device)
    if workspace is None:
        workspace = torch.empty(plan.direct_workspace_bytes, dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().wq8_direct_forward(plan.handle, _ptr(x), _ptr(Wq), _ptr(sW), _ptr(y),
                                     _ptr(workspace), nbytes, _stream(stream)))
    return y
