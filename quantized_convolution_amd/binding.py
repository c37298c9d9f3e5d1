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
                ("in_quant", C.c_int), ("stage1_rows", C.c_int), ("fused_waves", C.c_int),
                ("fused_block", C.c_int), ("stage2_rows", C.c_int), ("stage2_cols", C.c_int),
                ("stage2_waves", C.c_int), ("stage3_lanes", C.c_int)]


EXPORTS = ("wq8_plan_create", "wq8_plan_destroy", "wq8_plan_query", "wq8_plan_matrices",
           "wq8_plan_bt_codes",
           "wq8_weights_prepare", "wq8_conv_forward", "wq8_stage1", "wq8_stage2",
           "wq8_stage2_i32", "wq8_stage3", "wq8_stage23", "wq8_direct_query",
           "wq8_direct_weights_prepare", "wq8_direct_quantize_x", "wq8_direct_conv",
           "wq8_direct_forward", "wq8_conv_forward_noalloc", "wq8_status_string", "wq8_last_error")

# bytes of the device array wq8_conv_forward_noalloc uses as its workspace
NOALLOC_MAX_WORKSPACE = 64 << 20

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
    lib.wq8_conv_forward_noalloc.argtypes = [P, P, P, P, P, P]
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
    return C.c_void_p(t.data_ptr())


class _Bufs:
    """Checks every buffer of one call before anything reaches the library:
    a torch tensor of the expected dtype and shape (or, for a workspace, at
    least the expected bytes), contiguous, and (checked last, for all of them
    together) on a GPU, all on one device. The kernels size their accesses
    from the plan, so a buffer that fails any of these would be read or
    written out of bounds; ValueError instead."""

    def __init__(self):
        self.device = None
        self.bufs = []

    def __call__(self, t, name, dtype, shape=None, min_bytes=None):
        if t is None:
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {min_bytes}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.bufs.append((name, t))
        return t

    def call(self, fn, *args, stream=None):
        """Check the devices, then run the C call with the buffers' device
        current, on `stream` or that device's current stream."""
        for name, t in self.bufs:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on a GPU, got {t.device}")
            if self.device is None:
                self.device = t.device
            elif t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, other buffers on {self.device}")
        with torch.cuda.device(self.device):
            st = torch.cuda.current_stream(self.device) if stream is None else stream
            _check(fn(*args, C.c_void_p(st.cuda_stream)))


class Plan:
    """Owns a wq8_plan handle and the geometry needed to size buffers."""

    def __init__(self, m, N, Cin, Cout, H, W, pad=1, group=64, points=None, s_B=None, s_G=None,
                 x_dtype=torch.float32, y_dtype=None, algo="auto", y_group="tile",
                 in_quant="fp32", stage1_rows=0, fused_waves=0, fused_block=0, stage2_rows=0,
                 stage2_cols=0, stage2_waves=0, stage3_lanes=0):
        """Kernel shapes (0 = the library chooses; results never depend on
        them): stage1_rows 1 all / 2 half the input rows in the LDS window;
        fused_waves 4, 8 or 16; fused_block 1 16x16, 2 32x32, 3 32 tiles x 16
        channels, 4 16 x 32; stage2_rows 4, 5, 6 or 8 (tiles per staged
        Hadamard block / 16); stage2_cols 1 or 2 (channels per wave / 16);
        stage2_waves 2 or 4; stage3_lanes 1 or 2 (lanes per (tile, channel) pair
        of the staged output transform)."""
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
                     IN_QUANTS[in_quant], int(stage1_rows), int(fused_waves), int(fused_block),
                     int(stage2_rows), int(stage2_cols), int(stage2_waves), int(stage3_lanes))
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

    # ---- buffer shapes the kernels assume ----
    @property
    def x_shape(self):
        return (self.N, self.Cin, self.H, self.W)

    @property
    def y_shape(self):
        return (self.N, self.Cout, self.Ho, self.Wo)

    @property
    def uq_shape(self):
        return (self.n * self.n, self.Cout, self.Cin)

    @property
    def su_shape(self):
        return (self.n * self.n, self.Cout, self.ng)

    @property
    def vq_shape(self):
        return (self.n * self.n, self.T, self.Cin)

    @property
    def sv_shape(self):
        return (self.n * self.n, self.T, self.ng)

    @property
    def m_shape(self):
        return (self.n * self.n, self.T, self.Cout)

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
    b = _Bufs()
    b(w, "w", torch.float32, (plan.Cout, plan.Cin, 3, 3))
    if Uq is None:
        Uq, sU = plan.empty_weights(w.device)
    b(Uq, "Uq", torch.int8, plan.uq_shape)
    b(sU, "sU", torch.float32, plan.su_shape)
    b.call(load().wq8_weights_prepare, plan.handle, _ptr(w), _ptr(Uq), _ptr(sU), stream=stream)
    return Uq, sU


def _check_x(plan, b, x):
    b(x, "x", plan.x_dtype, plan.x_shape)


def _check_weights(plan, b, Uq, sU):
    b(Uq, "Uq", torch.int8, plan.uq_shape)
    b(sU, "sU", torch.float32, plan.su_shape)


def _check_codes(plan, b, Vq, sV):
    b(Vq, "Vq", torch.int8, plan.vq_shape)
    b(sV, "sV", torch.float32, plan.sv_shape)


def wq8_conv_forward(plan: Plan, x, Uq, sU, y=None, workspace=None, stream=None):
    b = _Bufs()
    _check_x(plan, b, x)
    _check_weights(plan, b, Uq, sU)
    if y is None:
        y = plan.empty_output(x.device)
    if workspace is None:
        workspace = plan.empty_workspace(x.device)
    b(y, "y", plan.y_dtype, plan.y_shape)
    b(workspace, "workspace", None, min_bytes=plan.workspace_bytes)
    if y.data_ptr() == x.data_ptr():
        raise ValueError("x and y must not overlap")
    nbytes = workspace.numel() * workspace.element_size()
    b.call(load().wq8_conv_forward, plan.handle, _ptr(x), _ptr(Uq), _ptr(sU), _ptr(y),
           _ptr(workspace), C.c_size_t(nbytes), stream=stream)
    return y


def wq8_conv_forward_noalloc(plan: Plan, x, Uq, sU, y, stream=None):
    """The forward on the library's built-in workspace (no device allocation
    by the library; y is the caller's). Calls that overlap on one GPU race."""
    b = _Bufs()
    _check_x(plan, b, x)
    _check_weights(plan, b, Uq, sU)
    b(y, "y", plan.y_dtype, plan.y_shape)
    if y.data_ptr() == x.data_ptr():
        raise ValueError("x and y must not overlap")
    b.call(load().wq8_conv_forward_noalloc, plan.handle, _ptr(x), _ptr(Uq), _ptr(sU), _ptr(y),
           stream=stream)
    return y


def wq8_stage1(plan: Plan, x, Vq=None, sV=None, stream=None):
    b = _Bufs()
    _check_x(plan, b, x)
    if Vq is None:
        Vq = torch.empty(plan.vq_shape, dtype=torch.int8, device=x.device)
        sV = torch.empty(plan.sv_shape, dtype=torch.float32, device=x.device)
    _check_codes(plan, b, Vq, sV)
    b.call(load().wq8_stage1, plan.handle, _ptr(x), _ptr(Vq), _ptr(sV), stream=stream)
    return Vq, sV


def wq8_stage2(plan: Plan, Vq, sV, Uq, sU, M=None, stream=None):
    b = _Bufs()
    _check_codes(plan, b, Vq, sV)
    _check_weights(plan, b, Uq, sU)
    if M is None:
        M = torch.empty(plan.m_shape, dtype=torch.float32, device=Vq.device)
    b(M, "M", torch.float32, plan.m_shape)
    b.call(load().wq8_stage2, plan.handle, _ptr(Vq), _ptr(sV), _ptr(Uq), _ptr(sU), _ptr(M),
           stream=stream)
    return M


def wq8_stage2_i32(plan: Plan, Vq, Uq, P=None, stream=None):
    b = _Bufs()
    b(Vq, "Vq", torch.int8, plan.vq_shape)
    b(Uq, "Uq", torch.int8, plan.uq_shape)
    pshape = (plan.n * plan.n, plan.ng, plan.T, plan.Cout)
    if P is None:
        P = torch.empty(pshape, dtype=torch.int32, device=Vq.device)
    b(P, "P", torch.int32, pshape)
    b.call(load().wq8_stage2_i32, plan.handle, _ptr(Vq), _ptr(Uq), _ptr(P), stream=stream)
    return P


def wq8_stage3(plan: Plan, M, y=None, Yq=None, sY=None, want_codes=False, stream=None):
    b = _Bufs()
    b(M, "M", torch.float32, plan.m_shape)
    if y is None:
        y = plan.empty_output(M.device)
    b(y, "y", plan.y_dtype, plan.y_shape)
    sshape = (plan.T, plan.Cout, plan.n) if plan.y_group == "row" else (plan.T, plan.Cout)
    yqshape = (plan.T, plan.Cout, plan.n * plan.n)
    if want_codes and Yq is None:
        Yq = torch.empty(yqshape, dtype=torch.int8, device=M.device)
        sY = torch.empty(sshape, dtype=torch.float32, device=M.device)
    if Yq is not None:
        b(Yq, "Yq", torch.int8, yqshape)
    if sY is not None:
        b(sY, "sY", torch.float32, sshape)
    b.call(load().wq8_stage3, plan.handle, _ptr(M), _ptr(y), _ptr(Yq), _ptr(sY), stream=stream)
    return (y, Yq, sY) if want_codes else y


def wq8_stage23(plan: Plan, Vq, sV, Uq, sU, y=None, stream=None):
    b = _Bufs()
    _check_codes(plan, b, Vq, sV)
    _check_weights(plan, b, Uq, sU)
    if y is None:
        y = plan.empty_output(Vq.device)
    b(y, "y", plan.y_dtype, plan.y_shape)
    b.call(load().wq8_stage23, plan.handle, _ptr(Vq), _ptr(sV), _ptr(Uq), _ptr(sU), _ptr(y),
           stream=stream)
    return y


def tiles(m, N, H, W, pad):
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    return N * math.ceil(Ho / m) * math.ceil(Wo / m)


# ---- group-wise W8A8 direct convolution (the non-Winograd baseline)
def _direct_shapes(plan):
    return ((9, plan.Cout, plan.Cin), (9, plan.Cout, plan.ng),
            (plan.N, plan.H, plan.W, plan.Cin), (plan.N, plan.H, plan.W, plan.ng))


def wq8_direct_weights_prepare(plan: Plan, w, Wq=None, sW=None, stream=None):
    wqs, sws, _, _ = _direct_shapes(plan)
    b = _Bufs()
    b(w, "w", torch.float32, (plan.Cout, plan.Cin, 3, 3))
    if Wq is None:
        Wq = torch.empty(wqs, dtype=torch.int8, device=w.device)
        sW = torch.empty(sws, dtype=torch.float32, device=w.device)
    b(Wq, "Wq", torch.int8, wqs)
    b(sW, "sW", torch.float32, sws)
    b.call(load().wq8_direct_weights_prepare, plan.handle, _ptr(w), _ptr(Wq), _ptr(sW), stream=stream)
    return Wq, sW


def wq8_direct_quantize_x(plan: Plan, x, Xq=None, sX=None, stream=None):
    _, _, xqs, sxs = _direct_shapes(plan)
    b = _Bufs()
    _check_x(plan, b, x)
    if Xq is None:
        Xq = torch.empty(xqs, dtype=torch.int8, device=x.device)
        sX = torch.empty(sxs, dtype=torch.float32, device=x.device)
    b(Xq, "Xq", torch.int8, xqs)
    b(sX, "sX", torch.float32, sxs)
    b.call(load().wq8_direct_quantize_x, plan.handle, _ptr(x), _ptr(Xq), _ptr(sX), stream=stream)
    return Xq, sX


def wq8_direct_conv(plan: Plan, Xq, sX, Wq, sW, y=None, stream=None):
    wqs, sws, xqs, sxs = _direct_shapes(plan)
    b = _Bufs()
    b(Xq, "Xq", torch.int8, xqs)
    b(sX, "sX", torch.float32, sxs)
    b(Wq, "Wq", torch.int8, wqs)
    b(sW, "sW", torch.float32, sws)
    if y is None:
        y = plan.empty_output(Xq.device)
    b(y, "y", plan.y_dtype, plan.y_shape)
    b.call(load().wq8_direct_conv, plan.handle, _ptr(Xq), _ptr(sX), _ptr(Wq), _ptr(sW), _ptr(y),
           stream=stream)
    return y


def wq8_direct_forward(plan: Plan, x, Wq, sW, y=None, workspace=None, stream=None):
    wqs, sws, _, _ = _direct_shapes(plan)
    b = _Bufs()
    _check_x(plan, b, x)
    b(Wq, "Wq", torch.int8, wqs)
    b(sW, "sW", torch.float32, sws)
    if y is None:
        y = plan.empty_output(x.device)
    if workspace is None:
        workspace = torch.empty(plan.direct_workspace_bytes, dtype=torch.uint8, device=x.device)
    b(y, "y", plan.y_dtype, plan.y_shape)
    b(workspace, "workspace", None, min_bytes=plan.direct_workspace_bytes)
    if y.data_ptr() == x.data_ptr():
        raise ValueError("x and y must not overlap")
    nbytes = workspace.numel() * workspace.element_size()
    b.call(load().wq8_direct_forward, plan.handle, _ptr(x), _ptr(Wq), _ptr(sW), _ptr(y),
           _ptr(workspace), C.c_size_t(nbytes), stream=stream)
    return y
