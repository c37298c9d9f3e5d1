"""CPU oracle for group-wise fully quantized 8-bit Winograd convolution F(m,3).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
reference. It shares no code with the HIP library (quantized_convolution_amd)
and must never be imported by it: only tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py use it.

Method: "Data-Free Group-Wise Fully Quantized Winograd Convolution via
Learnable Scales" (arXiv 2412.19867): Winograd F(m,3) with transforms
B^T = S_B V^-T, G = S_G V, A^T = V^T S_A (S_A S_B S_G = I), and group-wise
int8 quantization at the input transform, the Hadamard product and the output
transform.

Functions return numpy arrays in these layouts (n = m + 2, T tiles,
tile t = (img*tH + ty)*tW + tx):
  Uq [n*n][Cout][Cin] int8, sU [n*n][Cout][Cin/G]
  Vq [n*n][T][Cin]    int8, sV [n*n][T][Cin/G]
  P  [n*n][Cin/G][T][Cout] int32
  M  [n*n][T][Cout]
  Yq [T][Cout][n*n]   int8, sY [T][Cout]
  y  [N][Cout][Ho][Wo]

Parity pins: every function here is checked in tests/test_oracle_*.py against
closed forms, textbook matrices, exact rational arithmetic, brute force or an
error bound (see each test's docstring). Absolute SQNR values are
parity-unpinned: the pages print none.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import transforms
from .build import ensure_built

_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(ensure_built())
        P = C.c_void_p
        i, l = C.c_int, C.c_long
        _lib.wq8o_num_threads.restype = C.c_int
        _lib.wq8o_set_num_threads.argtypes = [C.c_int]
        _lib.wq8o_set_num_threads.restype = None
        _lib.wq8o_direct_conv_f64.argtypes = [i, i, i, i, i, i, P, P, P]
        _lib.wq8o_winograd_f64.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P]
        _lib.wq8o_stage2_i32.argtypes = [i, l, i, i, i, P, P, P]
        for s in ("_f32", "_f64"):
            getattr(_lib, "wq8o_weights" + s).argtypes = [i, i, i, i, P, P, P, P]
            getattr(_lib, "wq8o_stage1" + s).argtypes = [i, i, i, i, i, i, i, P, P, P, P]
            getattr(_lib, "wq8o_quant_bt" + s).argtypes = [i, i, P, P, P]
            getattr(_lib, "wq8o_stage1_int" + s).argtypes = [i, i, i, i, i, i, i, P, P, P, P, P,
                                                             P, P]
            getattr(_lib, "wq8o_stage2" + s).argtypes = [i, l, i, i, i, P, P, P, P, P]
            getattr(_lib, "wq8o_stage3" + s).argtypes = [i, i, i, i, i, i, P, P, P, P, P]
            getattr(_lib, "wq8o_stage3_rows" + s).argtypes = [i, i, i, i, i, i, P, P, P, P, P]
            getattr(_lib, "wq8o_sampled" + s).argtypes = [i, l, i, i, i, P, P, P, P, P, i, P, P, P,
                                                           P, P]
            getattr(_lib, "wq8o_w8a8_quant_x" + s).argtypes = [i, i, i, i, i, P, P, P]
            getattr(_lib, "wq8o_w8a8_quant_w" + s).argtypes = [i, i, i, P, P, P]
            getattr(_lib, "wq8o_w8a8_conv" + s).argtypes = [i, i, i, i, i, i, i, P, P, P, P, P]
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def num_threads() -> int:
    return lib().wq8o_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for later calls (timing only: results are independent of it)."""
    lib().wq8o_set_num_threads(int(n))


def out_size(H, W, pad):
    return H + 2 * pad - 2, W + 2 * pad - 2


def tiles(m, N, H, W, pad):
    Ho, Wo = out_size(H, W, pad)
    tH, tW = -(-Ho // m), -(-Wo // m)
    return tH, tW, N * tH * tW


# --------------------------------------------------------------------------
# bf16 helpers (activations in/out may be bfloat16)
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# exact references
# --------------------------------------------------------------------------
def direct_conv_f64(x, w, pad):
    x, w = _f32(x), _f32(w)
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    assert w.shape == (Cout, Cin, 3, 3)
    Ho, Wo = out_size(H, W, pad)
    y = np.zeros((N, Cout, Ho, Wo), np.float64)
    lib().wq8o_direct_conv_f64(N, Cin, Cout, H, W, pad, _p(x), _p(w), _p(y))
    return y


def winograd_f64(m, x, w, pad, Bt, Gm, At):
    x, w = _f32(x), _f32(w)
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    Bt, Gm, At = (np.ascontiguousarray(a, np.float64) for a in (Bt, Gm, At))
    Ho, Wo = out_size(H, W, pad)
    y = np.zeros((N, Cout, Ho, Wo), np.float64)
    lib().wq8o_winograd_f64(m, N, Cin, Cout, H, W, pad, _p(Bt), _p(Gm), _p(At),
                            _p(x), _p(w), _p(y))
    return y


# --------------------------------------------------------------------------
# the fixed-order quantized pipeline
# --------------------------------------------------------------------------
def _real(prec):
    return {"f32": np.float32, "f64": np.float64}[prec]


def weights(m, w, G, Gm, prec="f32"):
    w = _f32(w)
    Cout, Cin = w.shape[:2]
    n2 = (m + 2) ** 2
    R = _real(prec)
    Gm = np.ascontiguousarray(Gm, R)
    Uq = np.zeros((n2, Cout, Cin), np.int8)
    sU = np.zeros((n2, Cout, Cin // G), R)
    getattr(lib(), "wq8o_weights_" + prec)(m, Cin, Cout, G, _p(Gm), _p(w), _p(Uq), _p(sU))
    return Uq, sU


def stage1(m, x, pad, G, Bt, prec="f32"):
    x = _f32(x)
    N, Cin, H, W = x.shape
    _, _, T = tiles(m, N, H, W, pad)
    n2 = (m + 2) ** 2
    R = _real(prec)
    Bt = np.ascontiguousarray(Bt, R)
    Vq = np.zeros((n2, T, Cin), np.int8)
    sV = np.zeros((n2, T, Cin // G), R)
    getattr(lib(), "wq8o_stage1_" + prec)(m, N, Cin, H, W, pad, G, _p(Bt), _p(x), _p(Vq), _p(sV))
    return Vq, sV


IN_QUANT = ("fp32", "int_tensor", "int_row")


def quant_bt(Bt, rows, prec="f32"):
    """B^T quantized for the literal input stage: Bq [n][n] int8 and sB [n]
    (one scale per row when rows, else one for the matrix, repeated)."""
    R = _real(prec)
    Bt = np.ascontiguousarray(Bt, R)
    n = Bt.shape[0]
    Bq = np.zeros((n, n), np.int8)
    sB = np.zeros(n, R)
    getattr(lib(), "wq8o_quant_bt_" + prec)(n, int(bool(rows)), _p(Bt), _p(Bq), _p(sB))
    return Bq, sB


def stage1_int(m, x, pad, G, Bq, sB, prec="f32", keep=False):
    """Literal input stage: patch codes per (tile, group) and an integer
    transform with Bq; returns Vq, sV (and xq [T][Cin][n][n], sx [T][Cin/G]
    when keep)."""
    x = _f32(x)
    N, Cin, H, W = x.shape
    _, _, T = tiles(m, N, H, W, pad)
    n = m + 2
    R = _real(prec)
    Bq = np.ascontiguousarray(Bq, np.int8)
    sB = np.ascontiguousarray(sB, R)
    Vq = np.zeros((n * n, T, Cin), np.int8)
    sV = np.zeros((n * n, T, Cin // G), R)
    xq = np.zeros((T, Cin, n, n), np.int8)
    sx = np.zeros((T, Cin // G), R)
    getattr(lib(), "wq8o_stage1_int_" + prec)(m, N, Cin, H, W, pad, G, _p(Bq), _p(sB), _p(x),
                                               _p(Vq), _p(sV), _p(xq), _p(sx))
    if keep:
        return Vq, sV, xq, sx
    return Vq, sV


def stage2(Vq, sV, Uq, sU, G, prec="f32"):
    n2, T, Cin = Vq.shape
    Cout = Uq.shape[1]
    R = _real(prec)
    sV, sU = np.ascontiguousarray(sV, R), np.ascontiguousarray(sU, R)
    M = np.zeros((n2, T, Cout), R)
    getattr(lib(), "wq8o_stage2_" + prec)(n2, T, Cin, Cout, G, _p(np.ascontiguousarray(Vq)),
                                          _p(sV), _p(np.ascontiguousarray(Uq)), _p(sU), _p(M))
    return M


def stage2_i32(Vq, Uq, G):
    n2, T, Cin = Vq.shape
    Cout = Uq.shape[1]
    P = np.zeros((n2, Cin // G, T, Cout), np.int32)
    lib().wq8o_stage2_i32(n2, T, Cin, Cout, G, _p(np.ascontiguousarray(Vq)),
                          _p(np.ascontiguousarray(Uq)), _p(P))
    return P


def stage3(m, M, N, H, W, pad, At, prec="f32", y_group="tile"):
    """Y requantization + output transform. y_group "tile": one scale per
    (tile, co) over all taps, sY [T][Cout]; "row": one per row of taps,
    sY [T][Cout][n]."""
    n2, T, Cout = M.shape
    R = _real(prec)
    M = np.ascontiguousarray(M, R)
    At = np.ascontiguousarray(At, R)
    Ho, Wo = out_size(H, W, pad)
    y = np.zeros((N, Cout, Ho, Wo), R)
    Yq = np.zeros((T, Cout, n2), np.int8)
    if y_group == "tile":
        sY = np.zeros((T, Cout), R)
        fn = "wq8o_stage3_"
    elif y_group == "row":
        sY = np.zeros((T, Cout, m + 2), R)
        fn = "wq8o_stage3_rows_"
    else:
        raise ValueError(y_group)
    getattr(lib(), fn + prec)(m, N, Cout, H, W, pad, _p(At), _p(M), _p(y), _p(Yq), _p(sY))
    return y, Yq, sY


def sampled(m, Vq, sV, Uq, sU, At, pairs, prec="f32"):
    """Stages 2 and 3 at chosen (tile, co) pairs only: returns M [S][n*n],
    Yq [S][n*n], sY [S] and the uncropped output tiles [S][m][m]."""
    n2, T_, Cin = Vq.shape
    Cout = Uq.shape[1]
    G = Cin // sV.shape[2]
    R = _real(prec)
    pairs = np.ascontiguousarray(pairs, np.int64).reshape(-1, 2)
    S = pairs.shape[0]
    Ms = np.zeros((S, n2), R)
    Yq = np.zeros((S, n2), np.int8)
    sY = np.zeros(S, R)
    ys = np.zeros((S, m, m), R)
    sV, sU, At = (np.ascontiguousarray(a, R) for a in (sV, sU, At))
    getattr(lib(), "wq8o_sampled_" + prec)(m, T_, Cin, Cout, G, _p(np.ascontiguousarray(Vq)), _p(sV),
                                           _p(np.ascontiguousarray(Uq)), _p(sU), _p(At), S,
                                           _p(pairs), _p(Ms), _p(Yq), _p(sY), _p(ys))
    return Ms, Yq, sY, ys


def forward(m, x, w, pad, G, points=None, s_b=None, s_g=None, prec="f32", keep=False,
            y_group="tile", in_quant="fp32"):
    """Whole quantized pipeline. Returns y, or a dict of every stage if keep.
    in_quant "fp32": fp32 input transform; "int_tensor" / "int_row": the
    literal input stage with B^T quantized per matrix / per row."""
    n = m + 2
    points = transforms.standard_points(m) if points is None else points
    s_b = np.ones(n, np.float32) if s_b is None else s_b
    s_g = np.ones(n, np.float32) if s_g is None else s_g
    mk = transforms.transforms_f32 if prec == "f32" else transforms.transforms_f64
    Bt, Gm, At = mk(m, points, s_b, s_g)
    N, _, H, W = x.shape
    Uq, sU = weights(m, w, G, Gm, prec)
    if in_quant == "fp32":
        Vq, sV = stage1(m, x, pad, G, Bt, prec)
    elif in_quant in IN_QUANT:
        Bq, sB = quant_bt(Bt, in_quant == "int_row", prec)
        Vq, sV = stage1_int(m, x, pad, G, Bq, sB, prec)
    else:
        raise ValueError(in_quant)
    M = stage2(Vq, sV, Uq, sU, G, prec)
    y, Yq, sY = stage3(m, M, N, H, W, pad, At, prec, y_group)
    if not keep:
        return y
    return dict(Bt=Bt, G=Gm, At=At, Uq=Uq, sU=sU, Vq=Vq, sV=sV, M=M, Yq=Yq, sY=sY, y=y)


def sqnr_db(ref, out) -> float:
    """10 log10(sum ref^2 / sum (ref - out)^2) over the whole tensor (the SQNR
    the pages optimise per layer; their Eq. 17 is not printed, so this is the
    plain definition)."""
    ref = np.asarray(ref, np.float64)
    err = ref - np.asarray(out, np.float64)
    num, den = float(np.sum(ref * ref)), float(np.sum(err * err))
    if den == 0.0:
        return float("inf")
    return 10.0 * np.log10(num / den)


# --------------------------------------------------------------------------
# group-wise W8A8 direct convolution (the non-Winograd baseline)
# --------------------------------------------------------------------------
def direct_quant_x(x, G, prec="f32"):
    """xq [N][H][W][Cin] int8 and sx [N][H][W][Cin/G]: per pixel, groups of G
    consecutive input channels."""
    x = _f32(x)
    N, Cin, H, W = x.shape
    assert Cin % G == 0 and G <= 256
    rt = np.float32 if prec == "f32" else np.float64
    xq = np.zeros((N, H, W, Cin), np.int8)
    sx = np.zeros((N, H, W, Cin // G), rt)
    getattr(lib(), "wq8o_w8a8_quant_x_" + prec)(N, Cin, H, W, G, _p(x), _p(xq), _p(sx))
    return xq, sx


def direct_quant_w(w, G, prec="f32"):
    """wq [9][Cout][Cin] int8 and sw [9][Cout][Cin/G]: per kernel tap and
    output channel, groups of G consecutive input channels."""
    w = _f32(w)
    Cout, Cin = w.shape[:2]
    assert w.shape == (Cout, Cin, 3, 3) and Cin % G == 0 and G <= 256
    rt = np.float32 if prec == "f32" else np.float64
    wq = np.zeros((9, Cout, Cin), np.int8)
    sw = np.zeros((9, Cout, Cin // G), rt)
    getattr(lib(), "wq8o_w8a8_quant_w_" + prec)(Cin, Cout, G, _p(w), _p(wq), _p(sw))
    return wq, sw


def direct_w8a8(x, w, pad, G, prec="f32", keep=False):
    """Group-wise W8A8 direct 3x3 convolution: y [N][Cout][Ho][Wo]."""
    x = _f32(x)
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    xq, sx = direct_quant_x(x, G, prec)
    wq, sw = direct_quant_w(w, G, prec)
    Ho, Wo = out_size(H, W, pad)
    rt = np.float32 if prec == "f32" else np.float64
    y = np.zeros((N, Cout, Ho, Wo), rt)
    getattr(lib(), "wq8o_w8a8_conv_" + prec)(N, Cin, Cout, H, W, pad, G, _p(xq), _p(sx), _p(wq),
                                                _p(sw), _p(y))
    if keep:
        return dict(xq=xq, sx=sx, wq=wq, sw=sw, y=y)
    return y
