"""CPU oracle for the fine-grained quantized linear layer (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package. It shares nothing with the HIP path: the C code in
``oracle.c`` is compiled here with gcc, and these wrappers only marshal numpy
arrays. See the header of ``oracle.c`` for the passages each function follows.

Functions with no pin against the pages beyond invariants are marked in their
docstrings; every other function is pinned by the ``-m "not gpu"`` tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.orc_quant_sym_i8.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_quant_asym_u8.argtypes = [P, I64, I64, I64, P, P, P, P]
        lib.orc_group_quant_int4.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_group_quant_int8.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_layout_int8.argtypes = [P, I64, I64, P]
        lib.orc_unlayout_int8.argtypes = [P, I64, I64, P]
        lib.orc_amplifier_log2.argtypes = [P, I64, I]
        lib.orc_amplifier_log2.restype = I
        lib.orc_integer_scales.argtypes = [P, I64, I, P]
        lib.orc_f32_to_bf16.argtypes = [P, I64, P]
        lib.orc_narrow_iscale.argtypes = [P, I64, I, P]
        lib.orc_narrow_iscale.restype = I64
        lib.orc_weight_mse_is_fs.argtypes = [P, P, P, I, I64, I64, I64, P, P]
        lib.orc_weight_mse_is_fs.restype = ctypes.c_double
        lib.orc_pack_int4.argtypes = [P, I64, I64, P]
        lib.orc_unpack_int4.argtypes = [P, I64, I64, P]
        lib.orc_pack_int4_canonical.argtypes = [P, I64, I64, P]
        lib.orc_unpack_int4_canonical.argtypes = [P, I64, I64, P]
        lib.orc_w4a8_gemm_is.argtypes = [P, P, P, P, I, I64, I64, I64, I64, P, I64, P, I64, P, P]
        lib.orc_w4a8_gemm_is.restype = I64
        lib.orc_w4a8_gemm_fs.argtypes = [P, P, P, P, I64, I64, I64, I64, P, I64, P, I64, P]
        lib.orc_w8a8_gemm_zp.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, P, I64, P, I64, P, P]
        lib.orc_w8a8_gemm_zp.restype = I64
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ------------------------------------------------------------------ quantizers

def quant_sym_i8(x):
    """Per-token symmetric int8 codes and scales of X (rows x cols float32)."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    _load().orc_quant_sym_i8(_p(x), rows, cols, cols, _p(q), _p(s))
    return q, s


def quant_asym_u8(x):
    """Per-row asymmetric uint8 codes, scales, zero points and code row sums."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(rows, np.float32)
    z = np.empty(rows, np.int32)
    rs = np.empty(rows, np.int32)
    _load().orc_quant_asym_u8(_p(x), rows, cols, cols, _p(q), _p(s), _p(z), _p(rs))
    return q, s, z, rs


def group_quant_int4(w, g: int = 128):
    """Group-wise int4 codes (K x N int8) and float scales ((K/g) x N) of W (K x N)."""
    w = _c(w, np.float32)
    K, N = w.shape
    codes = np.empty((K, N), np.int8)
    fscale = np.empty((K // g, N), np.float32)
    _load().orc_group_quant_int4(_p(w), K, N, g, _p(codes), _p(fscale))
    return codes, fscale


def group_quant_int8(w, g: int = 128):
    """Group-wise int8 codes (K x N int8, [-127, 127]) and float scales ((K/g) x N) of W."""
    w = _c(w, np.float32)
    K, N = w.shape
    codes = np.empty((K, N), np.int8)
    fscale = np.empty((K // g, N), np.float32)
    _load().orc_group_quant_int8(_p(w), K, N, g, _p(codes), _p(fscale))
    return codes, fscale


def layout_int8(codes):
    """K x N int8 codes in the int8 fragment layout (N*K bytes)."""
    codes = _c(codes, np.int8)
    K, N = codes.shape
    out = np.empty(N * K, np.int8)
    _load().orc_layout_int8(_p(codes), K, N, _p(out))
    return out


def unlayout_int8(qw, K: int, N: int):
    qw = _c(qw, np.int8)
    codes = np.empty((K, N), np.int8)
    _load().orc_unlayout_int8(_p(qw), K, N, _p(codes))
    return codes


def pack_weights_int8(w, g: int = 128, alpha: int = 0):
    """Offline path of the fine-grained W8A8 integer-scale layer: codes (K x N),
    their int8 fragment layout qw, float and integer scales, and alpha
    (0 = the amplifier search)."""
    codes, fscale = group_quant_int8(w, g)
    if alpha == 0:
        alpha = 1 << amplifier_log2(fscale)
    return {"codes": codes, "qw": layout_int8(codes), "fscale": fscale,
            "iscale": integer_scales(fscale, alpha), "alpha": alpha}


def amplifier_log2(fscale, max_log2: int = 30) -> int:
    """Exponent n of the searched amplifier alpha = 2^n (-1 if above max_log2)."""
    f = _c(fscale, np.float32).ravel()
    return int(_load().orc_amplifier_log2(_p(f), f.size, max_log2))


def integer_scales(fscale, alpha: int):
    f = _c(fscale, np.float32)
    out = np.empty(f.shape, np.int32)
    _load().orc_integer_scales(_p(f), f.size, int(alpha), _p(out))
    return out


def f32_to_bf16_bits(x):
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_bf16(_p(x), x.size, _p(out))
    return out


def bf16_bits_to_f32(b):
    """float32 values of bfloat16 bit patterns (exact: the low 16 bits are zero)."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def narrow_iscale(iscale, width: int):
    """Integer scales as uint8 (width 1) or uint16 (width 2), same values.

    Returns (array, 0), or (None, number of values that do not fit)."""
    i = _c(iscale, np.int32)
    out = np.empty(i.shape, np.uint8 if width == 1 else np.uint16)
    bad = int(_load().orc_narrow_iscale(_p(i), i.size, int(width), _p(out)))
    if bad < 0:
        raise ValueError("width must be 1 or 2")
    return (out, 0) if bad == 0 else (None, bad)


def weight_mse_is_fs(codes, fscale, iscale, alpha: int, g: int = 128):
    """Weight MSE between integer-scale (q*S/alpha) and float-scale (q*s)
    dequantized weights, the largest integer scale, and how many integer
    scales need more than 8 bits."""
    codes = _c(codes, np.int8)
    f = _c(fscale, np.float32)
    i = _c(iscale, np.int32)
    K, N = codes.shape
    mx = ctypes.c_int32(0)
    wide = ctypes.c_int64(0)
    mse = _load().orc_weight_mse_is_fs(_p(codes), _p(f), _p(i), int(alpha), K, N, g,
                                       ctypes.byref(mx), ctypes.byref(wide))
    return float(mse), int(mx.value), int(wide.value)


def pack_int4(codes):
    """Pack K x N int4 codes into the library's N*K/2-byte layout."""
    codes = _c(codes, np.int8)
    K, N = codes.shape
    out = np.empty(N * K // 2, np.uint8)
    _load().orc_pack_int4(_p(codes), K, N, _p(out))
    return out


def unpack_int4(packed, K: int, N: int):
    packed = _c(packed, np.uint8)
    out = np.empty((K, N), np.int8)
    _load().orc_unpack_int4(_p(packed), K, N, _p(out))
    return out


def pack_int4_canonical(codes):
    """K x N int4 codes in the canonical layout: W^T, K contiguous, two codes
    per byte with even k in the low nibble (N*K/2 bytes)."""
    codes = _c(codes, np.int8)
    K, N = codes.shape
    out = np.empty(N * K // 2, np.uint8)
    _load().orc_pack_int4_canonical(_p(codes), K, N, _p(out))
    return out


def unpack_int4_canonical(packed, K: int, N: int):
    packed = _c(packed, np.uint8)
    out = np.empty((K, N), np.int8)
    _load().orc_unpack_int4_canonical(_p(packed), K, N, _p(out))
    return out


def pack_weights(w, g: int = 128, alpha: int = 1024):
    """Whole offline weight path: codes, packed bytes, float and integer scales, alpha.

    alpha == 0 runs the amplifier search.
    """
    codes, fscale = group_quant_int4(w, g)
    if alpha == 0:
        n = amplifier_log2(fscale)
        alpha = 1 << n
    return {"codes": codes, "packed": pack_int4(codes), "fscale": fscale,
            "iscale": integer_scales(fscale, alpha), "alpha": alpha}


# ----------------------------------------------------------------------- GEMMs

def _sel(idx):
    if idx is None:
        return None, 0
    a = np.ascontiguousarray(idx, dtype=np.int64)
    return a, a.size


def w4a8_gemm_is(qx, sx, codes, iscale, alpha: int, g: int = 128, rows=None, cols=None):
    """Integer-scale W4A8 GEMM on the listed rows x cols.

    Returns (A int64 [nrows x ncols], y float32 [nrows x ncols], overflow count).
    """
    qx = _c(qx, np.int8); sx = _c(sx, np.float32)
    codes = _c(codes, np.int8); iscale = _c(iscale, np.int32)
    M, K = qx.shape
    N = codes.shape[1]
    r, nr = _sel(rows); c, nc = _sel(cols)
    nr = nr if r is not None else M
    nc = nc if c is not None else N
    A = np.empty((nr, nc), np.int64)
    y = np.empty((nr, nc), np.float32)
    ov = _load().orc_w4a8_gemm_is(_p(qx), _p(sx), _p(codes), _p(iscale), int(alpha), M, N, K, g,
                                  _p(r), nr, _p(c), nc, _p(A), _p(y))
    return A, y, int(ov)


def w8a8_gemm_is(qx, sx, codes, iscale, alpha: int, g: int = 128, rows=None, cols=None):
    """Fine-grained W8A8 GEMM with the integer-scale epilogue: the definition of
    O3 with int8 weight codes in [-127, 127] (the epilogue does not depend on
    the weight width). Returns (A int64, y float32, overflow count)."""
    return w4a8_gemm_is(qx, sx, codes, iscale, alpha, g, rows, cols)


def moe_w4a8_gemm_is(qx, sx, codes, iscale, alpha: int, offs, tok, g: int = 128, cols=None):
    """Grouped (mixture-of-experts) integer-scale GEMM: expert e's slots
    offs[e] .. offs[e+1]-1 each multiply activation row tok[slot] by expert
    e's weights (codes[e], K x N; iscale[e]), with the O3 definition; y rows
    follow the slots. Returns (A int64 [R x ncols], y float32, overflow count)."""
    offs = np.asarray(offs, np.int64)
    tok = np.asarray(tok, np.int64)
    E = len(offs) - 1
    R = int(offs[-1])
    N = codes.shape[2]
    nc = N if cols is None else len(cols)
    A = np.zeros((R, nc), np.int64)
    y = np.zeros((R, nc), np.float32)
    ov = 0
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        rows = tok[a:b]
        Ae, ye, oe = w4a8_gemm_is(qx[rows], sx[rows], codes[e], iscale[e], alpha, g, cols=cols)
        A[a:b], y[a:b] = Ae, ye
        ov += oe
    return A, y, ov


def w4a8_gemm_fs(qx, sx, codes, fscale, g: int = 128, rows=None, cols=None):
    """Float-scale W4A8 GEMM (ascending-group fmaf chain). Parity unpinned beyond
    the shared integer partials and the error bound checked in the tests."""
    qx = _c(qx, np.int8); sx = _c(sx, np.float32)
    codes = _c(codes, np.int8); fscale = _c(fscale, np.float32)
    M, K = qx.shape
    N = codes.shape[1]
    r, nr = _sel(rows); c, nc = _sel(cols)
    nr = nr if r is not None else M
    nc = nc if c is not None else N
    y = np.empty((nr, nc), np.float32)
    _load().orc_w4a8_gemm_fs(_p(qx), _p(sx), _p(codes), _p(fscale), M, N, K, g,
                             _p(r), nr, _p(c), nc, _p(y))
    return y


def w8a8_gemm_zp(qx, sx, zx, rowsum_x, qw, sw, zw, colsum_w, rows=None, cols=None):
    """Asymmetric W8A8 GEMM through the zero-point expansion.

    Returns (A int64, y float32, overflow count).
    """
    qx = _c(qx, np.uint8); qw = _c(qw, np.uint8)
    sx = _c(sx, np.float32); sw = _c(sw, np.float32)
    zx = _c(zx, np.int32); zw = _c(zw, np.int32)
    rowsum_x = _c(rowsum_x, np.int32); colsum_w = _c(colsum_w, np.int32)
    M, K = qx.shape
    N = qw.shape[0]
    r, nr = _sel(rows); c, nc = _sel(cols)
    nr = nr if r is not None else M
    nc = nc if c is not None else N
    A = np.empty((nr, nc), np.int64)
    y = np.empty((nr, nc), np.float32)
    ov = _load().orc_w8a8_gemm_zp(_p(qx), _p(sx), _p(zx), _p(rowsum_x), _p(qw), _p(sw), _p(zw),
                                  _p(colsum_w), M, N, K, _p(r), nr, _p(c), nc, _p(A), _p(y))
    return A, y, int(ov)
