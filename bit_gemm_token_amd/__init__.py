"""bit_gemm_token_amd -- fine-grained W4A8 integer-scale linear layer for MI355X.

A thin Python binding over libbgt.so (include/bgt.h): it checks tensor dtypes,
devices and shapes, passes data pointers and torch's current HIP stream, and
turns non-zero status codes into exceptions. Every step of the computation
runs in the HIP kernels of libbgt; there is no fallback. If the library is not
built, importing the entry points raises.

Entry points (same names as the C ABI without the ``bgt_`` prefix; the _ex
and _narrow C variants are reached through the dtype of the tensors passed):
    quantize_act(x, mode="sym")            -> (q, scale[, zero], rowsum)
    pack_weights_int4(w, alpha=1024)       -> dict(packed, fscale, iscale, alpha, status)
    narrow_iscale(iscale, width)           -> iscale as uint8 / uint16
    w4a8_gemm_is(qx, sx, packed, iscale, alpha, N)   -> y
    w4a8_gemm_is_narrow(qx, sx, packed, iscale, alpha, N, out_dtype=None) -> y
    w4a8_linear_is(x, packed, iscale, alpha, N)      -> (y, qx, sx)
    w4a8_linear_fused(x)                   -> bool (one launch for this x)
    w4a8_gemm_fs(qx, sx, packed, fscale, N, out_dtype=None) -> y
    w8a8_gemm_zp(qx, sx, zx, rowsum_x, qw, sw, zw, colsum_w) -> y
    w4a8_moe_gemm_is(qx, sx, offsets, slot_token, packed, iscale, alpha, N) -> y
    pack_weights_int8(w, alpha=0)          -> dict(qw, fscale, iscale, alpha, status)
    w8a8_gemm_is(qx, sx, qw, iscale, alpha, N)       -> y
    w4a8_kernel_name / w8a8_is_kernel_name / w4a8_moe_kernel_name -> kernel a shape runs
    set_prefill_kernel("auto" | "wide" | "tiled")   tile kernel of the W4A8 GEMMs for M > 64
    w4a8_workspace_bytes(M, N, K)          -> split-K workspace the integer-scale GEMM uses
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbgt.so")

BGT_OK = 0
BGT_WARN_ACC_MAY_OVERFLOW = 1
BGT_ERR_NULL = -1
BGT_ERR_SHAPE = -2
BGT_ERR_ALIGN = -3
BGT_ERR_ALPHA = -4
BGT_ERR_MODE = -5
BGT_ERR_HIP = -6
BGT_ERR_RANGE = -7
BGT_F32 = 0
BGT_F16 = 1
BGT_BF16 = 2
BGT_QUANT_SYM_I8 = 0
BGT_QUANT_ASYM_U8 = 1
GROUP = 128

EXPORTED = (
    "bgt_quantize_act", "bgt_pack_weights_int4", "bgt_w4a8_gemm_is", "bgt_w4a8_gemm_fs",
    "bgt_w8a8_gemm_zp", "bgt_status_string", "bgt_abi_version", "bgt_w4a8_kernel_name",
    "bgt_narrow_iscale", "bgt_w4a8_gemm_is_narrow", "bgt_w4a8_linear_is", "bgt_w4a8_linear_fused",
    "bgt_quantize_act_ex", "bgt_w4a8_gemm_is_ex", "bgt_w4a8_gemm_fs_ex",
    "bgt_pack_weights_int8", "bgt_w8a8_gemm_is", "bgt_w8a8_is_kernel_name",
    "bgt_w4a8_moe_gemm_is", "bgt_w4a8_moe_kernel_name", "bgt_repack_int4_canonical",
    "bgt_set_prefill_kernel", "bgt_w4a8_workspace_bytes", "bgt_w4a8_gemm_is_noalloc",
)
_NAMES = ("bgt_status_string", "bgt_w4a8_kernel_name", "bgt_w8a8_is_kernel_name",
          "bgt_w4a8_moe_kernel_name")

_lib = None


class BgtError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


def lib():
    """The loaded libbgt.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_gemm_token_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bgt_quantize_act.argtypes = [P, I64, I64, I64, I, P, P, P, P, P]
        L.bgt_pack_weights_int4.argtypes = [P, I64, I64, I64, I, P, P, P, ctypes.POINTER(I), P]
        L.bgt_w4a8_gemm_is.argtypes = [P, P, P, P, I, I64, I64, I64, P, P, P]
        L.bgt_w4a8_gemm_fs.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        L.bgt_narrow_iscale.argtypes = [P, I64, I, P, P]
        L.bgt_w4a8_gemm_is_narrow.argtypes = [P, P, P, P, I, I, I64, I64, I64, P, P, P]
        L.bgt_w4a8_linear_is.argtypes = [P, I, I64, P, P, I, I, I64, I64, I64, P, P, P, I, P]
        L.bgt_quantize_act_ex.argtypes = [P, I, I64, I64, I64, I, P, P, P, P, P]
        L.bgt_w4a8_gemm_is_ex.argtypes = [P, P, P, P, I, I, I64, I64, I64, P, I, P, P]
        L.bgt_w4a8_gemm_fs_ex.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
        L.bgt_w4a8_linear_fused.argtypes = [I64, I64, P, I64]
        L.bgt_w8a8_gemm_zp.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, P, P, P]
        L.bgt_status_string.argtypes = [I]
        L.bgt_status_string.restype = ctypes.c_char_p
        L.bgt_abi_version.restype = I
        L.bgt_w4a8_kernel_name.argtypes = [I64, I64, I64, I]
        L.bgt_pack_weights_int8.argtypes = [P, I64, I64, I64, I, P, P, P, ctypes.POINTER(I), P]
        L.bgt_w8a8_gemm_is.argtypes = [P, P, P, P, I, I, I64, I64, I64, P, I, P, P]
        L.bgt_w8a8_is_kernel_name.argtypes = [I64, I64, I64]
        L.bgt_w4a8_moe_gemm_is.argtypes = [P, P, I64, P, P, I64, I64, P, P, I, I, I64, I64, P, I,
                                           P, P]
        L.bgt_w4a8_moe_kernel_name.argtypes = [I64, I64, I64, I64]
        L.bgt_repack_int4_canonical.argtypes = [P, I64, I64, P, P]
        L.bgt_set_prefill_kernel.argtypes = [I]
        L.bgt_w4a8_workspace_bytes.argtypes = [I64, I64, I64]
        L.bgt_w4a8_gemm_is_noalloc.argtypes = [P, P, P, P, I, I64, I64, I64, P, P, P]
        for f in EXPORTED:
            getattr(L, f).restype = ctypes.c_char_p if f in _NAMES else I
        L.bgt_w4a8_workspace_bytes.restype = I64
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bgt_status_string(int(status)).decode()


PREFILL_KERNELS = {"auto": 0, "wide": 1, "tiled": 2}


def set_prefill_kernel(mode: str = "auto"):
    """Tile kernel of the dense W4A8 GEMMs for M > 64: "auto" (by launch
    rounds), "wide" (256 x 256 tiles) or "tiled" (256 x 128). Process-wide."""
    if mode not in PREFILL_KERNELS:
        raise ValueError(f"mode must be one of {sorted(PREFILL_KERNELS)}")
    _raise("bgt_set_prefill_kernel", lib().bgt_set_prefill_kernel(PREFILL_KERNELS[mode]))


def w4a8_workspace_bytes(M: int, N: int, K: int) -> int:
    """Device workspace (bytes) the integer-scale W4A8 GEMM uses at this shape."""
    r = lib().bgt_w4a8_workspace_bytes(M, N, K)
    _raise("bgt_w4a8_workspace_bytes", r if r < 0 else 0)
    return r


def w4a8_kernel_name(M: int, N: int, K: int, float_scale: bool = False) -> str:
    """Name of the GEMM kernel a W4A8 call of this shape launches (profiling aid)."""
    return lib().bgt_w4a8_kernel_name(int(M), int(N), int(K), 1 if float_scale else 0).decode()


def w8a8_is_kernel_name(M: int, N: int, K: int) -> str:
    """Name of the kernel a fine-grained W8A8 integer-scale call launches."""
    return lib().bgt_w8a8_is_kernel_name(int(M), int(N), int(K)).decode()


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _elem_type(t, name):
    """BGT element-type code of a float32 / float16 / bfloat16 tensor."""
    torch = _torch()
    codes = {torch.float32: BGT_F32, torch.float16: BGT_F16, torch.bfloat16: BGT_BF16}
    if t.dtype not in codes:
        raise TypeError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}")
    return codes[t.dtype]


def _raise(fn, st):
    if st < 0:
        raise BgtError(fn, st)
    return st


# ------------------------------------------------------------------ entry points
def quantize_act(x, mode: str = "sym", q=None, scale=None, zero=None, rowsum=None,
                 want_rowsum: bool = False):
    """Per-row dynamic quantization of x (rows x cols float32, float16 or
    bfloat16, row-major; half types are widened to fp32 exactly).

    mode "sym": int8 codes in [-127, 127] and one scale per row.
    mode "asym": uint8 codes in [0, 255], scale, zero point and code row sum.
    Returns (q, scale, rowsum) for "sym" (rowsum None unless asked for) and
    (q, scale, zero, rowsum) for "asym".
    """
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a GPU tensor with unit column stride")
    xt = _elem_type(x, "x")
    ld = x.stride(0)
    asym = mode == "asym"
    if mode not in ("sym", "asym"):
        raise ValueError("mode must be 'sym' or 'asym'")
    dev = x.device
    qdt = torch.uint8 if asym else torch.int8
    q = torch.empty((rows, cols), dtype=qdt, device=dev) if q is None else q
    scale = torch.empty(rows, dtype=torch.float32, device=dev) if scale is None else scale
    if asym and zero is None:
        zero = torch.empty(rows, dtype=torch.int32, device=dev)
    if (asym or want_rowsum) and rowsum is None:
        rowsum = torch.empty(rows, dtype=torch.int32, device=dev)
    _check(q, "q", qdt, (rows, cols))
    _check(scale, "scale", torch.float32, (rows,))
    if zero is not None:
        _check(zero, "zero", torch.int32, (rows,))
    if rowsum is not None:
        _check(rowsum, "rowsum", torch.int32, (rows,))
    st = lib().bgt_quantize_act_ex(_ptr(x), xt, rows, cols, ld,
                                   BGT_QUANT_ASYM_U8 if asym else BGT_QUANT_SYM_I8,
                                   _ptr(q), _ptr(scale), _ptr(zero), _ptr(rowsum), _stream(dev))
    _raise("bgt_quantize_act_ex", st)
    return (q, scale, zero, rowsum) if asym else (q, scale, rowsum)


def pack_weights_int4(w, alpha: int = 1024, group: int = GROUP, packed=None, fscale=None,
                      iscale=None):
    """Offline int4 group quantization of w (K x N float32) and its integer scales.

    alpha=0 runs the amplifier search. Synchronous. Returns a dict with
    packed (N*K/2 uint8), fscale, iscale ((K/128) x N), alpha and status
    (0, or 1 = the worst-case accumulator may exceed int32).
    """
    torch = _torch()
    _check(w, "w", torch.float32)
    K, N = w.shape
    dev = w.device
    G = K // group if group else 0
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=dev) if packed is None else packed
    fscale = torch.empty((G, N), dtype=torch.float32, device=dev) if fscale is None else fscale
    iscale = torch.empty((G, N), dtype=torch.int32, device=dev) if iscale is None else iscale
    _check(packed, "packed", torch.uint8, (N * K // 2,))
    _check(fscale, "fscale", torch.float32, (G, N))
    _check(iscale, "iscale", torch.int32, (G, N))
    a_out = ctypes.c_int(0)
    st = lib().bgt_pack_weights_int4(_ptr(w), K, N, group, int(alpha), _ptr(packed), _ptr(fscale),
                                     _ptr(iscale), ctypes.byref(a_out), _stream(dev))
    _raise("bgt_pack_weights_int4", st)
    return {"packed": packed, "fscale": fscale, "iscale": iscale, "alpha": a_out.value,
            "status": st}


def _gemm_common(qx, sx, packed, scale, scale_dtype, N):
    torch = _torch()
    _check(qx, "qx", torch.int8)
    M, K = qx.shape
    _check(sx, "sx", torch.float32, (M,))
    _check(packed, "packed", torch.uint8, (N * K // 2,))
    _check(scale, "scale", scale_dtype, (K // GROUP, N))
    return M, K


def w4a8_gemm_is(qx, sx, packed, iscale, alpha: int, N: int, y=None, acc_out=None):
    """Y = X.W with the integer-scale epilogue; returns y (M x N float32)."""
    torch = _torch()
    M, K = _gemm_common(qx, sx, packed, iscale, torch.int32, N)
    y = torch.empty((M, N), dtype=torch.float32, device=qx.device) if y is None else y
    _check(y, "y", torch.float32, (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", torch.int32, (M, N))
    st = lib().bgt_w4a8_gemm_is(_ptr(qx), _ptr(sx), _ptr(packed), _ptr(iscale), int(alpha), M, N,
                                K, _ptr(y), _ptr(acc_out), _stream(qx.device))
    _raise("bgt_w4a8_gemm_is", st)
    return y


_NARROW = {1: "uint8", 2: "uint16", 4: "int32"}


def repack_int4_canonical(canonical, K: int, N: int, packed=None):
    """int4 codes in the canonical layout (W^T, K contiguous, two per byte, even
    k in the low nibble; N*K/2 uint8) rewritten into the GEMMs' layout; returns
    the packed tensor (N*K/2 uint8)."""
    torch = _torch()
    _check(canonical, "canonical", torch.uint8, (N * K // 2,))
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=canonical.device) if packed is None else packed
    _check(packed, "packed", torch.uint8, (N * K // 2,))
    st = lib().bgt_repack_int4_canonical(_ptr(canonical), int(K), int(N), _ptr(packed),
                                         _stream(canonical.device))
    _raise("bgt_repack_int4_canonical", st)
    return packed


def narrow_iscale(iscale, width: int, out=None):
    """Integer scales stored in `width`-byte elements (1: uint8, 2: uint16).

    Same values; raises BgtError (BGT_ERR_RANGE) if one does not fit.
    Blocks until the scales have been checked on the host."""
    torch = _torch()
    _check(iscale, "iscale", torch.int32)
    if width not in (1, 2):
        raise ValueError("width must be 1 or 2")
    dt = getattr(torch, _NARROW[width])
    out = torch.empty(iscale.shape, dtype=dt, device=iscale.device) if out is None else out
    _check(out, "out", dt, tuple(iscale.shape))
    st = lib().bgt_narrow_iscale(_ptr(iscale), iscale.numel(), int(width), _ptr(out),
                                 _stream(iscale.device))
    _raise("bgt_narrow_iscale", st)
    return out


def w4a8_gemm_is_narrow(qx, sx, packed, iscale, alpha: int, N: int, y=None, acc_out=None,
                        out_dtype=None):
    """w4a8_gemm_is with integer scales stored as uint8, uint16 or int32
    (width taken from iscale's dtype) and y as float32, float16 or bfloat16
    (y's dtype, or out_dtype when y is not given); returns y (M x N)."""
    torch = _torch()
    widths = {torch.uint8: 1, torch.uint16: 2, torch.int32: 4}
    if not isinstance(iscale, torch.Tensor) or iscale.dtype not in widths:
        raise TypeError("iscale must be a uint8, uint16 or int32 tensor")
    M, K = _gemm_common(qx, sx, packed, iscale, iscale.dtype, N)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qx.device)
    _check(y, "y", y.dtype, (M, N))
    yt = _elem_type(y, "y")
    if acc_out is not None:
        _check(acc_out, "acc_out", torch.int32, (M, N))
    st = lib().bgt_w4a8_gemm_is_ex(_ptr(qx), _ptr(sx), _ptr(packed), _ptr(iscale),
                                   widths[iscale.dtype], int(alpha), M, N, K, _ptr(y), yt,
                                   _ptr(acc_out), _stream(qx.device))
    _raise("bgt_w4a8_gemm_is_ex", st)
    return y


def w4a8_linear_is(x, packed, iscale, alpha: int, N: int, qx=None, sx=None, y=None,
                   out_dtype=None):
    """Per-token quantization of x (M x K float32, float16 or bfloat16) and the
    integer-scale GEMM; y float32, float16 or bfloat16 (y's dtype, else
    out_dtype, else x's dtype).

    One launch for M <= 4 on the decode path (see w4a8_linear_fused); returns
    (y, qx, sx), the quantized activations included."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D GPU tensor with unit column stride")
    xt = _elem_type(x, "x")
    M, K = x.shape
    widths = {torch.uint8: 1, torch.uint16: 2, torch.int32: 4}
    if not isinstance(iscale, torch.Tensor) or iscale.dtype not in widths:
        raise TypeError("iscale must be a uint8, uint16 or int32 tensor")
    _check(packed, "packed", torch.uint8, (N * K // 2,))
    _check(iscale, "iscale", iscale.dtype, (K // GROUP, N))
    dev = x.device
    qx = torch.empty((M, K), dtype=torch.int8, device=dev) if qx is None else qx
    sx = torch.empty(M, dtype=torch.float32, device=dev) if sx is None else sx
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or x.dtype, device=dev)
    _check(qx, "qx", torch.int8, (M, K))
    _check(sx, "sx", torch.float32, (M,))
    _check(y, "y", y.dtype, (M, N))
    yt = _elem_type(y, "y")
    st = lib().bgt_w4a8_linear_is(_ptr(x), xt, x.stride(0), _ptr(packed), _ptr(iscale),
                                  widths[iscale.dtype], int(alpha), M, N, K, _ptr(qx), _ptr(sx),
                                  _ptr(y), yt, _stream(dev))
    _raise("bgt_w4a8_linear_is", st)
    return y, qx, sx


def w4a8_linear_fused(x) -> bool:
    """True when w4a8_linear_is runs as a single launch for this x."""
    M, K = x.shape
    return bool(lib().bgt_w4a8_linear_fused(M, K, _ptr(x), x.stride(0)))


def w4a8_gemm_fs(qx, sx, packed, fscale, N: int, y=None, out_dtype=None):
    """Y = X.W with the float-scale epilogue (the control); y float32, float16
    or bfloat16 (y's dtype, or out_dtype); returns y."""
    torch = _torch()
    M, K = _gemm_common(qx, sx, packed, fscale, torch.float32, N)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qx.device)
    _check(y, "y", y.dtype, (M, N))
    yt = _elem_type(y, "y")
    st = lib().bgt_w4a8_gemm_fs_ex(_ptr(qx), _ptr(sx), _ptr(packed), _ptr(fscale), M, N, K,
                                   _ptr(y), yt, _stream(qx.device))
    _raise("bgt_w4a8_gemm_fs_ex", st)
    return y


def w8a8_gemm_zp(qx, sx, zx, rowsum_x, qw, sw, zw, colsum_w, y=None, acc_out=None):
    """Asymmetric W8A8 GEMM via the zero-point expansion; returns y (M x N)."""
    torch = _torch()
    _check(qx, "qx", torch.uint8)
    _check(qw, "qw", torch.uint8)
    M, K = qx.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("qw must be N x K")
    for t, n, nm in ((sx, M, "sx"), (sw, N, "sw")):
        _check(t, nm, torch.float32, (n,))
    for t, n, nm in ((zx, M, "zx"), (rowsum_x, M, "rowsum_x"), (zw, N, "zw"), (colsum_w, N, "colsum_w")):
        _check(t, nm, torch.int32, (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=qx.device) if y is None else y
    _check(y, "y", torch.float32, (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", torch.int32, (M, N))
    st = lib().bgt_w8a8_gemm_zp(_ptr(qx), _ptr(sx), _ptr(zx), _ptr(rowsum_x), _ptr(qw), _ptr(sw),
                                _ptr(zw), _ptr(colsum_w), M, N, K, _ptr(y), _ptr(acc_out),
                                _stream(qx.device))
    _raise("bgt_w8a8_gemm_zp", st)
    return y


def pack_weights_int8(w, alpha: int = 0, group: int = GROUP, qw=None, fscale=None, iscale=None):
    """Offline int8 group quantization of w (K x N float32) into the int8
    fragment layout, with float and integer scales.

    alpha=0 runs the amplifier search. Synchronous. Returns a dict with qw
    (N*K int8), fscale, iscale ((K/128) x N), alpha and status (0, or 1 = the
    worst-case accumulator may exceed int32).
    """
    torch = _torch()
    _check(w, "w", torch.float32)
    K, N = w.shape
    dev = w.device
    G = K // group if group else 0
    qw = torch.empty(N * K, dtype=torch.int8, device=dev) if qw is None else qw
    fscale = torch.empty((G, N), dtype=torch.float32, device=dev) if fscale is None else fscale
    iscale = torch.empty((G, N), dtype=torch.int32, device=dev) if iscale is None else iscale
    _check(qw, "qw", torch.int8, (N * K,))
    _check(fscale, "fscale", torch.float32, (G, N))
    _check(iscale, "iscale", torch.int32, (G, N))
    a_out = ctypes.c_int(0)
    st = lib().bgt_pack_weights_int8(_ptr(w), K, N, group, int(alpha), _ptr(qw), _ptr(fscale),
                                     _ptr(iscale), ctypes.byref(a_out), _stream(dev))
    _raise("bgt_pack_weights_int8", st)
    return {"qw": qw, "fscale": fscale, "iscale": iscale, "alpha": a_out.value, "status": st}


def w8a8_gemm_is(qx, sx, qw, iscale, alpha: int, N: int, y=None, acc_out=None, out_dtype=None):
    """Fine-grained W8A8 Y = X.W with the integer-scale epilogue. iscale is
    uint8, uint16 or int32 ((K/128) x N); y float32, float16 or bfloat16
    (y's dtype, or out_dtype when y is not given). Returns y (M x N)."""
    torch = _torch()
    widths = {torch.uint8: 1, torch.uint16: 2, torch.int32: 4}
    if not isinstance(iscale, torch.Tensor) or iscale.dtype not in widths:
        raise TypeError("iscale must be a uint8, uint16 or int32 tensor")
    _check(qx, "qx", torch.int8)
    M, K = qx.shape
    _check(sx, "sx", torch.float32, (M,))
    _check(qw, "qw", torch.int8, (N * K,))
    _check(iscale, "iscale", iscale.dtype, (K // GROUP, N))
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qx.device)
    _check(y, "y", y.dtype, (M, N))
    yt = _elem_type(y, "y")
    if acc_out is not None:
        _check(acc_out, "acc_out", torch.int32, (M, N))
    st = lib().bgt_w8a8_gemm_is(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(iscale), widths[iscale.dtype],
                                int(alpha), M, N, K, _ptr(y), yt, _ptr(acc_out),
                                _stream(qx.device))
    _raise("bgt_w8a8_gemm_is", st)
    return y


def w4a8_moe_kernel_name(T: int, E: int, R: int, K: int) -> str:
    """Name of the kernel a grouped W4A8 call with T tokens, E experts and R
    routed slots launches."""
    return lib().bgt_w4a8_moe_kernel_name(int(T), int(E), int(R), int(K)).decode()


def w4a8_moe_gemm_is(qx, sx, offsets, slot_token, packed, iscale, alpha: int, N: int, y=None,
                     acc_out=None, out_dtype=None):
    """Grouped (mixture-of-experts) W4A8 GEMM with the integer-scale epilogue.

    qx (T x K int8) and sx (T) are the tokens; offsets (E+1 int32) and
    slot_token (R int32) the expert-sorted routing; packed (E x N*K/2 uint8)
    and iscale (E x K/128 x N; uint8, uint16 or int32) the experts' weights.
    Returns y (R x N; float32, float16 or bfloat16), row r for slot r."""
    torch = _torch()
    widths = {torch.uint8: 1, torch.uint16: 2, torch.int32: 4}
    if not isinstance(iscale, torch.Tensor) or iscale.dtype not in widths:
        raise TypeError("iscale must be a uint8, uint16 or int32 tensor")
    _check(qx, "qx", torch.int8)
    T, K = qx.shape
    _check(sx, "sx", torch.float32, (T,))
    _check(offsets, "offsets", torch.int32)
    E = offsets.numel() - 1
    _check(slot_token, "slot_token", torch.int32)
    R = slot_token.numel()
    _check(packed, "packed", torch.uint8, (E, N * K // 2))
    _check(iscale, "iscale", iscale.dtype, (E, K // GROUP, N))
    if y is None:
        y = torch.empty((R, N), dtype=out_dtype or torch.float32, device=qx.device)
    _check(y, "y", y.dtype, (R, N))
    yt = _elem_type(y, "y")
    if acc_out is not None:
        _check(acc_out, "acc_out", torch.int32, (R, N))
    st = lib().bgt_w4a8_moe_gemm_is(_ptr(qx), _ptr(sx), T, _ptr(offsets), _ptr(slot_token), E, R,
                                    _ptr(packed), _ptr(iscale), widths[iscale.dtype], int(alpha),
                                    N, K, _ptr(y), yt, _ptr(acc_out), _stream(qx.device))
    _raise("bgt_w4a8_moe_gemm_is", st)
    return y

