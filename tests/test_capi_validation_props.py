"""Property tests of the C ABI's argument validation (no GPU needed).

For random argument tuples with at least one invalid field, the GEMM entry
points must return the status that the documented checks give, in their
documented order (NULL pointers, then mode / element type / width, then
shapes, then the amplifier, then alignment), before any HIP call. A small
model of those rules, written from include/bgt.h, predicts the status.
Pointers are never dereferenced: an invalid call fails validation first.
The module is skipped where a GPU is visible, so that a mistake in the model
(a valid tuple predicted invalid) can never launch a kernel on fake pointers;
examples are derandomized so every run checks the same tuples.
"""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import torch  # noqa: E402

import bit_gemm_token_amd as bgt  # noqa: E402

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake device pointers: runs only where no GPU is visible")

P = ctypes.c_void_p
ALIGNED = 0x10000
MISALIGNED = 0x10004


def _ptr(kind):
    return None if kind == "null" else P(ALIGNED if kind == "ok" else MISALIGNED)


def _shape_ok(M, N, K, kmax=65536):
    return 1 <= M <= 65536 and 16 <= N <= (1 << 24) and N % 16 == 0 and \
        128 <= K <= kmax and K % 128 == 0


def _alpha_ok(a):
    return 1 <= a <= (1 << 30) and (a & (a - 1)) == 0


ptr_kinds = st.sampled_from(["ok", "ok", "ok", "null", "mis"])
dims = st.one_of(st.integers(-5, 70000), st.sampled_from([0, 1, 16, 128, 4096, 65536, 65537]))
ns = st.one_of(st.integers(-5, 5000), st.sampled_from([16, 4096, 22016, 1 << 24, (1 << 24) + 16]))
alphas = st.one_of(st.integers(-3, 5000), st.sampled_from([1, 1024, 1 << 30, 3, 0]))


def _expect(ptrs, required, mode_ok, M, N, K, alpha, kmax=65536, alpha_used=True):
    if any(ptrs[n] == "null" for n in required):
        return bgt.BGT_ERR_NULL
    if not mode_ok:
        return bgt.BGT_ERR_MODE
    if not _shape_ok(M, N, K, kmax):
        return bgt.BGT_ERR_SHAPE
    if alpha_used and not _alpha_ok(alpha):
        return bgt.BGT_ERR_ALPHA
    if any(v == "mis" for v in ptrs.values()):
        return bgt.BGT_ERR_ALIGN
    return None                               # valid: would launch; not called here


@settings(max_examples=400, deadline=None, derandomize=True)
@given(qx=ptr_kinds, sx=st.sampled_from(["ok", "null"]), pk=ptr_kinds, isc=ptr_kinds, y=ptr_kinds,
       acc=st.sampled_from(["ok", "null", "mis"]), width=st.sampled_from([1, 2, 4, 0, 3, 8]),
       yt=st.sampled_from([0, 1, 2, 3, -1]), M=dims, N=ns, K=dims, alpha=alphas)
def test_w4a8_gemm_is_ex_validation(qx, sx, pk, isc, y, acc, width, yt, M, N, K, alpha):
    ptrs = {"qx": qx, "sx": sx, "pk": pk, "isc": isc, "y": y, "acc": acc}
    mode_ok = width in (1, 2, 4) and yt in (0, 1, 2)
    want = _expect(ptrs, ("qx", "sx", "pk", "isc", "y"), mode_ok, M, N, K, alpha)
    if want is None:
        return
    got = bgt.lib().bgt_w4a8_gemm_is_ex(_ptr(qx), _ptr(sx), _ptr(pk), _ptr(isc), width, alpha, M, N,
                                        K, _ptr(y), yt, _ptr(acc), None)
    assert got == want


@settings(max_examples=400, deadline=None, derandomize=True)
@given(qx=ptr_kinds, sx=st.sampled_from(["ok", "null"]), qw=ptr_kinds, isc=ptr_kinds, y=ptr_kinds,
       width=st.sampled_from([1, 2, 4, 5]), yt=st.sampled_from([0, 1, 2, 7]), M=dims, N=ns,
       K=dims, alpha=alphas)
def test_w8a8_gemm_is_validation(qx, sx, qw, isc, y, width, yt, M, N, K, alpha):
    ptrs = {"qx": qx, "sx": sx, "qw": qw, "isc": isc, "y": y}
    want = _expect(ptrs, ("qx", "sx", "qw", "isc", "y"), width in (1, 2, 4) and yt in (0, 1, 2),
                   M, N, K, alpha)
    if want is None:
        return
    got = bgt.lib().bgt_w8a8_gemm_is(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(isc), width, alpha, M, N,
                                     K, _ptr(y), yt, None, None)
    assert got == want


@settings(max_examples=400, deadline=None, derandomize=True)
@given(qx=ptr_kinds, pk=ptr_kinds, isc=ptr_kinds, y=ptr_kinds, offs=st.sampled_from(["ok", "null"]),
       T=dims, E=st.integers(-2, 300), R=st.integers(-2, 3000), N=ns, K=dims, alpha=alphas,
       width=st.sampled_from([1, 2, 4, 6]))
def test_moe_validation(qx, pk, isc, y, offs, T, E, R, N, K, alpha, width):
    ptrs = {"qx": qx, "pk": pk, "isc": isc, "y": y, "offs": offs}
    if any(ptrs[n] == "null" for n in ptrs):
        want = bgt.BGT_ERR_NULL
    elif width not in (1, 2, 4):
        want = bgt.BGT_ERR_MODE
    elif not _shape_ok(T, N, K) or not (1 <= E <= 256 and 1 <= R <= T * E and R <= (1 << 24)):
        want = bgt.BGT_ERR_SHAPE
    elif not _alpha_ok(alpha):
        want = bgt.BGT_ERR_ALPHA
    elif any(v == "mis" for n, v in ptrs.items() if n != "offs"):
        want = bgt.BGT_ERR_ALIGN
    else:
        return
    got = bgt.lib().bgt_w4a8_moe_gemm_is(_ptr(qx), P(ALIGNED), T, _ptr(offs), P(ALIGNED), E, R,
                                         _ptr(pk), _ptr(isc), width, alpha, N, K, _ptr(y), 0, None,
                                         None)
    assert got == want
