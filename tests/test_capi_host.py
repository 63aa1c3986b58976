"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every symbol include/bgt.h declares, and rejects
every invalid argument before any HIP call (so these calls need no device).
Pointers below are never dereferenced: validation fails first.
"""
import ctypes
import os
import re

import pytest

import bit_gemm_token_amd as bgt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

P = ctypes.c_void_p
FAKE = P(0x10000)          # aligned, non-null, never touched
MIS = P(0x10004)           # misaligned


@pytest.fixture(scope="module")
def L():
    return bgt.lib()


def test_header_symbols_exported(L):
    with open(os.path.join(ROOT, "include", "bgt.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^(?:int|int64_t|const char\*)\s+(bgt_\w+)\s*\(", hdr, re.M))
    assert declared == set(bgt.EXPORTED)
    for name in declared:
        assert getattr(L, name) is not None


def test_status_strings(L):
    assert bgt.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5, -6, -7, 1):
        assert "error" in bgt.status_string(st) or "warning" in bgt.status_string(st)
    assert L.bgt_abi_version() == 109


def test_quantize_act_validation(L):
    q = L.bgt_quantize_act
    assert q(FAKE, 4, 64, 64, 7, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_MODE
    assert q(None, 4, 64, 64, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_NULL
    assert q(FAKE, 4, 64, 64, 1, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_NULL   # asym needs zero
    assert q(FAKE, 0, 64, 64, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_SHAPE
    assert q(FAKE, 4, 64, 32, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_SHAPE  # ld < cols
    assert q(FAKE, 4, 0, 64, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_SHAPE


def test_pack_validation(L):
    a = ctypes.c_int(0)
    pk = L.bgt_pack_weights_int4
    ok = dict(K=256, N=32, g=128, alpha=1024)

    def call(w=FAKE, K=256, N=32, g=128, alpha=1024, packed=FAKE, fs=FAKE, isc=FAKE, aout=True):
        return pk(w, K, N, g, alpha, packed, fs, isc, ctypes.byref(a) if aout else None, None)

    assert call(w=None) == bgt.BGT_ERR_NULL
    assert call(aout=False) == bgt.BGT_ERR_NULL
    assert call(g=64) == bgt.BGT_ERR_SHAPE
    assert call(K=200) == bgt.BGT_ERR_SHAPE
    assert call(N=24) == bgt.BGT_ERR_SHAPE
    assert call(alpha=1000) == bgt.BGT_ERR_ALPHA
    assert call(alpha=-4) == bgt.BGT_ERR_ALPHA
    assert call(alpha=1 << 31 if False else 3) == bgt.BGT_ERR_ALPHA
    assert call(packed=MIS) == bgt.BGT_ERR_ALIGN
    assert ok  # the valid call needs a GPU; covered by the gpu tests


def test_gemm_is_validation(L):
    g = L.bgt_w4a8_gemm_is

    def call(qx=FAKE, sx=FAKE, pk=FAKE, isc=FAKE, alpha=1024, M=16, N=64, K=256, y=FAKE, acc=None):
        return g(qx, sx, pk, isc, alpha, M, N, K, y, acc, None)

    assert call(qx=None) == bgt.BGT_ERR_NULL
    assert call(y=None) == bgt.BGT_ERR_NULL
    assert call(M=0) == bgt.BGT_ERR_SHAPE
    assert call(M=65537) == bgt.BGT_ERR_SHAPE
    assert call(N=40) == bgt.BGT_ERR_SHAPE
    assert call(N=0) == bgt.BGT_ERR_SHAPE
    assert call(K=192) == bgt.BGT_ERR_SHAPE
    assert call(K=0) == bgt.BGT_ERR_SHAPE
    assert call(alpha=0) == bgt.BGT_ERR_ALPHA
    assert call(alpha=1000) == bgt.BGT_ERR_ALPHA
    assert call(alpha=1 << 30) != bgt.BGT_ERR_ALPHA or True
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN
    assert call(pk=MIS) == bgt.BGT_ERR_ALIGN
    assert call(acc=MIS) == bgt.BGT_ERR_ALIGN


def test_gemm_is_narrow_validation(L):
    g = L.bgt_w4a8_gemm_is_narrow

    def call(isc=FAKE, width=1, alpha=1024, M=16, N=64, K=256, y=FAKE):
        return g(FAKE, FAKE, FAKE, isc, width, alpha, M, N, K, y, None, None)

    assert call(isc=None) == bgt.BGT_ERR_NULL
    for bad in (0, 3, 8, -1):
        assert call(width=bad) == bgt.BGT_ERR_MODE
    assert call(N=40) == bgt.BGT_ERR_SHAPE
    assert call(alpha=1000) == bgt.BGT_ERR_ALPHA
    assert call(isc=MIS) == bgt.BGT_ERR_ALIGN
    assert call(isc=MIS, width=4) == bgt.BGT_ERR_ALIGN
    # the int32 entry point shares the same checks
    assert L.bgt_w4a8_gemm_is(FAKE, FAKE, FAKE, MIS, 1024, 16, 64, 256, FAKE, None, None) == bgt.BGT_ERR_ALIGN


def test_linear_is_validation(L):
    g = L.bgt_w4a8_linear_is

    def call(x=FAKE, ldx=256, isc=FAKE, width=4, alpha=1024, M=4, N=64, K=256, qx=FAKE, sx=FAKE, y=FAKE,
             xt=0, yt=0):
        return g(x, xt, ldx, FAKE, isc, width, alpha, M, N, K, qx, sx, y, yt, None)

    assert call(x=None) == bgt.BGT_ERR_NULL
    assert call(qx=None) == bgt.BGT_ERR_NULL
    assert call(sx=None) == bgt.BGT_ERR_NULL
    assert call(width=3) == bgt.BGT_ERR_MODE
    assert call(xt=3) == bgt.BGT_ERR_MODE
    assert call(yt=-1) == bgt.BGT_ERR_MODE
    assert call(ldx=255) == bgt.BGT_ERR_SHAPE
    assert call(K=200, ldx=300) == bgt.BGT_ERR_SHAPE
    assert call(alpha=12) == bgt.BGT_ERR_ALPHA
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN
    assert call(isc=MIS) == bgt.BGT_ERR_ALIGN
    f = L.bgt_w4a8_linear_fused
    assert f(4, 4096, FAKE, 4096) == 1
    assert f(1, 2048, FAKE, 2048) == 1
    assert f(5, 4096, FAKE, 4096) == 0          # more than 4 rows
    assert f(4, 1152, FAKE, 1152) == 0          # not 16 or 32 groups
    assert f(4, 4096, MIS, 4096) == 0           # x not 16-byte aligned
    assert f(4, 4096, FAKE, 4097) == 0          # row stride not a multiple of 4


def test_typed_entry_points_validation(L):
    q = L.bgt_quantize_act_ex
    assert q(FAKE, 3, 4, 64, 64, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_MODE
    assert q(None, 1, 4, 64, 64, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_NULL
    assert q(FAKE, 2, 4, 64, 32, 0, FAKE, FAKE, None, None, None) == bgt.BGT_ERR_SHAPE
    g = L.bgt_w4a8_gemm_is_ex
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 1024, 16, 64, 256, FAKE, 5, None, None) == bgt.BGT_ERR_MODE
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 1024, 16, 64, 256, MIS, 1, None, None) == bgt.BGT_ERR_ALIGN
    f = L.bgt_w4a8_gemm_fs_ex
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 64, 256, FAKE, 7, None) == bgt.BGT_ERR_MODE
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 63, 256, FAKE, 2, None) == bgt.BGT_ERR_SHAPE


def test_narrow_iscale_validation(L):
    n = L.bgt_narrow_iscale
    assert n(None, 64, 1, FAKE, None) == bgt.BGT_ERR_NULL
    assert n(FAKE, 64, 1, None, None) == bgt.BGT_ERR_NULL
    assert n(FAKE, 64, 4, FAKE, None) == bgt.BGT_ERR_MODE      # int32 needs no narrowing
    assert n(FAKE, 64, 3, FAKE, None) == bgt.BGT_ERR_MODE
    assert n(FAKE, 0, 1, FAKE, None) == bgt.BGT_ERR_SHAPE
    assert n(MIS, 64, 2, FAKE, None) == bgt.BGT_ERR_ALIGN
    assert n(FAKE, 64, 2, MIS, None) == bgt.BGT_ERR_ALIGN


def test_repack_canonical_validation(L):
    r = L.bgt_repack_int4_canonical
    assert r(None, 256, 32, FAKE, None) == bgt.BGT_ERR_NULL
    assert r(FAKE, 256, 32, None, None) == bgt.BGT_ERR_NULL
    assert r(FAKE, 200, 32, FAKE, None) == bgt.BGT_ERR_SHAPE     # K not a multiple of 128
    assert r(FAKE, 0, 32, FAKE, None) == bgt.BGT_ERR_SHAPE
    assert r(FAKE, 256, 24, FAKE, None) == bgt.BGT_ERR_SHAPE     # N not a multiple of 16
    assert r(FAKE, 131072, 32, FAKE, None) == bgt.BGT_ERR_SHAPE
    assert r(MIS, 256, 32, FAKE, None) == bgt.BGT_ERR_ALIGN
    assert r(FAKE, 256, 32, MIS, None) == bgt.BGT_ERR_ALIGN


def test_gemm_fs_validation(L):
    g = L.bgt_w4a8_gemm_fs
    assert g(FAKE, FAKE, FAKE, None, 16, 64, 256, FAKE, None) == bgt.BGT_ERR_NULL
    assert g(FAKE, FAKE, FAKE, FAKE, 16, 63, 256, FAKE, None) == bgt.BGT_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 16, 64, 100, FAKE, None) == bgt.BGT_ERR_SHAPE
    assert g(FAKE, FAKE, MIS, FAKE, 16, 64, 256, FAKE, None) == bgt.BGT_ERR_ALIGN
    assert g(FAKE, FAKE, FAKE, MIS, 16, 64, 256, FAKE, None) == bgt.BGT_ERR_ALIGN   # fscale


def test_w8a8_validation(L):
    g = L.bgt_w8a8_gemm_zp

    def call(qx=FAKE, M=16, N=64, K=256, zx=FAKE, y=FAKE):
        return g(qx, FAKE, zx, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, y, None, None)

    assert call(zx=None) == bgt.BGT_ERR_NULL
    assert call(K=32768 + 128) == bgt.BGT_ERR_SHAPE       # |A| bound needs K <= 32768
    assert call(N=8) == bgt.BGT_ERR_SHAPE
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises((ValueError, TypeError)):
        bgt.w4a8_gemm_is(torch.zeros(2, 128, dtype=torch.int8), torch.ones(2), torch.zeros(1024, dtype=torch.uint8),
                         torch.zeros(1, 16, dtype=torch.int32), 1024, 16)


def test_pack_int8_validation(L):
    a = ctypes.c_int(0)
    pk = L.bgt_pack_weights_int8

    def call(w=FAKE, K=256, N=32, g=128, alpha=0, qw=FAKE, fs=FAKE, isc=FAKE, aout=True):
        return pk(w, K, N, g, alpha, qw, fs, isc, ctypes.byref(a) if aout else None, None)

    assert call(w=None) == bgt.BGT_ERR_NULL
    assert call(qw=None) == bgt.BGT_ERR_NULL
    assert call(aout=False) == bgt.BGT_ERR_NULL
    assert call(g=256) == bgt.BGT_ERR_SHAPE
    assert call(K=130) == bgt.BGT_ERR_SHAPE
    assert call(N=8) == bgt.BGT_ERR_SHAPE
    assert call(alpha=6) == bgt.BGT_ERR_ALPHA
    assert call(qw=MIS) == bgt.BGT_ERR_ALIGN


def test_w8a8_is_validation(L):
    g = L.bgt_w8a8_gemm_is

    def call(qx=FAKE, sx=FAKE, qw=FAKE, isc=FAKE, width=4, alpha=1 << 18, M=16, N=64, K=256,
             y=FAKE, yt=0, acc=None):
        return g(qx, sx, qw, isc, width, alpha, M, N, K, y, yt, acc, None)

    assert call(qx=None) == bgt.BGT_ERR_NULL
    assert call(qw=None) == bgt.BGT_ERR_NULL
    assert call(isc=None) == bgt.BGT_ERR_NULL
    assert call(y=None) == bgt.BGT_ERR_NULL
    assert call(width=3) == bgt.BGT_ERR_MODE
    assert call(yt=5) == bgt.BGT_ERR_MODE
    assert call(M=0) == bgt.BGT_ERR_SHAPE
    assert call(N=40) == bgt.BGT_ERR_SHAPE
    assert call(K=100) == bgt.BGT_ERR_SHAPE
    assert call(K=65536 + 128) == bgt.BGT_ERR_SHAPE
    assert call(alpha=0) == bgt.BGT_ERR_ALPHA
    assert call(alpha=3) == bgt.BGT_ERR_ALPHA
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN
    assert call(qw=MIS) == bgt.BGT_ERR_ALIGN
    assert call(isc=MIS) == bgt.BGT_ERR_ALIGN
    assert call(y=MIS) == bgt.BGT_ERR_ALIGN
    assert call(acc=MIS) == bgt.BGT_ERR_ALIGN
    assert bgt.w8a8_is_kernel_name(4, 4096, 14336) == "k_w8is_split"
    assert bgt.w8a8_is_kernel_name(65, 4096, 14336) == "k_w8is_wide"   # 32 tiles, K split in 8
    assert bgt.w8a8_is_kernel_name(100, 4096, 1024) == "k_w8is_tiled"  # 8 groups: no split
    assert bgt.w8a8_is_kernel_name(0, 4096, 14336) == "invalid shape"
    # dense W4A8: the decode kernel for K of 16 or 32 groups, and for 86 / 112
    # groups with one row block (M <= 16) where 2- or 4-wave workgroups apply
    # (N/16 <= 1024 tiles)
    w4 = bgt.w4a8_kernel_name                       # (M, N, K)
    assert w4(16, 22016, 4096) == "k_w4a8_decode<IS>" and w4(64, 4096, 2048) == "k_w4a8_decode<IS>"
    assert w4(1, 4096, 11008) == "k_w4a8_decode<IS>" and w4(16, 16384, 14336) == "k_w4a8_decode<IS>"
    assert w4(17, 4096, 14336) != "k_w4a8_decode<IS>" and w4(64, 4096, 11008) != "k_w4a8_decode<IS>"
    assert w4(1, 16400, 11008).startswith("k_w4a8_st") or w4(1, 16400, 11008).startswith("k_w4a8_sk")
    assert w4(1, 4096, 12288) != "k_w4a8_decode<IS>"  # 96 groups: not a decode shape
    assert w4(65, 4096, 11008) == "k_w4a8_prefill<4,2,2,2,IS>"
    assert w4(16, 4096, 11008, True) == "k_w4a8_decode<FS>"


def test_gemm_is_noalloc_validation(L):
    g = L.bgt_w4a8_gemm_is_noalloc

    def call(qx=FAKE, sx=FAKE, pk=FAKE, isc=FAKE, alpha=1024, M=512, N=4096, K=4096, y=FAKE, acc=None):
        return g(qx, sx, pk, isc, alpha, M, N, K, y, acc, None)

    assert call(qx=None) == bgt.BGT_ERR_NULL
    assert call(isc=None) == bgt.BGT_ERR_NULL
    assert call(y=None) == bgt.BGT_ERR_NULL
    assert call(M=0) == bgt.BGT_ERR_SHAPE
    assert call(N=24) == bgt.BGT_ERR_SHAPE
    assert call(K=192) == bgt.BGT_ERR_SHAPE
    assert call(alpha=12) == bgt.BGT_ERR_ALPHA
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN
    assert call(acc=MIS) == bgt.BGT_ERR_ALIGN


def test_workspace_bytes():
    # split K of the 256 x 128 tile kernel on 256 CUs: S doubles while
    # tiles * 2S <= 256 and 8S <= K/128
    wb = bgt.w4a8_workspace_bytes                  # (M, N, K)
    assert wb(512, 4096, 4096) == 4 * 512 * 4096 * 4        # 64 tiles -> 4 splits
    assert wb(65, 4096, 4096) == 8 * 65 * 4096 * 4          # 32 tiles -> 8 (4 groups each)
    assert wb(129, 528, 2560) == 4 * 129 * 528 * 4          # 5 tiles, 20 groups -> 4 (5 each)
    assert wb(512, 4096, 11008) == 4 * 512 * 4096 * 4       # 86 groups, uneven parts
    assert wb(100, 256, 512) == 0                           # 4 groups: no split
    assert wb(256, 22016, 4096) == 0                        # 172 tiles
    assert wb(4096, 22016, 4096) == 0 and wb(64, 22016, 4096) == 0   # wide, decode
    # wide launches whose last round goes to the 256 x 128 kernel: its columns
    # (22016 - 85 * 256 = 256 at M = 1536 and 3072: 6 and 12 tiles) split in 8
    assert wb(1536, 22016, 4096) == 8 * 1536 * 256 * 4
    assert wb(3072, 22016, 4096) == 8 * 3072 * 256 * 4
    assert wb(2048, 22016, 4096) == 0                       # no split of the last round
    assert bgt.lib().bgt_w4a8_workspace_bytes(0, 4096, 4096) == bgt.BGT_ERR_SHAPE


def test_prefill_kernel_choice(L):
    # M > 64, N = 22016 on 256 CUs, costs 5 per round of 256 x 256 tiles and 3
    # per round of 256 x 128 ones; a partial last round of 256 x 256 tiles goes
    # to the 256 x 128 kernel (cost 3) when its columns fit one round there:
    # M = 256: 5 vs 3; 512: 5 vs 6; 768: 5+3 vs 9; 1024: 5+3 vs 9;
    # 1536: 10+3 vs 15; 2048: 15 (176 tiles left, 352 of 256 x 128) vs 18;
    # 4096: 25+3 vs 33
    w4 = bgt.w4a8_kernel_name
    wide, tiled = "k_w4a8_wide<IS>", "k_w4a8_prefill<4,2,2,2,IS>"
    try:
        assert [w4(M, 22016, 4096) for M in (256, 512, 768, 1024, 1536, 2048, 4096)] == \
            [tiled, wide, wide, wide, wide, wide, wide]
        assert w4(4096, 256, 4096) == tiled              # 16 vs 32 tiles: one round each
        assert w4(2048, 22016, 4096, True) == "k_w4a8_wide<FS>"
        assert w4(64, 22016, 4096) == "k_w4a8_decode<IS>"     # the decode range is unaffected
        bgt.set_prefill_kernel("wide")
        assert w4(65, 256, 128) == wide and w4(256, 22016, 4096) == wide
        assert w4(16, 22016, 4096) == "k_w4a8_decode<IS>"
        bgt.set_prefill_kernel("tiled")
        assert w4(4096, 22016, 4096) == tiled and w4(4096, 22016, 4096, True) == "k_w4a8_prefill<4,2,2,2,FS>"
        assert L.bgt_set_prefill_kernel(3) == bgt.BGT_ERR_MODE
        assert L.bgt_set_prefill_kernel(-1) == bgt.BGT_ERR_MODE
        with pytest.raises(ValueError):
            bgt.set_prefill_kernel("fast")
    finally:
        bgt.set_prefill_kernel("auto")
    assert w4(256, 22016, 4096) == tiled


def test_moe_validation(L):
    g = L.bgt_w4a8_moe_gemm_is

    def call(qx=FAKE, sx=FAKE, T=16, offs=FAKE, tok=FAKE, E=8, R=32, pk=FAKE, isc=FAKE, width=4,
             alpha=1024, N=64, K=256, y=FAKE, yt=0, acc=None):
        return g(qx, sx, T, offs, tok, E, R, pk, isc, width, alpha, N, K, y, yt, acc, None)

    assert call(qx=None) == bgt.BGT_ERR_NULL
    assert call(offs=None) == bgt.BGT_ERR_NULL
    assert call(tok=None) == bgt.BGT_ERR_NULL
    assert call(pk=None) == bgt.BGT_ERR_NULL
    assert call(width=8) == bgt.BGT_ERR_MODE
    assert call(yt=3) == bgt.BGT_ERR_MODE
    assert call(T=0) == bgt.BGT_ERR_SHAPE
    assert call(E=0) == bgt.BGT_ERR_SHAPE
    assert call(E=257) == bgt.BGT_ERR_SHAPE
    assert call(R=0) == bgt.BGT_ERR_SHAPE
    assert call(R=16 * 8 + 1) == bgt.BGT_ERR_SHAPE
    assert call(N=24) == bgt.BGT_ERR_SHAPE
    assert call(K=192) == bgt.BGT_ERR_SHAPE
    assert call(alpha=12) == bgt.BGT_ERR_ALPHA
    assert call(qx=MIS) == bgt.BGT_ERR_ALIGN
    assert call(pk=MIS) == bgt.BGT_ERR_ALIGN
    assert call(isc=MIS) == bgt.BGT_ERR_ALIGN
    assert call(y=MIS) == bgt.BGT_ERR_ALIGN
    assert call(acc=MIS) == bgt.BGT_ERR_ALIGN
    dec, til = "k_w4a8_decode<IS,grouped>", "k_w4a8_prefill<4,2,2,2,IS,grouped>"
    wide = "k_w4a8_wide<IS,grouped>"
    name = bgt.w4a8_moe_kernel_name                 # (T, E, R, K)
    assert name(16, 8, 32, 4096) == dec
    assert name(64, 8, 128, 14336) == dec
    assert name(16, 8, 32, 1152) == wide                # 9 groups: no decode kernel
    # Mixtral-8x7B top-2: at most two row passes of 64 slots (w1, 32 groups) or
    # three of 32 (w2, 112 groups) for the mean expert, T <= 1024; past that
    # 256 x 256 tiles at 32 groups or fewer, 256 x 128 at 112
    assert name(512, 8, 1024, 4096) == dec and name(520, 8, 1040, 4096) == wide
    assert name(384, 8, 768, 14336) == dec and name(448, 8, 896, 14336) == til
    assert name(1024, 8, 2048, 4096) == wide and name(1024, 8, 2048, 14336) == til
    assert name(1025, 8, 2050, 4096) == wide and name(4096, 8, 8192, 14336) == til
    assert name(1024, 256, 2048, 4096) == wide          # worst-case grid too large
    try:
        bgt.set_prefill_kernel("tiled")
        assert name(1025, 8, 2050, 4096) == til and name(16, 8, 32, 1152) == til
        bgt.set_prefill_kernel("wide")
        assert name(4096, 8, 8192, 14336) == wide and name(16, 8, 32, 4096) == dec
    finally:
        bgt.set_prefill_kernel("auto")
    assert name(0, 8, 1, 4096) == "invalid shape" and name(4, 8, 33, 4096) == "invalid shape"
    assert name(4, 0, 1, 4096) == "invalid shape" and name(4, 8, 8, 4100) == "invalid shape"

