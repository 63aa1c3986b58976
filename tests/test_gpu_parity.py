"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

The bar: bit-exact on every integer quantity (codes, packed bytes, integer
scales, int32 accumulators, zero points, row sums) and on the float scales;
the fp32 outputs are compared bit-exactly as well (both sides perform the same
IEEE operations in the same order), which is tighter than the 1-ulp tolerance
of the target. Outputs are pre-filled with NaN so unwritten elements show.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def bgt():
    import bit_gemm_token_amd
    bit_gemm_token_amd.lib()
    return bit_gemm_token_amd


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def nan_like(shape, dev):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=dev)


def ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def assert_f32_exact(got, ref, what):
    assert not np.isnan(got).any(), f"{what}: unwritten (NaN) outputs"
    d = ulp_diff(np.ascontiguousarray(got, np.float32), np.ascontiguousarray(ref, np.float32))
    assert d.max() == 0, f"{what}: max ulp diff {d.max()} at {np.unravel_index(d.argmax(), d.shape)}"


# ----------------------------------------------------------------- quantize_act

# rows held in 4 register slots per thread (K <= 4096), in 16 (K <= 16384, the
# last one partial at 4160 and 11008), and past 16384 (the rest streamed again)
@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (16, 4096), (33, 512), (5, 11008), (2, 16384),
                                 (7, 100), (4, 4097), (3, 4160), (2, 20480), (3, 32768)])
def test_quantize_sym(bgt, orc, dev, M, K):
    say(f"quantize_act sym M={M} K={K}")
    x = synth.activations(M + K, M, K)
    x[0, :5] = [0.5, -0.5, 2.5, -2.5, 1e-3]
    if M > 2:
        x[2] = 0.0                       # zero row
    q, s, rs = bgt.quantize_act(to_dev(x, dev), want_rowsum=True)
    oq, os_ = orc.quant_sym_i8(x)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(rs.cpu().numpy(), oq.astype(np.int64).sum(1))


def test_quantize_sym_strided_rows(bgt, orc, dev):
    say("quantize_act sym with ld > cols")
    big = synth.activations(5, 6, 1040)
    xd = to_dev(big, dev)[:, :1024]
    q, s, _ = bgt.quantize_act(xd)
    oq, os_ = orc.quant_sym_i8(np.ascontiguousarray(big[:, :1024]))
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)


def test_quantize_sym_ties_exact(bgt, orc, dev):
    say("quantize_act sym ties")
    x = np.zeros((2, 128), np.float32)
    x[0, :7] = [127.0, 0.5, -0.5, 2.5, -63.5, 1.49, -126.6]
    g = synth.rng(1, 1)
    x[1] = (g.integers(-254, 255, 128) / 2.0).astype(np.float32)
    x[1, 0] = 127.0
    q, s, _ = bgt.quantize_act(to_dev(x, dev))
    oq, _ = orc.quant_sym_i8(x)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    assert q.cpu().numpy()[0, :7].tolist() == [127, 1, -1, 3, -64, 1, -127]


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_quantize_scale_range(bgt, orc, dev, mode):
    # rows scaled from 2^-120 to 2^120: the quantizer takes x*r corrected by
    # one fma (r = 1/s) for s in [2^-100, 2^100] and the division outside, and
    # must give the division's codes everywhere; rows 0 and 1 put quotients
    # exactly on and one ulp beside half-integers
    say(f"quantize_act {mode} across scales")
    K = 1024
    g = synth.rng(17, 3)
    base = g.standard_normal((24, K)).astype(np.float32)
    base = np.sign(base) * (np.abs(base) + np.float32(0.25))   # |x| >= 2^-122: no subnormal inputs
    base[0] = (g.integers(-254, 255, K) / 2.0).astype(np.float32)
    base[0, 0] = 127.0
    base[1] = np.nextafter(base[0], np.float32(np.inf))
    base[1, 0] = 127.0
    exps = [0, 0, -120, -110, -101, -100, -99, -90, -60, -30, -10, -1, 1, 10, 30, 60, 90, 99, 100, 101,
            110, 115, 120, 5]
    x = np.stack([np.ldexp(base[i], e) for i, e in enumerate(exps)]).astype(np.float32)
    assert np.isfinite(x).all()
    if mode == "sym":
        q, s, _ = bgt.quantize_act(to_dev(x, dev))
        oq, os_ = orc.quant_sym_i8(x)
        np.testing.assert_array_equal(s.cpu().numpy(), os_)
        np.testing.assert_array_equal(q.cpu().numpy(), oq)
    else:
        x[2::2] += np.float32(0.75) * np.abs(x[2::2]).max(1, keepdims=True)
        q, s, z, rs = bgt.quantize_act(to_dev(x, dev), mode="asym")
        oq, os_, oz, ors = orc.quant_asym_u8(x)
        np.testing.assert_array_equal(s.cpu().numpy(), os_)
        np.testing.assert_array_equal(z.cpu().numpy(), oz)
        np.testing.assert_array_equal(q.cpu().numpy(), oq)
        np.testing.assert_array_equal(rs.cpu().numpy(), ors)


@pytest.mark.parametrize("M,K,relu", [(256, 4096, False), (256, 4096, True), (9, 300, False),
                                      (4096, 4096, False), (5, 14336, True), (3, 20480, False)])
def test_quantize_asym(bgt, orc, dev, M, K, relu):
    say(f"quantize_act asym M={M} K={K} relu={relu}")
    x = synth.activations(M, M, K, outlier_frac=0.0, mean=0.5, relu=relu)
    if M > 3:
        x[3] = 1.25                      # degenerate constant row
    q, s, z, rs = bgt.quantize_act(to_dev(x, dev), mode="asym")
    oq, os_, oz, ors = orc.quant_asym_u8(x)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)
    np.testing.assert_array_equal(z.cpu().numpy(), oz)
    np.testing.assert_array_equal(rs.cpu().numpy(), ors)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)


# -------------------------------------------------------------------- packing

@pytest.mark.parametrize("K,N,alpha", [(128, 16, 1024), (512, 48, 1024), (4096, 4096, 1024),
                                       (1024, 272, 0), (11008, 64, 1024), (4096, 22016, 1024)])
def test_pack(bgt, orc, dev, K, N, alpha):
    say(f"pack_weights_int4 K={K} N={N} alpha={alpha}")
    w = synth.weights(K + N, K, N, std=0.02, outlier_prob=0.001)
    w[:128, 1] = 0.0                      # an all-zero group
    pw = bgt.pack_weights_int4(to_dev(w, dev), alpha=alpha)
    ow = orc.pack_weights(w, 128, alpha)
    assert pw["alpha"] == ow["alpha"]
    np.testing.assert_array_equal(pw["fscale"].cpu().numpy(), ow["fscale"])
    np.testing.assert_array_equal(pw["iscale"].cpu().numpy(), ow["iscale"])
    np.testing.assert_array_equal(pw["packed"].cpu().numpy(), ow["packed"])
    assert pw["status"] == 0


def test_pack_search_small_scales(bgt, orc, dev):
    say("pack_weights_int4 amplifier search, tiny weights")
    w = synth.weights(3, 256, 32, std=1e-4)
    pw = bgt.pack_weights_int4(to_dev(w, dev), alpha=0)
    ow = orc.pack_weights(w, 128, 0)
    assert pw["alpha"] == ow["alpha"] and pw["alpha"] > 1024
    np.testing.assert_array_equal(pw["iscale"].cpu().numpy(), ow["iscale"])


def test_pack_range_error(bgt, dev):
    say("pack_weights_int4 range error")
    w = np.full((128, 16), 100.0, np.float32)        # s = 14.3, s * 2^20 >= 2^23
    with pytest.raises(bgt.BgtError) as e:
        bgt.pack_weights_int4(to_dev(w, dev), alpha=1 << 20)
    assert e.value.status == bgt.BGT_ERR_RANGE


def test_pack_overflow_warning(bgt, dev):
    say("pack_weights_int4 accumulator warning")
    w = np.full((4096, 16), 1.0, np.float32)         # s = 1/7 -> iscale 2341 at 2^14; 113792*32*2341 >= 2^31
    pw = bgt.pack_weights_int4(to_dev(w, dev), alpha=1 << 14)
    assert pw["status"] == bgt.BGT_WARN_ACC_MAY_OVERFLOW


# ----------------------------------------------------------------- W4A8 GEMMs

def _w4_case(orc, bgt, dev, seed, M, K, N, alpha=1024):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, alpha)
    d = dict(qx=to_dev(oq, dev), sx=to_dev(os_, dev), packed=to_dev(ow["packed"], dev),
             iscale=to_dev(ow["iscale"], dev), fscale=to_dev(ow["fscale"], dev))
    return oq, os_, ow, d


SHAPES = [(1, 128, 16), (3, 384, 48), (16, 1024, 144), (17, 512, 64), (33, 256, 272),
          (64, 1024, 128), (65, 512, 144), (100, 384, 272), (128, 1024, 256), (200, 640, 400),
          (257, 256, 528),
          # K of 16 or 32 groups with M <= 64: the one-wave-per-tile kernel (ragged rows,
          # row blocks, tile sets with idle waves)
          (1, 2048, 64), (5, 4096, 48), (17, 2048, 96), (33, 4096, 80), (40, 4096, 16),
          (64, 2048, 160),
          # the same kernel with 6 and 8 waves per workgroup (N/16 > 1024 and > 1536 tiles;
          # the last workgroup partly past N)
          (3, 4096, 16400), (20, 2048, 24576), (1, 4096, 24592), (50, 2048, 28672),
          # four row blocks split over two waves per tile on 4- and 6-wave workgroups
          # (the second wave's last block ragged at M = 49, 57, 61)
          (49, 4096, 4096), (57, 2048, 20480), (61, 4096, 16400),
          # one row block, K split over four waves per tile (8 or 4 groups each): one tile
          # per workgroup up to 256 tiles, two above (the last workgroup partly past N at
          # 8176 columns)
          (16, 4096, 4096), (7, 2048, 8192), (12, 4096, 8176), (1, 2048, 16),
          (9, 4096, 4080), (3, 2048, 400),
          # 86 groups (run as 96, the last ten masked) and 112 groups, one row block on 2-wave
          # (N <= 8192) and 4-wave workgroups; more rows take the weight-split kernels
          (1, 11008, 64), (16, 11008, 80), (2, 11008, 8208), (5, 14336, 48), (16, 14336, 4096),
          (17, 11008, 80), (40, 14336, 16)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a8_is_small(bgt, orc, dev, M, K, N):
    say(f"w4a8_gemm_is M={M} K={K} N={N}")
    oq, os_, ow, d = _w4_case(orc, bgt, dev, 10 * M + K + N, M, K, N)
    y = nan_like((M, N), dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_f32_exact(y.cpu().numpy(), oy, "y_is")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a8_fs_small(bgt, orc, dev, M, K, N):
    say(f"w4a8_gemm_fs M={M} K={K} N={N}")
    oq, os_, ow, d = _w4_case(orc, bgt, dev, 10 * M + K + N, M, K, N)
    y = nan_like((M, N), dev)
    bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], N, y=y)
    oy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"])
    assert_f32_exact(y.cpu().numpy(), oy, "y_fs")


@pytest.mark.parametrize("M", [1, 16, 100])
def test_w4a8_is_overflow_wraps_like_oracle(bgt, orc, dev, M):
    say(f"w4a8_gemm_is int32 wrap M={M}")
    K, N = 4096, 32
    qx = np.full((M, K), 127, np.int8)
    qx[:, ::3] = -127
    codes = np.full((K, N), 7, np.int8)
    codes[::5] = -8
    isc = np.full((K // 128, N), (1 << 23) - 1, np.int32)
    isc[:, ::2] = 300
    sx = np.full(M, 0.01, np.float32)
    packed = orc.pack_int4(codes)
    y = nan_like((M, N), dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(to_dev(qx, dev), to_dev(sx, dev), to_dev(packed, dev), to_dev(isc, dev), 1024,
                     N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(qx, sx, codes, isc, 1024)
    assert ov > 0
    wrapped = ((oA + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int64)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), wrapped)
    assert_f32_exact(y.cpu().numpy(), oy, "y_wrap")


def test_w4a8_deterministic(bgt, orc, dev):
    say("w4a8 run-twice determinism")
    for M in (4, 200):
        oq, os_, ow, d = _w4_case(orc, bgt, dev, 77, M, 1024, 256)
        y1 = bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, 256)
        y2 = bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, 256)
        f1 = bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], 256)
        f2 = bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], 256)
        assert torch.equal(y1, y2) and torch.equal(f1, f2)


# ------------------------------------------------------------------ W8A8 ZP

@pytest.mark.parametrize("M,K,N,relu", [(1, 128, 16, False), (37, 384, 80, False), (256, 4096, 4096, False),
                                        (256, 4096, 4096, True), (130, 1024, 208, False),
                                        (65, 2048, 144, False), (64, 4096, 64, True), (3, 896, 48, False)])
def test_w8a8_zp(bgt, orc, dev, M, K, N, relu):
    say(f"w8a8_gemm_zp M={M} K={K} N={N} relu={relu}")
    x, w = synth.w8a8_inputs(M + K, M, K, N, relu=relu)
    xd = to_dev(x, dev)
    wtd = to_dev(np.ascontiguousarray(w.T), dev)
    qx, sx, zx, rx = bgt.quantize_act(xd, mode="asym")
    qw, sw, zw, cw = bgt.quantize_act(wtd, mode="asym")
    oqx, osx, ozx, orx = orc.quant_asym_u8(x)
    oqw, osw, ozw, ocw = orc.quant_asym_u8(np.ascontiguousarray(w.T))
    np.testing.assert_array_equal(qw.cpu().numpy(), oqw)
    np.testing.assert_array_equal(cw.cpu().numpy(), ocw)
    y = nan_like((M, N), dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw, y=y, acc_out=acc)
    if M * N * K > 2 ** 28:
        g = synth.rng(M, 5)
        rows = np.unique(np.r_[0, M - 1, g.integers(0, M, 30)])
        cols = np.unique(np.r_[0, N - 1, g.integers(0, N, 200)])
    else:
        rows, cols = np.arange(M), np.arange(N)
    oA, oy, ov = orc.w8a8_gemm_zp(oqx, osx, ozx, orx, oqw, osw, ozw, ocw, rows=rows, cols=cols)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy()[np.ix_(rows, cols)].astype(np.int64), oA)
    assert_f32_exact(y.cpu().numpy()[np.ix_(rows, cols)], oy, "y_zp")
