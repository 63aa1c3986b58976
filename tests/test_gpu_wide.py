"""GPU parity of the large-M W4A8 kernel (256 x 256 output tiles) against the oracle.

The module forces that kernel for every M > 64 (bgt_set_prefill_kernel), so
small shapes reach it too. Shapes with more tiles than one round of CUs and a
partial last round run the 256 x 256 kernel on the columns of the full rounds
and the 256 x 128 kernel on the rest (row stride N in both; the rest split in
K when its tiles are few). Cases span several tiles with ragged rows and
ragged column tiles (N not a multiple of 256, down to one 16-column tile),
group counts of 1, 2, 3, 5 and 32 (the pipeline's three stages wrap at
different points), integer scales of 4, 2 and 1 bytes, the float-scale
control, fp16 / bf16 outputs, and int32 wrap-around of the accumulator. Every
output is compared bit for bit; outputs start as NaN so unwritten ones show.
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
    bit_gemm_token_amd.set_prefill_kernel("wide")
    yield bit_gemm_token_amd
    bit_gemm_token_amd.set_prefill_kernel("auto")


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def nan_like(shape, dev, dtype=None):
    return torch.full(shape, float("nan"), dtype=dtype or torch.float32, device=dev)


def assert_bits(got, ref, what):
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    assert not np.isnan(got).any(), f"{what}: unwritten (NaN) outputs"
    bad = got.view(np.int32) != ref.view(np.int32)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs differ, first at {np.argwhere(bad)[0]}"


def case(orc, dev, seed, M, K, N, alpha=1024):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, alpha)
    d = dict(qx=to_dev(oq, dev), sx=to_dev(os_, dev), packed=to_dev(ow["packed"], dev),
             iscale=to_dev(ow["iscale"], dev), fscale=to_dev(ow["fscale"], dev))
    return oq, os_, ow, d


SHAPES = [
    (1024, 128, 256),      # one group, one column tile, 4 row tiles
    (1024, 256, 512),      # two groups
    (1100, 384, 272),      # three groups; ragged rows and a 16-column ragged tile
    (1300, 640, 16),       # five groups; a single 16-column tile
    (2048, 4096, 48),      # the full 32 groups; 48 columns (tiles past N clamp)
    (1031, 512, 784),      # ragged rows and columns together
    (1536, 1024, 1024),    # whole tiles only
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_wide_is(bgt, orc, dev, M, K, N):
    say(f"wide w4a8_gemm_is M={M} K={K} N={N}")
    assert bgt.w4a8_kernel_name(M, N, K).startswith("k_w4a8_wide")
    oq, os_, ow, d = case(orc, dev, 7 * M + K + N, M, K, N)
    y = nan_like((M, N), dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_bits(y.cpu().numpy(), oy, "y_is")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_wide_fs(bgt, orc, dev, M, K, N):
    say(f"wide w4a8_gemm_fs M={M} K={K} N={N}")
    assert bgt.w4a8_kernel_name(M, N, K, True).startswith("k_w4a8_wide")
    oq, os_, ow, d = case(orc, dev, 7 * M + K + N, M, K, N)
    y = nan_like((M, N), dev)
    bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], N, y=y)
    oy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"])
    assert_bits(y.cpu().numpy(), oy, "y_fs")


@pytest.mark.parametrize("width", [1, 2])
@pytest.mark.parametrize("M,K,N", [(1100, 384, 272), (1024, 4096, 528)])
def test_wide_narrow_scales(bgt, orc, dev, M, K, N, width):
    say(f"wide narrow iscale width={width} M={M} K={K} N={N}")
    oq, os_, ow, d = case(orc, dev, 11 * M + K + N + width, M, K, N)
    isc = bgt.narrow_iscale(d["iscale"], width)
    y = nan_like((M, N), dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is_narrow(d["qx"], d["sx"], d["packed"], isc, 1024, N, y=y, acc_out=acc)
    oA, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_bits(y.cpu().numpy(), oy, "y_narrow")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_wide_half_outputs(bgt, orc, dev, kind):
    M, K, N = 1100, 512, 272
    say(f"wide half output {kind} M={M} K={K} N={N}")
    oq, os_, ow, d = case(orc, dev, 99, M, K, N)
    dt = torch.float16 if kind == "f16" else torch.bfloat16
    y = nan_like((M, N), dev, dt)
    bgt.w4a8_gemm_is_narrow(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y)
    _, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    oy = oy.astype(np.float32)
    want = oy.astype(np.float16).view(np.uint16) if kind == "f16" else orc.f32_to_bf16_bits(oy)
    np.testing.assert_array_equal(bits, want)
    yf = nan_like((M, N), dev, dt)
    bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], N, y=yf)
    ofy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"]).astype(np.float32)
    bits = yf.view(torch.int16).cpu().numpy().view(np.uint16)
    want = ofy.astype(np.float16).view(np.uint16) if kind == "f16" else orc.f32_to_bf16_bits(ofy)
    np.testing.assert_array_equal(bits, want)


def test_wide_overflow_wraps_like_oracle(bgt, orc, dev):
    M, K, N = 1024, 4096, 48
    say(f"wide int32 wrap M={M} K={K} N={N}")
    qx = np.full((M, K), 127, np.int8)
    qx[:, ::3] = -127
    qx[::7] = -qx[::7]
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
    assert_bits(y.cpu().numpy(), oy, "y_wrap")


# (M, K, N, columns of the 256 x 256 launch) on 256 CUs
SPLIT_SHAPES = [
    (1024, 256, 16640, 16384),     # 260 tiles: 64 column tiles wide, 256 columns left
    (1031, 1024, 16400, 13056),    # 325 tiles, ragged rows; 3344 columns left, ragged
    (1024, 1024, 16640, 16384),    # the 8 tiles left split K in 2
]


@pytest.mark.parametrize("M,K,N,NW", SPLIT_SHAPES)
def test_wide_last_round_split(bgt, orc, dev, M, K, N, NW):
    say(f"wide + last round M={M} K={K} N={N} (wide columns {NW})")
    assert bgt.w4a8_kernel_name(M, N, K).startswith("k_w4a8_wide")
    oq, os_, ow, d = case(orc, dev, 3 * M + K + N, M, K, N)
    y = nan_like((M, N), dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_bits(y.cpu().numpy(), oy, "y_is")
    yf = nan_like((M, N), dev)
    bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], N, y=yf)
    assert_bits(yf.cpu().numpy(), orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"]), "y_fs")
    isc = bgt.narrow_iscale(d["iscale"], 2)
    yn = nan_like((M, N), dev, torch.bfloat16)
    bgt.w4a8_gemm_is_narrow(d["qx"], d["sx"], d["packed"], isc, 1024, N, y=yn)
    want = orc.f32_to_bf16_bits(oy.astype(np.float32))
    np.testing.assert_array_equal(yn.view(torch.int16).cpu().numpy().view(np.uint16), want)
