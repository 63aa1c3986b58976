"""GPU parity of the split-K path of the 256 x 128 tile W4A8 kernel.

With few tiles (M > 64, tiles filling at most half of the CUs) the
integer-scale GEMM splits the groups into S parts whose int32 sums a second
kernel adds (exact mod 2^32), then converts once per output. Cases: S = 2, 4
and 8, parts of unequal group counts (K = 11008: 86 groups), ragged rows,
narrow integer scales, fp16 / bf16 outputs, int32 wrap-around, and the
float-scale control on the same shapes (it runs unsplit). Every output is
compared bit for bit with the oracle; outputs start as NaN.
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
    bit_gemm_token_amd.set_prefill_kernel("auto")
    return bit_gemm_token_amd


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def assert_bits(got, ref, what):
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    assert not np.isnan(got).any(), f"{what}: unwritten (NaN) outputs"
    bad = got.view(np.int32) != ref.view(np.int32)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs differ, first at {np.argwhere(bad)[0]}"


def case(orc, dev, seed, M, K, N):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, 1024)
    d = dict(qx=to_dev(oq, dev), sx=to_dev(os_, dev), packed=to_dev(ow["packed"], dev),
             iscale=to_dev(ow["iscale"], dev), fscale=to_dev(ow["fscale"], dev))
    return oq, os_, ow, d


# (M, K, N, splits on 256 CUs)
SHAPES = [
    (65, 4096, 4096, 8),       # 32 tiles, 4 groups per part
    (512, 4096, 4096, 4),      # the 4096 x 4096 linears of a decoder block at M = 512
    (300, 11008, 4096, 4),     # 86 groups: parts of 21 and 22
    (129, 2560, 528, 4),       # 5 groups per part, ragged rows and columns
    (1000, 1024, 2048, 2),     # 8 groups: 2 parts
]


@pytest.mark.parametrize("M,K,N,S", SHAPES)
def test_splitk_is(bgt, orc, dev, M, K, N, S):
    say(f"split-K w4a8_gemm_is M={M} K={K} N={N} S={S}")
    assert bgt.w4a8_kernel_name(M, N, K) == "k_w4a8_prefill<4,2,2,2,IS>"
    assert bgt.w4a8_workspace_bytes(M, N, K) == S * M * N * 4
    oq, os_, ow, d = case(orc, dev, 5 * M + K + N, M, K, N)
    y = torch.full((M, N), float("nan"), device=dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_bits(y.cpu().numpy(), oy, "y_is")
    # the float-scale control on the same shape (unsplit)
    yf = torch.full((M, N), float("nan"), device=dev)
    bgt.w4a8_gemm_fs(d["qx"], d["sx"], d["packed"], d["fscale"], N, y=yf)
    assert_bits(yf.cpu().numpy(), orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"]), "y_fs")


@pytest.mark.parametrize("width", [1, 2])
def test_splitk_narrow_scales(bgt, orc, dev, width):
    M, K, N = 129, 2560, 528
    say(f"split-K narrow iscale width={width} M={M} K={K} N={N}")
    oq, os_, ow, d = case(orc, dev, 31 + width, M, K, N)
    isc = bgt.narrow_iscale(d["iscale"], width)
    y = torch.full((M, N), float("nan"), device=dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is_narrow(d["qx"], d["sx"], d["packed"], isc, 1024, N, y=y, acc_out=acc)
    oA, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    assert_bits(y.cpu().numpy(), oy, "y_narrow")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_splitk_half_outputs(bgt, orc, dev, kind):
    M, K, N = 200, 2048, 1024
    assert bgt.w4a8_workspace_bytes(M, N, K) > 0
    say(f"split-K half output {kind} M={M} K={K} N={N}")
    oq, os_, ow, d = case(orc, dev, 77, M, K, N)
    dt = torch.float16 if kind == "f16" else torch.bfloat16
    y = torch.full((M, N), float("nan"), dtype=dt, device=dev)
    bgt.w4a8_gemm_is_narrow(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y)
    _, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    oy = oy.astype(np.float32)
    want = oy.astype(np.float16).view(np.uint16) if kind == "f16" else orc.f32_to_bf16_bits(oy)
    np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_splitk_overflow_wraps_like_oracle(bgt, orc, dev):
    M, K, N = 256, 4096, 256
    assert bgt.w4a8_workspace_bytes(M, N, K) > 0
    say(f"split-K int32 wrap M={M} K={K} N={N}")
    qx = np.full((M, K), 127, np.int8)
    qx[:, ::3] = -127
    qx[::7] = -qx[::7]
    codes = np.full((K, N), 7, np.int8)
    codes[::5] = -8
    isc = np.full((K // 128, N), (1 << 23) - 1, np.int32)
    isc[:, ::2] = 300
    sx = np.full(M, 0.01, np.float32)
    packed = orc.pack_int4(codes)
    y = torch.full((M, N), float("nan"), device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(to_dev(qx, dev), to_dev(sx, dev), to_dev(packed, dev), to_dev(isc, dev), 1024,
                     N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(qx, sx, codes, isc, 1024)
    assert ov > 0
    wrapped = ((oA + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int64)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), wrapped)
    assert_bits(y.cpu().numpy(), oy, "y_wrap")


def test_splitk_shapes_in_sequence(bgt, orc, dev):
    # the workspace grows from a small split to a larger one and is reused
    for M, K, N in [(100, 1024, 256), (512, 4096, 4096), (100, 1024, 256)]:
        say(f"split-K sequence M={M} K={K} N={N}")
        oq, os_, ow, d = case(orc, dev, M + K + N, M, K, N)
        y = torch.full((M, N), float("nan"), device=dev)
        bgt.w4a8_gemm_is(d["qx"], d["sx"], d["packed"], d["iscale"], 1024, N, y=y)
        _, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
        assert_bits(y.cpu().numpy(), oy, "y_seq")
