"""GPU parity of the fine-grained W8A8 integer-scale path through the C ABI.

bgt_pack_weights_int8 must give the oracle's codes in the int8 fragment
layout, its float and integer scales and its amplifier, bit-exactly.
bgt_w8a8_gemm_is must give the oracle's int32 accumulators (mod 2^32) and
outputs bit-exactly on both kernels (split: M <= 64; tiled: M > 64), with
ragged rows and column tiles, 1-, 2- and 4-byte scales and fp16 / bf16
outputs, and at the LLaMA-3-8B down-projection shape (K = 14336, N = 4096)
on sampled outputs.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# int8 weights: group scales 127/7 times smaller than int4 ones; at 2^16 the
# integer scales fit 16 bits, nearly all of them 8 bits
ALPHA = 1 << 16


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


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def dev_bits16(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("K,N,alpha", [(128, 16, ALPHA), (384, 48, 0), (4096, 208, ALPHA),
                                       (1152, 64, 1024)])
def test_pack_int8_matches_oracle(bgt, orc, dev, K, N, alpha):
    say(f"pack_weights_int8 K={K} N={N} alpha={alpha}")
    w = synth.weights(K + N, K, N, std=0.02, outlier_prob=0.001)
    w[:128, 3] = 0.0                                  # one all-zero group
    ref = orc.pack_weights_int8(w, 128, alpha)
    got = bgt.pack_weights_int8(to_dev(w, dev), alpha=alpha)
    assert got["alpha"] == ref["alpha"]
    np.testing.assert_array_equal(got["qw"].cpu().numpy(), ref["qw"])
    np.testing.assert_array_equal(got["fscale"].cpu().numpy().view(np.int32),
                                  ref["fscale"].view(np.int32))
    np.testing.assert_array_equal(got["iscale"].cpu().numpy(), ref["iscale"])


def test_pack_int8_range_error(bgt, dev):
    say("pack_weights_int8 range error")
    w = np.full((128, 16), 100.0, np.float32)        # s = 100/127, s * 2^24 >= 2^23
    with pytest.raises(bgt.BgtError) as e:
        bgt.pack_weights_int8(to_dev(w, dev), alpha=1 << 24)
    assert e.value.status == bgt.BGT_ERR_RANGE


def test_pack_int8_overflow_warning(bgt, dev):
    say("pack_weights_int8 accumulator warning")
    # s = 1/127 -> iscale 129 at 2^14; 2064512 * 16 * 129 >= 2^31, but not for int4's bound
    w = np.full((2048, 16), 1.0, np.float32)
    pw = bgt.pack_weights_int8(to_dev(w, dev), alpha=1 << 14)
    assert pw["status"] == bgt.BGT_WARN_ACC_MAY_OVERFLOW
    assert 113792 * 16 * 129 < 2 ** 31 <= 2064512 * 16 * 129
    ok = bgt.pack_weights_int8(to_dev(np.full((128, 16), 1.0, np.float32), dev), alpha=1 << 14)
    assert ok["status"] == bgt.BGT_OK                 # one group: 2064512 * 129 < 2^31


def _case(orc, seed, M, K, N, alpha=ALPHA):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    return oq, os_, orc.pack_weights_int8(w, 128, alpha)


SHAPES = [(1, 128, 16), (1, 4096, 64), (3, 384, 48), (16, 1152, 96), (5, 14336, 32),   # split
          (17, 2048, 80), (33, 512, 144), (64, 4096, 16), (40, 256, 208),
          (65, 512, 144), (128, 4096, 64), (200, 640, 400), (257, 256, 16),          # tiled
          (96, 14336, 48), (130, 1280, 80),
          (1024, 512, 4096), (1000, 384, 4000), (1100, 4096, 2048),               # wide
          (20, 4096, 96), (40, 4480, 64), (33, 8192, 160), (64, 14336, 32),        # split, 2 tiles
          (17, 4096, 4096), (17, 32768, 32)]                       # over parts (2 .. 8 parts)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8is_gemm(bgt, orc, dev, M, K, N):
    say(f"w8a8_gemm_is {bgt.w8a8_is_kernel_name(M, N, K)} M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, 13 * M + K + N, M, K, N)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev),
                     to_dev(ow["iscale"], dev), ALPHA, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], ALPHA)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("M,K,N", [(2, 2048, 64), (20, 384, 48), (70, 1024, 80), (300, 256, 144),
                                   (24, 4096, 64), (60, 8192, 32)])
@pytest.mark.parametrize("width", [1, 2])
def test_w8is_narrow_scales(bgt, orc, dev, width, M, K, N):
    # width 1: alpha 2^14 keeps every integer scale below 2^8; width 2: alpha
    # 2^18 pushes some past 8 bits
    alpha = 1 << 14 if width == 1 else 1 << 18
    say(f"w8a8_gemm_is width={width} alpha={alpha} M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, 17 * M + K, M, K, N, alpha)
    if width == 1:
        assert ow["iscale"].max() <= 255
    else:
        assert 255 < ow["iscale"].max() <= 65535
    isc = bgt.narrow_iscale(to_dev(ow["iscale"], dev), width)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev), isc, alpha, N,
                         acc_out=acc)
    oA, oy, ov = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], alpha)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.int32), oy.astype(np.float32).view(np.int32))


# (M, K, N): the 256 x 128 tiles fill at most half of the CUs, so the groups
# split in S parts (65 x 4096: 4 parts of 8 groups; 3200: 25 groups in parts
# of 12 and 13; 14336: 8 parts of 14) whose int32 sums a second kernel adds
@pytest.mark.parametrize("M,K,N", [(65, 4096, 4096), (300, 3200, 528), (512, 14336, 1024)])
def test_w8is_split_k(bgt, orc, dev, M, K, N):
    assert bgt.w8a8_is_kernel_name(M, N, K) == "k_w8is_wide"
    say(f"w8a8_gemm_is split K M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, 7 * M + K, M, K, N)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev),
                     to_dev(ow["iscale"], dev), ALPHA, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], ALPHA)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))
    isc = bgt.narrow_iscale(to_dev(ow["iscale"], dev), 2)
    yb = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev), isc, ALPHA, N,
                          out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(dev_bits16(yb), orc.f32_to_bf16_bits(oy.astype(np.float32)))


@pytest.mark.parametrize("width", [1, 2])
def test_w8is_wide_narrow_scales(bgt, orc, dev, width):
    M, K, N = 1000, 256, 4000
    alpha = 1 << 14 if width == 1 else 1 << 18
    assert bgt.w8a8_is_kernel_name(M, N, K) == "k_w8is_wide"
    say(f"w8a8_gemm_is wide width={width} M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, 23 + width, M, K, N, alpha)
    isc = bgt.narrow_iscale(to_dev(ow["iscale"], dev), width)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev), isc, alpha, N,
                         acc_out=acc, out_dtype=torch.bfloat16)
    oA, oy, _ = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], alpha)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    np.testing.assert_array_equal(dev_bits16(y), orc.f32_to_bf16_bits(oy.astype(np.float32)))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N", [(4, 2048, 48), (100, 512, 80), (40, 4096, 64)])
def test_w8is_half_outputs(bgt, orc, dev, kind, M, K, N):
    say(f"w8a8_gemm_is y={kind} M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, 19 * M + K, M, K, N)
    dt = torch.float16 if kind == "f16" else torch.bfloat16
    y = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev),
                         to_dev(ow["iscale"], dev), ALPHA, N, out_dtype=dt)
    _, oy, _ = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], ALPHA)
    oy = oy.astype(np.float32)
    want = oy.astype(np.float16).view(np.uint16) if kind == "f16" else orc.f32_to_bf16_bits(oy)
    np.testing.assert_array_equal(dev_bits16(y), want)


@pytest.mark.parametrize("m,N", [(3, 32), (70, 32), (1100, 4000)])
def test_w8is_wraps_like_the_oracle(bgt, orc, dev, m, N):
    # extreme codes and scales: A leaves int32; device and oracle agree mod 2^32
    K = 1024
    qx = np.full((m, K), 127, np.int8)
    qx[1::3] = -127
    codes = np.full((K, N), 127, np.int8)
    isc = np.full((K // 128, N), 3000, np.int32)
    sx = np.ones(m, np.float32)
    say(f"w8a8_gemm_is wrap-around {bgt.w8a8_is_kernel_name(m, N, K)} M={m} N={N}")
    oA, oy, ov = orc.w8a8_gemm_is(qx, sx, codes, isc, 1)
    assert ov == m * N
    acc = torch.zeros((m, N), dtype=torch.int32, device=dev)
    y = bgt.w8a8_gemm_is(to_dev(qx, dev), to_dev(sx, dev), to_dev(orc.layout_int8(codes), dev),
                         to_dev(isc, dev), 1, N, acc_out=acc)
    wrapped = ((oA + 2 ** 31) % 2 ** 32) - 2 ** 31
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), wrapped)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.int32), oy.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("M", [16, 64, 4096])
def test_w8is_down_proj_sampled(bgt, orc, dev, M):
    """The LLaMA-3-8B down projection (K = 14336, N = 4096), packed on the GPU
    (layout and scales checked whole), in the launch the bench times; sampled
    rows and columns of y against the oracle."""
    K, N = 14336, 4096
    say(f"w8a8_gemm_is down_proj M={M} K={K} N={N} (sampled)")
    x = synth.activations(900 + M, M, K)
    w = synth.weights(901, K, N, std=0.02, outlier_prob=0.001)
    ref = orc.pack_weights_int8(w, 128, ALPHA)
    got = bgt.pack_weights_int8(to_dev(w, dev), alpha=ALPHA)
    np.testing.assert_array_equal(got["qw"].cpu().numpy(), ref["qw"])
    np.testing.assert_array_equal(got["iscale"].cpu().numpy(), ref["iscale"])
    oq, os_ = orc.quant_sym_i8(x)
    y = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), got["qw"], got["iscale"], ALPHA, N)
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, min(M, 24), replace=False)]))
    cols = np.unique(np.concatenate([np.arange(0, 32), np.arange(N - 32, N),
                                     g.choice(N, 200, replace=False)]))
    _, oy, ov = orc.w8a8_gemm_is(oq, os_, ref["codes"], ref["iscale"], ALPHA, rows=rows, cols=cols)
    assert ov == 0
    got_y = y.cpu().numpy()[np.ix_(rows, cols)]
    np.testing.assert_array_equal(got_y.view(np.int32), oy.astype(np.float32).view(np.int32))
