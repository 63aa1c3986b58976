"""GPU parity of the narrow integer-scale storage through the C ABI.

bgt_narrow_iscale must store the oracle's values bit-exactly and refuse any
value that does not fit; bgt_w4a8_gemm_is_narrow with 1-, 2- and 4-byte
scales must give the oracle's int32 accumulators and fp32 outputs bit-exactly
on every kernel path (one-wave-per-tile decode kernel for K of 16 or 32
groups, stream / skinny kernels for other K at M <= 64, the tiled kernel for
M > 64), with ragged rows and column tiles.
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


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def say(*a):
    print(*a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_narrow_iscale_matches_oracle(bgt, orc, dev):
    rng = np.random.default_rng(5)
    for width, top in ((1, 255), (2, 65535)):
        say(f"narrow_iscale width={width}")
        isc = rng.integers(0, top + 1, size=(7, 400), dtype=np.int64).astype(np.int32)
        isc[0, 0], isc[0, 1] = 0, top
        ref, bad = orc.narrow_iscale(isc, width)
        assert bad == 0
        got = bgt.narrow_iscale(to_dev(isc, dev), width).cpu().numpy()
        assert got.dtype == ref.dtype
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("width,value", [(1, 256), (1, -1), (2, 65536), (2, -3)])
def test_narrow_iscale_range_error(bgt, orc, dev, width, value):
    say(f"narrow_iscale range error width={width} value={value}")
    isc = np.full((4, 32), 7, np.int32)
    isc[2, 5] = value
    _, bad = orc.narrow_iscale(isc, width)
    assert bad == 1
    out_dt = torch.uint8 if width == 1 else torch.uint16
    out = torch.full((4, 32), 9, dtype=out_dt, device=dev)
    with pytest.raises(bgt.BgtError) as e:
        bgt.narrow_iscale(to_dev(isc, dev), width, out=out)
    assert e.value.status == bgt.BGT_ERR_RANGE
    assert (out.cpu().numpy() == 9).all(), "a refused call must write nothing"


def _case(orc, dev, seed, M, K, N, alpha):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, alpha)
    return oq, os_, ow


NARROW_SHAPES = [(1, 2048, 64), (5, 4096, 48), (33, 4096, 80), (64, 2048, 160),   # decode
                 (2, 2048, 16400), (20, 2048, 24592),                             # 6, 8 waves
                 (3, 11008, 48), (16, 14336, 32),                                 # 86, 112 groups
                 (3, 384, 48), (17, 512, 64), (40, 1152, 32),                     # stream / skinny
                 (65, 512, 144), (200, 640, 400), (257, 256, 528)]                # tiled


@pytest.mark.parametrize("M,K,N", NARROW_SHAPES)
@pytest.mark.parametrize("width", [1, 2, 4])
def test_w4a8_is_narrow(bgt, orc, dev, width, M, K, N):
    # alpha 2^14 pushes the integer scales past 8 bits for the 16-bit case
    alpha = 1024 if width != 2 else 1 << 14
    say(f"w4a8_gemm_is_narrow width={width} alpha={alpha} M={M} K={K} N={N}")
    oq, os_, ow = _case(orc, dev, 31 * M + K + N, M, K, N, alpha)
    if width == 2:
        assert ow["iscale"].max() > 255, "the 16-bit case must need more than 8 bits"
    if width == 4:
        isc = to_dev(ow["iscale"], dev)
    else:
        isc = bgt.narrow_iscale(to_dev(ow["iscale"], dev), width)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is_narrow(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev), isc,
                            alpha, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], alpha)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))


def test_w4a8_is_narrow_decode_layer_sampled(bgt, orc, dev):
    """The K=4096, N=22016 layer at M=16 with 1-byte scales, in the launch the
    decode bench times; sampled output columns against the oracle."""
    M, K, N = 16, synth.K_LAYER, synth.N_LAYER
    say(f"w4a8_gemm_is_narrow width=1 layer M={M} K={K} N={N} (sampled)")
    x, w = synth.layer_inputs(0, M=M, K=K, N=N)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, 1024)
    assert ow["iscale"].max() <= 255
    isc = bgt.narrow_iscale(to_dev(ow["iscale"], dev), 1)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    bgt.w4a8_gemm_is_narrow(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev), isc,
                            1024, N, y=y)
    cols = np.unique(np.concatenate([np.arange(0, 64), np.arange(N - 64, N),
                                     np.random.default_rng(3).choice(N, 500, replace=False)]))
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024, cols=cols)
    assert ov == 0
    got = y.cpu().numpy()[:, cols]
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))


def test_w4a8_is_narrow_bad_width(bgt, dev):
    M, K, N = 2, 128, 16
    qx = torch.zeros((M, K), dtype=torch.int8, device=dev)
    sx = torch.ones(M, dtype=torch.float32, device=dev)
    packed = torch.zeros(N * K // 2, dtype=torch.uint8, device=dev)
    isc = torch.zeros((1, N), dtype=torch.int8, device=dev)
    with pytest.raises(TypeError):
        bgt.w4a8_gemm_is_narrow(qx, sx, packed, isc, 1024, N)
