"""GPU parity of bgt_w4a8_linear_is (per-token quantization + integer-scale GEMM).

For M <= 4 on the decode path the decode kernel quantizes the fp32 rows
itself (one launch; the quotient x/s by Markstein's corrected product); every
other case runs the quantizer and the GEMM. Either way the codes, the token
scales and y must equal the oracle's quantizer and GEMM bit-exactly, including
ties at half-integer quotients, zero rows, strided rows and narrow scales.
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


def _weights(orc, seed, K, N):
    w = synth.weights(seed, K, N, std=0.02, outlier_prob=0.001)
    return orc.pack_weights(w, 128, 1024)


def _check(bgt, orc, dev, x, ow, N, width=4, ldx_pad=0, expect_fused=None):
    M, K = x.shape
    if ldx_pad:
        xs = np.zeros((M, K + ldx_pad), np.float32)
        xs[:, :K] = x
        xd = to_dev(xs, dev)[:, :K]
    else:
        xd = to_dev(x, dev)
    isc = to_dev(ow["iscale"], dev)
    if width != 4:
        isc = bgt.narrow_iscale(isc, width)
    if expect_fused is not None:
        assert bgt.w4a8_linear_fused(xd) == expect_fused
    y, qx, sx = bgt.w4a8_linear_is(xd, to_dev(ow["packed"], dev), isc, 1024, N)
    oq, os_ = orc.quant_sym_i8(x)
    np.testing.assert_array_equal(qx.cpu().numpy(), oq)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.int32), os_.view(np.int32))
    _, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1376), (2, 4096, 272), (3, 2048, 528), (4, 4096, 400),
                                   (4, 2048, 16),
                                   # 4, 6 and 8 waves per workgroup (N/16 tiles past 512, 1024,
                                   # 1536); on 6 waves each thread's last group of four row
                                   # elements is partial (K/4 not a multiple of 384)
                                   (2, 4096, 11008), (4, 2048, 8208), (3, 2048, 20480),
                                   (1, 4096, 28672),
                                   # 86 groups (run as 96, the last ten masked) and 112: rows
                                   # staged compactly, 2-wave workgroups splitting K in four
                                   # (N/16 <= 512 tiles) or 8-wave workgroups
                                   (1, 11008, 4096), (4, 11008, 4096), (2, 14336, 4096),
                                   (3, 14336, 528), (1, 11008, 8208), (4, 14336, 16384)])
def test_linear_fused(bgt, orc, dev, M, K, N):
    say(f"w4a8_linear_is fused M={M} K={K} N={N}")
    x = synth.activations(40 + M, M, K)
    _check(bgt, orc, dev, x, _weights(orc, 41 + M, K, N), N, expect_fused=True)


@pytest.mark.parametrize("M,K,N", [(5, 4096, 64), (16, 2048, 96), (65, 512, 144), (2, 1152, 48)])
def test_linear_two_launches(bgt, orc, dev, M, K, N):
    say(f"w4a8_linear_is quantizer+GEMM M={M} K={K} N={N}")
    x = synth.activations(50 + M, M, K)
    _check(bgt, orc, dev, x, _weights(orc, 51 + M, K, N), N, expect_fused=False)


@pytest.mark.parametrize("width", [1, 2])
def test_linear_fused_narrow_scales(bgt, orc, dev, width):
    M, K, N = 3, 4096, 208
    say(f"w4a8_linear_is fused width={width}")
    x = synth.activations(60, M, K)
    _check(bgt, orc, dev, x, _weights(orc, 61, K, N), N, width=width, expect_fused=True)


def test_linear_fused_ties_and_zero_row(bgt, orc, dev):
    # row 0: values at exact half-integer multiples of its scale (s = 1 with
    # max 127) and exact multiples; row 1 all zero; row 2 tiny but normal;
    # row 3 ordinary
    M, K, N = 4, 2048, 64
    say("w4a8_linear_is fused ties / zero row")
    rng = np.random.default_rng(8)
    x = np.zeros((M, K), np.float32)
    k = rng.integers(-127, 127, size=K)
    x[0] = (k + 0.5).astype(np.float32)
    x[0, ::3] = k[::3].astype(np.float32)
    x[0, 7] = 127.0
    x[2] = rng.standard_normal(K).astype(np.float32) * np.float32(1e-30)
    x[3] = synth.activations(62, 1, K)[0]
    _check(bgt, orc, dev, x, _weights(orc, 63, K, N), N, expect_fused=True)


def test_linear_fused_strided_rows(bgt, orc, dev):
    M, K, N = 4, 4096, 96
    say("w4a8_linear_is fused, row stride K+16")
    x = synth.activations(70, M, K)
    _check(bgt, orc, dev, x, _weights(orc, 71, K, N), N, ldx_pad=16, expect_fused=True)


def test_linear_unaligned_rows_take_two_launches(bgt, orc, dev):
    M, K, N = 2, 2048, 48
    say("w4a8_linear_is, row stride K+1 (scalar quantizer path)")
    x = synth.activations(72, M, K)
    _check(bgt, orc, dev, x, _weights(orc, 73, K, N), N, ldx_pad=1, expect_fused=False)


def test_linear_decode_layer_sampled(bgt, orc, dev):
    """The K=4096, N=22016 layer at M=4, fused, in the launch the bench times;
    all codes and scales, sampled output columns."""
    M, K, N = 4, synth.K_LAYER, synth.N_LAYER
    say(f"w4a8_linear_is fused layer M={M} (sampled columns)")
    x, w = synth.layer_inputs(0, M=M, K=K, N=N)
    ow = orc.pack_weights(w, 128, 1024)
    xd = to_dev(x, dev)
    assert bgt.w4a8_linear_fused(xd)
    y, qx, sx = bgt.w4a8_linear_is(xd, to_dev(ow["packed"], dev), to_dev(ow["iscale"], dev), 1024, N)
    oq, os_ = orc.quant_sym_i8(x)
    np.testing.assert_array_equal(qx.cpu().numpy(), oq)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.int32), os_.view(np.int32))
    cols = np.unique(np.concatenate([np.arange(0, 48), np.arange(N - 48, N),
                                     np.random.default_rng(4).choice(N, 400, replace=False)]))
    _, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024, cols=cols)
    assert ov == 0
    got = y.cpu().numpy()[:, cols]
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))
