"""GPU parity of the fp16 / bf16 activation and output types through the C ABI.

fp16 and bf16 activations are widened exactly, so the codes and scales must
equal the oracle's quantizer on the widened fp32 values; fp16 and bf16
outputs are the fp32 result rounded once to nearest even, so they must equal
the oracle's fp32 output rounded the same way (numpy for fp16, the oracle's
bf16 rounding for bf16), bit for bit, on every kernel path.
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


def half_input(orc, x, kind, dev):
    """(device tensor of x in `kind`, the exactly widened fp32 values)."""
    if kind == "f16":
        h = x.astype(np.float16)
        return to_dev(h, dev), h.astype(np.float32)
    bits = orc.f32_to_bf16_bits(x)
    t = to_dev(bits.view(np.int16), dev).view(torch.bfloat16)
    return t, orc.bf16_bits_to_f32(bits)


def out_bits(orc, y32, kind):
    """Bit patterns of the oracle's fp32 output rounded to `kind`."""
    if kind == "f16":
        return y32.astype(np.float16).view(np.uint16)
    return orc.f32_to_bf16_bits(y32)


def dev_bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


TORCH_T = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", [(3, 4096), (16, 1024), (5, 300)])
def test_quantize_half_inputs(bgt, orc, dev, kind, M, K):
    say(f"quantize_act {kind} M={M} K={K}")
    x, xw = half_input(orc, synth.activations(80 + K, M, K), kind, dev)
    q, s, _ = bgt.quantize_act(x)
    oq, os_ = orc.quant_sym_i8(xw)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.int32), os_.view(np.int32))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_quantize_asym_half_input(bgt, orc, dev, kind):
    M, K = 7, 2048
    say(f"quantize_act asym {kind}")
    x, xw = half_input(orc, synth.activations(90, M, K, outlier_frac=0.0, mean=0.5), kind, dev)
    q, s, z, r = bgt.quantize_act(x, mode="asym")
    oq, os_, oz, orow = orc.quant_asym_u8(xw)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.int32), os_.view(np.int32))
    np.testing.assert_array_equal(z.cpu().numpy(), oz)
    np.testing.assert_array_equal(r.cpu().numpy(), orow)


def _w4_case(orc, seed, M, K, N):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    return oq, os_, orc.pack_weights(w, 128, 1024)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 272), (17, 2048, 96), (3, 384, 48), (300, 512, 208),
                                   (2, 2048, 24592)])
def test_gemm_is_half_outputs(bgt, orc, dev, kind, M, K, N):
    say(f"w4a8_gemm_is y={kind} M={M} K={K} N={N}")
    oq, os_, ow = _w4_case(orc, 7 * M + K + N, M, K, N)
    y = torch.full((M, N), float("nan"), dtype=TORCH_T[kind], device=dev)
    bgt.w4a8_gemm_is_narrow(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev),
                            to_dev(ow["iscale"], dev), 1024, N, y=y)
    _, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(dev_bits(y), out_bits(orc, oy.astype(np.float32), kind))


@pytest.mark.parametrize("M,K,N", [(2, 4096, 64), (80, 512, 144)])
def test_gemm_fs_bf16_output(bgt, orc, dev, M, K, N):
    say(f"w4a8_gemm_fs y=bf16 M={M} K={K} N={N}")
    oq, os_, ow = _w4_case(orc, 5 * M + K, M, K, N)
    y = bgt.w4a8_gemm_fs(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev),
                         to_dev(ow["fscale"], dev), N, out_dtype=torch.bfloat16)
    oy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"])
    np.testing.assert_array_equal(dev_bits(y), out_bits(orc, oy.astype(np.float32), "bf16"))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N,fused", [(3, 4096, 208, True), (1, 2048, 64, True), (20, 2048, 96, False)])
def test_linear_half_io(bgt, orc, dev, kind, M, K, N, fused):
    say(f"w4a8_linear_is x=y={kind} M={M} K={K} N={N} fused={fused}")
    x, xw = half_input(orc, synth.activations(100 + M, M, K), kind, dev)
    w = synth.weights(101 + M, K, N, std=0.02, outlier_prob=0.001)
    ow = orc.pack_weights(w, 128, 1024)
    assert bgt.w4a8_linear_fused(x) == fused
    y, qx, sx = bgt.w4a8_linear_is(x, to_dev(ow["packed"], dev), to_dev(ow["iscale"], dev), 1024, N)
    assert y.dtype == TORCH_T[kind]
    oq, os_ = orc.quant_sym_i8(xw)
    np.testing.assert_array_equal(qx.cpu().numpy(), oq)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.int32), os_.view(np.int32))
    _, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(dev_bits(y), out_bits(orc, oy.astype(np.float32), kind))
