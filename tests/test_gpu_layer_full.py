"""Full-output parity at the layer's full size (K=4096, N=22016).

The sampled comparisons of the config tests check about 0.01% of the outputs
at M=4096; these compare every accumulator and every output against the
oracle, in the decode regime (M=64: the weight-streaming kernel) and the
prefill regime (M=4096: the 256 x 256 tile kernel, its XCD-ordered grid of
1376 tiles), integer-scale and float-scale. The oracle takes tens of seconds
at M=4096 on a many-core host, hence the longer time limit.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


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
def layer(orc):
    x, w = synth.layer_inputs(0, M=4096)
    ow = orc.pack_weights(w, 128, 1024)
    return x, ow


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run(bgt, orc, dev, x, ow, fs):
    M, K = x.shape
    N = ow["iscale"].shape[1]
    oq, os_ = orc.quant_sym_i8(x)
    qx, sx = to_dev(oq, dev), to_dev(os_, dev)
    packed = to_dev(ow["packed"], dev)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    if fs:
        bgt.w4a8_gemm_fs(qx, sx, packed, to_dev(ow["fscale"], dev), N, y=y)
        oy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"])
        got = y.cpu().numpy()
        assert not np.isnan(got).any()
        np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))
        return
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(qx, sx, packed, to_dev(ow["iscale"], dev), 1024, N, y=y, acc_out=acc)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got.view(np.int32), oy.astype(np.float32).view(np.int32))


@pytest.mark.timeout(300)
def test_full_decode_m64(bgt, orc, dev, layer):
    x, ow = layer
    say("full output M=64 K=4096 N=22016 (IS), kernel", bgt.w4a8_kernel_name(64, 22016, 4096))
    run(bgt, orc, dev, np.ascontiguousarray(x[:64]), ow, fs=False)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fs", [False, True])
def test_full_prefill_m4096(bgt, orc, dev, layer, fs):
    x, ow = layer
    say(f"full output M=4096 K=4096 N=22016 ({'FS' if fs else 'IS'}), kernel",
        bgt.w4a8_kernel_name(4096, 22016, 4096, fs))
    run(bgt, orc, dev, x, ow, fs=fs)
