"""GPU parity of the canonical int4 layout entry point against the oracle.

Codes packed by the oracle into the canonical layout (W^T, K contiguous, even
k in the low nibble) are rewritten by bgt_repack_int4_canonical; the result
must equal, byte for byte, the oracle's own packing of the same codes into the
kernel-native layout, and a GEMM on it must give the oracle's outputs.
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


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 48), (640, 80), (4096, 528), (11008, 64)])
def test_repack_matches_native_packing(bgt, orc, dev, K, N):
    print(f"repack canonical K={K} N={N}", flush=True)
    g = synth.rng(K + N, 7)
    codes = g.integers(-8, 8, size=(K, N)).astype(np.int8)
    can = orc.pack_int4_canonical(codes)
    packed = bgt.repack_int4_canonical(to_dev(can, dev), K, N)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy(), orc.pack_int4(codes))


def test_repack_then_gemm(bgt, orc, dev):
    M, K, N = 40, 4096, 272
    print(f"repack canonical then w4a8_gemm_is M={M} K={K} N={N}", flush=True)
    x = synth.activations(3, M, K)
    w = synth.weights(4, K, N, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, 1024)
    packed = bgt.repack_int4_canonical(to_dev(orc.pack_int4_canonical(ow["codes"]), dev), K, N)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    y = bgt.w4a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), packed, to_dev(ow["iscale"], dev), 1024, N,
                         acc_out=acc)
    oA, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.int32), oy.astype(np.float32).view(np.int32))
