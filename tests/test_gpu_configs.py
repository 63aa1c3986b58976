"""GPU parity at the workloads' full sizes, in the launch configuration the bench times.

Each test runs the whole GPU path (per-token quantization -> int4 packing ->
W4A8 GEMM) on the seeded synthetic inputs and compares with the oracle run
on the same inputs: quantized codes, scales, packed bytes and integer scales
in full; GEMM accumulators and outputs on sampled rows x columns (first and
last tiles always included), since the oracle is a plain triple loop.
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


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def sample(n, k, seed, tile=16):
    g = synth.rng(seed, 77)
    idx = np.r_[np.arange(min(n, tile)), np.arange(max(0, n - tile), n), g.integers(0, n, k)]
    return np.unique(idx)


def check_layer(bgt, orc, dev, x, w, alpha=1024, fs=False, nrows=48, ncols=384, seed=0):
    M, K = x.shape
    N = w.shape[1]
    xd = to_dev(x, dev)
    qx, sx, _ = bgt.quantize_act(xd)
    pw = bgt.pack_weights_int4(to_dev(w, dev), alpha=alpha)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(qx, sx, pw["packed"], pw["iscale"], pw["alpha"], N, y=y, acc_out=acc)
    yf = None
    if fs:
        yf = bgt.w4a8_gemm_fs(qx, sx, pw["packed"], pw["fscale"], N)
    torch.cuda.synchronize()

    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, alpha)
    np.testing.assert_array_equal(qx.cpu().numpy(), oq)
    np.testing.assert_array_equal(sx.cpu().numpy(), os_)
    assert pw["alpha"] == ow["alpha"]
    np.testing.assert_array_equal(pw["iscale"].cpu().numpy(), ow["iscale"])
    np.testing.assert_array_equal(pw["fscale"].cpu().numpy(), ow["fscale"])
    np.testing.assert_array_equal(pw["packed"].cpu().numpy(), ow["packed"])

    rows = np.arange(M) if M <= nrows else sample(M, nrows, seed + 1)
    cols = sample(N, ncols, seed + 2)
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], ow["alpha"], rows=rows, cols=cols)
    assert ov == 0
    yh = y.cpu().numpy()
    assert not np.isnan(yh).any()
    np.testing.assert_array_equal(acc.cpu().numpy()[np.ix_(rows, cols)].astype(np.int64), oA)
    np.testing.assert_array_equal(yh[np.ix_(rows, cols)], oy)
    if fs:
        oyf = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"], rows=rows, cols=cols)
        np.testing.assert_array_equal(yf.cpu().numpy()[np.ix_(rows, cols)], oyf)


def test_single_gemm_16x4096x4096(bgt, orc, dev):
    say("config: single W4A8-IS GEMM M=16 K=4096 N=4096 seed 0")
    x, w = synth.single_gemm_inputs(0)
    check_layer(bgt, orc, dev, x, w, fs=True, nrows=16, ncols=4096)


@pytest.fixture(scope="module")
def layer(orc):
    x, w = synth.layer_inputs(0, M=max(synth.PREFILL_M))
    return x, w


@pytest.mark.parametrize("M", synth.DECODE_M)
def test_decode_sweep(bgt, orc, dev, layer, M):
    say(f"config: decode sweep K=4096 N=22016 M={M}")
    x, w = layer
    check_layer(bgt, orc, dev, np.ascontiguousarray(x[:M]), w, fs=True, seed=M)


@pytest.mark.parametrize("M", synth.PREFILL_M)
def test_prefill_sweep(bgt, orc, dev, layer, M):
    say(f"config: prefill sweep K=4096 N=22016 M={M} (IS and FS)")
    x, w = layer
    check_layer(bgt, orc, dev, np.ascontiguousarray(x[:M]), w, fs=True, seed=M, nrows=24, ncols=160)


@pytest.mark.parametrize("M", [1, 512])
def test_llama2_7b_block(bgt, orc, dev, M):
    for name, x, w in synth.block_inputs(0, M):
        say(f"config: LLaMA-2-7B block {name} K={w.shape[0]} N={w.shape[1]} M={M}")
        check_layer(bgt, orc, dev, x, w, nrows=16, ncols=160, seed=M)


def test_searched_amplifier_layer(bgt, orc, dev, layer):
    say("config: decode layer M=16 with the searched amplifier")
    x, w = layer
    check_layer(bgt, orc, dev, np.ascontiguousarray(x[:16]), w, alpha=0)
