"""The no-allocation W4A8 integer-scale GEMM (bgt_w4a8_gemm_is_noalloc),
called through the C ABI, against bgt_w4a8_gemm_is on the same inputs: y bit
for bit and the int32 accumulators exactly, on two calls in a row (the second
smaller), where both split K and keep the split sums in the static scratch,
then on shapes of the unsplit paths. The oracle checks the first shape too."""
import ctypes

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


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def run_pair(bgt, dev, M, K, N, seed):
    x = synth.activations(seed, M, K)
    w = synth.weights(seed + 1, K, N, std=0.02, outlier_prob=0.001)
    xd = torch.from_numpy(x).to(dev)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=1024)
    q, s, _ = bgt.quantize_act(xd)
    y_ref = torch.full((M, N), float("nan"), device=dev)
    a_ref = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(q, s, pw["packed"], pw["iscale"], 1024, N, y=y_ref, acc_out=a_ref)
    y = torch.full((M, N), float("nan"), device=dev)
    a = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = bgt.lib().bgt_w4a8_gemm_is_noalloc(ptr(q), ptr(s), ptr(pw["packed"]), ptr(pw["iscale"]),
                                            1024, M, N, K, ptr(y), ptr(a), stream)
    assert st == 0, bgt.status_string(st)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    assert torch.equal(a, a_ref)
    return q, s, w, y, a


def test_noalloc_split_then_smaller(bgt, orc, dev):
    first = (512, 4096, 4096)                      # 4 splits: the whole 32 MiB scratch
    assert bgt.w4a8_workspace_bytes(first[0], first[2], first[1]) == 32 << 20
    print("noalloc M=512 K=4096 N=4096", flush=True)
    q, s, w, y, a = run_pair(bgt, dev, *first, seed=41)
    oq, os_ = q.cpu().numpy(), s.cpu().numpy()
    ow = orc.pack_weights(w, 128, 1024)
    oA, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    np.testing.assert_array_equal(a.cpu().numpy().astype(np.int64), oA)
    assert np.array_equal(y.cpu().numpy().view(np.int32), oy.astype(np.float32).view(np.int32))
    second = (129, 2560, 528)                      # 4 splits of 5 groups, ragged
    assert 0 < bgt.w4a8_workspace_bytes(second[0], second[2], second[1]) < 32 << 20
    print("noalloc M=129 K=2560 N=528", flush=True)
    run_pair(bgt, dev, *second, seed=43)


@pytest.mark.parametrize("M,K,N", [(16, 4096, 4096), (256, 1024, 22016), (2048, 512, 22016)])
def test_noalloc_unsplit_and_other_paths(bgt, dev, M, K, N):
    print(f"noalloc M={M} K={K} N={N} kernel={bgt.w4a8_kernel_name(M, N, K)} "
          f"workspace={bgt.w4a8_workspace_bytes(M, N, K)}", flush=True)
    run_pair(bgt, dev, M, K, N, seed=M + K + N)
