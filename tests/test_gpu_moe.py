"""GPU parity of the grouped (mixture-of-experts) W4A8 integer-scale GEMM.

bgt_w4a8_moe_gemm_is must give, for every routed slot, the oracle's int32
accumulators and outputs bit-exactly: on the decode path (T <= 64 tokens,
K/128 in {16, 32, 112}: one workgroup row per expert and row pass, experts
without tokens skipped) and on the tiled path (the experts' row tiles in one launch), with
skewed and degenerate routings, narrow scales, fp16 / bf16 outputs, and the
Mixtral-8x7B expert shapes (w1/w3: 4096 -> 14336, w2: 14336 -> 4096) on
sampled columns. The 256 x 256 tile kernel over the experts' row tiles runs
when bgt_set_prefill_kernel forces it: on small, ragged, skewed and
Mixtral-sized routings, with narrow scales and half outputs.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALPHA = 1024


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


def _experts(orc, seed, E, K, N):
    w = synth.expert_weights(seed, E, K, N)
    pws = [orc.pack_weights(w[e], 128, ALPHA) for e in range(E)]
    codes = np.stack([p["codes"] for p in pws])
    packed = np.stack([p["packed"] for p in pws])
    isc = np.stack([p["iscale"] for p in pws])
    return codes, packed, isc


def _run(bgt, orc, dev, T, E, K, N, seed, routing=None, width=4, out_dtype=None, cols=None):
    x = synth.activations(seed, T, K)
    oq, os_ = orc.quant_sym_i8(x)
    if routing is None:
        routing = synth.moe_routing(seed, T, E, min(2, E))
    offs, tok = synth.route_by_expert(routing, E)
    codes, packed, isc = _experts(orc, seed + 7, E, K, N)
    R = len(tok)
    isc_d = to_dev(isc, dev)
    if width != 4:
        isc_d = bgt.narrow_iscale(isc_d, width)
    acc = torch.full((R, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w4a8_moe_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(offs, dev), to_dev(tok, dev),
                             to_dev(packed, dev), isc_d, ALPHA, N, acc_out=acc, out_dtype=out_dtype)
    oA, oy, ov = orc.moe_w4a8_gemm_is(oq, os_, codes, isc, ALPHA, offs, tok, cols=cols)
    assert ov == 0
    got_a = acc.cpu().numpy().astype(np.int64)
    if cols is not None:
        got_a = got_a[:, cols]
    np.testing.assert_array_equal(got_a, oA)
    oy = oy.astype(np.float32)
    if out_dtype is None:
        got = y.cpu().numpy()
        if cols is not None:
            got = got[:, cols]
        assert not np.isnan(got).any()
        np.testing.assert_array_equal(got.view(np.int32), oy.view(np.int32))
    else:
        bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oy.astype(np.float16).view(np.uint16) if out_dtype == torch.float16 \
            else orc.f32_to_bf16_bits(oy)
        np.testing.assert_array_equal(bits, want)
    return offs


DECODE = "k_w4a8_decode<IS,grouped>"
TILED = "k_w4a8_prefill<4,2,2,2,IS,grouped>"
WIDE = "k_w4a8_wide<IS,grouped>"


@pytest.mark.parametrize("T,E,K,N", [(1, 8, 4096, 64), (5, 8, 4096, 208), (16, 8, 2048, 96),
                                     (33, 8, 4096, 48), (64, 8, 2048, 16), (20, 3, 4096, 80),
                                     (1, 8, 14336, 48), (12, 8, 14336, 80), (32, 5, 14336, 32),
                                     (64, 8, 14336, 48), (50, 2, 2048, 32),
                                     # more tokens, up to two row passes of 64 slots (16, 32
                                     # groups) or three of 32 (112 groups) per mean expert
                                     (128, 8, 4096, 64), (300, 8, 2048, 48), (512, 8, 4096, 32),
                                     (200, 8, 14336, 32), (384, 8, 14336, 16), (250, 6, 14336, 16)])
def test_moe_decode_path(bgt, orc, dev, T, E, K, N):
    name = bgt.w4a8_moe_kernel_name(T, E, T * min(2, E), K)
    say(f"moe {name} T={T} E={E} K={K} N={N}")
    assert name == DECODE
    offs = _run(bgt, orc, dev, T, E, K, N, seed=T * 31 + K + N)
    if T == 1:
        assert (np.diff(offs) > 0).sum() == 2             # six experts read nothing


@pytest.fixture
def forced(bgt):
    yield bgt.set_prefill_kernel
    bgt.set_prefill_kernel("auto")


@pytest.mark.parametrize("T,E,K,N", [(65, 8, 512, 144), (300, 8, 256, 48), (20, 8, 1152, 64),
                                     (130, 4, 640, 400), (257, 8, 128, 16),
                                     # past the decode kernel's range: T > 1024, or more row
                                     # passes for the mean expert
                                     (1100, 8, 4096, 16), (600, 8, 14336, 16), (700, 2, 2048, 32),
                                     (1024, 8, 4096, 32), (520, 8, 4096, 32), (1000, 8, 4096, 16),
                                     (300, 6, 14336, 16),
                                     (1100, 16, 512, 48)])
def test_moe_tiled_path(bgt, orc, dev, forced, T, E, K, N):
    # past the decode range: the 256 x 128 tile kernel (forced; automatic at
    # K/128 > 32)
    forced("tiled")
    name = bgt.w4a8_moe_kernel_name(T, E, T * min(2, E), K)
    say(f"moe {name} T={T} E={E} K={K} N={N}")
    assert name == TILED
    _run(bgt, orc, dev, T, E, K, N, seed=T * 37 + K + N)


@pytest.mark.parametrize("T,E,K,N", [(1100, 8, 4096, 16), (65, 8, 512, 144), (600, 8, 14336, 16),
                                     (2100, 8, 14336, 16), (520, 8, 4096, 32)])
def test_moe_auto_tile_kernel(bgt, orc, dev, T, E, K, N):
    # past the decode range, automatically: 256 x 256 tiles at K/128 <= 32,
    # 256 x 128 beyond
    name = bgt.w4a8_moe_kernel_name(T, E, T * min(2, E), K)
    say(f"moe auto {name} T={T} E={E} K={K} N={N}")
    assert name == (WIDE if K // 128 <= 32 else TILED)
    _run(bgt, orc, dev, T, E, K, N, seed=T * 47 + K + N)


@pytest.mark.parametrize("T,E,K,N", [(65, 8, 512, 144), (300, 8, 256, 48), (20, 8, 1152, 64),
                                     (130, 4, 640, 400), (257, 8, 128, 16), (600, 8, 14336, 16),
                                     (1100, 8, 4096, 16), (700, 2, 2048, 32), (1200, 4, 512, 400),
                                     (2100, 8, 14336, 16), (1500, 3, 384, 272)])
def test_moe_wide_forced(bgt, orc, dev, forced, T, E, K, N):
    forced("wide")
    name = bgt.w4a8_moe_kernel_name(T, E, T * min(2, E), K)
    say(f"moe forced {name} T={T} E={E} K={K} N={N}")
    assert name == WIDE
    _run(bgt, orc, dev, T, E, K, N, seed=T * 43 + K + N)


def test_moe_wide_forced_skewed_narrow_half(bgt, orc, dev, forced):
    forced("wide")
    T, K = 300, 4096
    say(f"moe forced wide: one busy expert, narrow scales, half outputs T={T} K={K}")
    routing = np.full((T, 1), 5, np.int32)
    routing[0, 0] = 2
    _run(bgt, orc, dev, T, 8, K, 64, seed=T + 5, routing=routing)
    for width in (1, 2):
        _run(bgt, orc, dev, 150, 8, 384, 96, seed=150 + width, width=width)
    for dt in (torch.float16, torch.bfloat16):
        _run(bgt, orc, dev, 100, 8, 256, 48, seed=117, out_dtype=dt)


def test_moe_wide_forced_mixtral_sampled(bgt, orc, dev, forced):
    forced("wide")
    T, K, N = 4096, 4096, 14336
    assert bgt.w4a8_moe_kernel_name(T, 8, 2 * T, K) == WIDE
    say(f"moe forced wide mixtral T={T} K={K} N={N} (sampled)")
    cols = np.unique(np.concatenate([np.arange(0, 32), np.arange(N - 32, N),
                                     np.random.default_rng(T + 1).choice(N, 160, replace=False)]))
    _run(bgt, orc, dev, T, 8, K, N, seed=T + 23, cols=cols)


@pytest.mark.parametrize("T,K", [(64, 4096), (200, 512), (64, 14336), (40, 2048), (300, 4096),
                                 (200, 14336)])
def test_moe_all_tokens_one_expert(bgt, orc, dev, T, K):
    # maximal imbalance: expert 5 takes every token, expert 2 one, the rest none
    # (on the decode path the busy expert takes several row passes)
    say(f"moe skewed T={T} K={K}")
    routing = np.full((T, 1), 5, np.int32)
    routing[0, 0] = 2
    _run(bgt, orc, dev, T, 8, K, 64, seed=T + 3, routing=routing)


# The grouped tile kernels deal the routing's row tiles evenly over the XCDs
# (workgroup id % 8) and let the rest of the grid, an upper bound computed
# without the routing, exit: grids that are not a multiple of 8, experts
# without slots between busy ones, one busy expert, row tiles of several
# experts in one column run; every output compared.
SPREAD = [
    (300, 11, 512, 272, None),        # grid (3 + 11) x 3 = 42 workgroups
    (400, 8, 1024, 144, (2, 5)),      # two busy experts, six idle
    (700, 16, 256, 48, (9,)),         # one busy expert with 700 slots (three row tiles)
    (1100, 5, 384, 400, None),        # 5 experts, 4 column tiles of 128 (one ragged)
    (200, 130, 256, 48, None),        # 130 experts: the offsets are read 64 experts at a time
]


@pytest.mark.parametrize("T,E,K,N,busy", SPREAD)
@pytest.mark.parametrize("kernel", ["tiled", "wide"])
def test_moe_tile_spread(bgt, orc, dev, forced, T, E, K, N, busy, kernel):
    forced(kernel)
    routing = None
    if busy is not None:
        routing = np.asarray([[busy[(t + i) % len(busy)] for i in range(len(busy))]
                              for t in range(T)], np.int32)
    R = T * (len(busy) if busy is not None else min(2, E))
    name = bgt.w4a8_moe_kernel_name(T, E, R, K)
    say(f"moe spread {name} T={T} E={E} K={K} N={N} busy={busy}")
    assert name == (WIDE if kernel == "wide" else TILED)
    _run(bgt, orc, dev, T, E, K, N, seed=T * 41 + E + K + N, routing=routing)


@pytest.mark.parametrize("T,K", [(12, 4096), (150, 384), (9, 14336), (200, 4096), (200, 14336)])
@pytest.mark.parametrize("width", [1, 2])
def test_moe_narrow_scales(bgt, orc, dev, width, T, K):
    say(f"moe width={width} T={T} K={K}")
    _run(bgt, orc, dev, T, 8, K, 96, seed=T + K + width, width=width)


@pytest.mark.parametrize("T,K", [(8, 2048), (100, 256)])
def test_moe_half_outputs(bgt, orc, dev, T, K):
    for dt in (torch.float16, torch.bfloat16):
        say(f"moe y={dt} T={T} K={K}")
        _run(bgt, orc, dev, T, 8, K, 48, seed=T + 11, out_dtype=dt)


@pytest.mark.parametrize("T,K,N", [(16, 4096, 14336), (64, 4096, 14336), (512, 4096, 14336),
                                   (4096, 4096, 14336), (16, 14336, 4096), (64, 14336, 4096),
                                   (512, 14336, 4096), (4096, 14336, 4096)])
def test_moe_mixtral_shapes_sampled(bgt, orc, dev, T, K, N):
    """Mixtral-8x7B experts (8, top-2) at the w1/w3 and w2 shapes, in the
    launches the bench times; sampled output columns against the oracle."""
    say(f"moe mixtral {bgt.w4a8_moe_kernel_name(T, 8, 2 * T, K)} T={T} K={K} N={N} (sampled)")
    cols = np.unique(np.concatenate([np.arange(0, 32), np.arange(N - 32, N),
                                     np.random.default_rng(T).choice(N, 160, replace=False)]))
    _run(bgt, orc, dev, T, 8, K, N, seed=T + 21, cols=cols)
