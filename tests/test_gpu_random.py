"""GPU parity on seeded random shapes, for every GEMM entry point and the quantizer.

Shapes, amplifiers, scale widths, output types and routings are drawn from a
fixed seed, so each case is reproducible by its id; the draws cover every
kernel path (decode, stream, skinny and tiled W4A8; split, 64 x 64 and wide
W8A8 integer-scale; both grouped paths) with ragged rows, ragged column tiles
and uneven group counts. Every output is compared with the oracle bit for bit
(int32 accumulators and fp32 / fp16 / bf16 outputs).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_MAC = 6e8            # keeps each oracle run well under a second


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


TORCH_T = {"f32": None, "f16": "float16", "bf16": "bfloat16"}


def _draw_shape(g, m_hi, k_hi, n_hi):
    while True:
        M = int(g.integers(1, m_hi + 1))
        K = 128 * int(g.integers(1, k_hi + 1))
        N = 16 * int(g.integers(1, n_hi + 1))
        if M * K * N <= MAX_MAC:
            return M, K, N


def _check_y(orc, y, oy, kind):
    oy = oy.astype(np.float32)
    if kind == "f32":
        got = y.cpu().numpy()
        assert not np.isnan(got).any()
        np.testing.assert_array_equal(got.view(np.int32), oy.view(np.int32))
    else:
        bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oy.astype(np.float16).view(np.uint16) if kind == "f16" else orc.f32_to_bf16_bits(oy)
        np.testing.assert_array_equal(bits, want)


def _out_dtype(kind):
    return None if kind == "f32" else getattr(torch, TORCH_T[kind])


@pytest.mark.parametrize("case", range(24))
def test_random_w4a8_is(bgt, orc, dev, case):
    g = np.random.default_rng(1000 + case)
    # small M on most draws (decode, stream and skinny paths), some tiled
    M, K, N = _draw_shape(g, 64 if case % 3 else 700, 48, 96)
    alpha = int(2 ** g.integers(8, 13))
    width = int(g.choice([1, 2, 4]))
    kind = str(g.choice(["f32", "f16", "bf16"]))
    say(f"random w4a8_is #{case}: M={M} K={K} N={N} alpha={alpha} width={width} y={kind} "
        f"kernel={bgt.w4a8_kernel_name(M, N, K)}")
    x = synth.activations(2000 + case, M, K)
    w = synth.weights(3000 + case, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, alpha)
    if width != 4 and ow["iscale"].max() >= 256 ** width:
        width = 4
    isc = to_dev(ow["iscale"], dev)
    if width != 4:
        isc = bgt.narrow_iscale(isc, width)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w4a8_gemm_is_narrow(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev), isc,
                                alpha, N, acc_out=acc, out_dtype=_out_dtype(kind))
    oA, oy, ov = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], alpha)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    _check_y(orc, y, oy, kind)


@pytest.mark.parametrize("case", range(10))
def test_random_w4a8_fs(bgt, orc, dev, case):
    g = np.random.default_rng(4000 + case)
    M, K, N = _draw_shape(g, 64 if case % 2 else 600, 40, 80)
    say(f"random w4a8_fs #{case}: M={M} K={K} N={N} kernel={bgt.w4a8_kernel_name(M, N, K, True)}")
    x = synth.activations(5000 + case, M, K)
    w = synth.weights(6000 + case, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights(w, 128, 1024)
    y = bgt.w4a8_gemm_fs(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["packed"], dev),
                         to_dev(ow["fscale"], dev), N)
    oy = orc.w4a8_gemm_fs(oq, os_, ow["codes"], ow["fscale"])
    _check_y(orc, y, oy, "f32")


@pytest.mark.parametrize("case", range(16))
def test_random_w8a8_is(bgt, orc, dev, case):
    g = np.random.default_rng(7000 + case)
    M, K, N = _draw_shape(g, 64 if case % 2 else 1200, 40, 256)
    alpha = int(2 ** g.integers(12, 19))
    width = int(g.choice([1, 2, 4]))
    kind = str(g.choice(["f32", "f16", "bf16"]))
    say(f"random w8a8_is #{case}: M={M} K={K} N={N} alpha={alpha} width={width} y={kind} "
        f"kernel={bgt.w8a8_is_kernel_name(M, N, K)}")
    x = synth.activations(8000 + case, M, K)
    w = synth.weights(9000 + case, K, N, std=0.02, outlier_prob=0.001)
    oq, os_ = orc.quant_sym_i8(x)
    ow = orc.pack_weights_int8(w, 128, alpha)
    if width != 4 and ow["iscale"].max() >= 256 ** width:
        width = 4
    isc = to_dev(ow["iscale"], dev)
    if width != 4:
        isc = bgt.narrow_iscale(isc, width)
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w8a8_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(ow["qw"], dev), isc, alpha, N,
                         acc_out=acc, out_dtype=_out_dtype(kind))
    oA, oy, ov = orc.w8a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], alpha)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    _check_y(orc, y, oy, kind)


@pytest.mark.parametrize("case", range(12))
def test_random_moe(bgt, orc, dev, case):
    g = np.random.default_rng(10000 + case)
    E = int(g.integers(1, 17))
    topk = int(min(E, g.integers(1, 3)))
    T = int(g.integers(1, 65 if case % 2 else 400))
    K = 128 * int(g.choice([16, 32] if case % 2 else [3, 8, 16, 32]))
    N = 16 * int(g.integers(1, 40))
    kind = str(g.choice(["f32", "bf16"]))
    routing = synth.moe_routing(11000 + case, T, E, topk)
    offs, tok = synth.route_by_expert(routing, E)
    say(f"random moe #{case}: T={T} E={E} topk={topk} K={K} N={N} y={kind} "
        f"kernel={bgt.w4a8_moe_kernel_name(T, E, len(tok), K)}")
    x = synth.activations(12000 + case, T, K)
    w = synth.expert_weights(13000 + case, E, K, N)
    oq, os_ = orc.quant_sym_i8(x)
    pws = [orc.pack_weights(w[e], 128, 1024) for e in range(E)]
    codes = np.stack([p["codes"] for p in pws])
    isc = np.stack([p["iscale"] for p in pws])
    packed = np.stack([p["packed"] for p in pws])
    acc = torch.full((len(tok), N), -1, dtype=torch.int32, device=dev)
    y = bgt.w4a8_moe_gemm_is(to_dev(oq, dev), to_dev(os_, dev), to_dev(offs, dev), to_dev(tok, dev),
                             to_dev(packed, dev), to_dev(isc, dev), 1024, N, acc_out=acc,
                             out_dtype=_out_dtype(kind))
    oA, oy, ov = orc.moe_w4a8_gemm_is(oq, os_, codes, isc, 1024, offs, tok)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    _check_y(orc, y, oy, kind)


@pytest.mark.parametrize("case", range(10))
def test_random_linear(bgt, orc, dev, case):
    g = np.random.default_rng(14000 + case)
    M = int(g.integers(1, 5 if case % 2 else 40))
    K = 128 * int(g.choice([16, 32] if case % 2 else [5, 16, 32]))
    N = 16 * int(g.integers(1, 120))
    kind = str(g.choice(["f32", "f16", "bf16"]))
    x = synth.activations(15000 + case, M, K)
    if kind == "f32":
        xd, xw = to_dev(x, dev), x
    elif kind == "f16":
        h = x.astype(np.float16)
        xd, xw = to_dev(h, dev), h.astype(np.float32)
    else:
        bits = orc.f32_to_bf16_bits(x)
        xd, xw = to_dev(bits.view(np.int16), dev).view(torch.bfloat16), orc.bf16_bits_to_f32(bits)
    w = synth.weights(16000 + case, K, N, std=0.02, outlier_prob=0.001)
    ow = orc.pack_weights(w, 128, 1024)
    say(f"random linear #{case}: M={M} K={K} N={N} x=y={kind} fused={bgt.w4a8_linear_fused(xd)}")
    y, qx, sx = bgt.w4a8_linear_is(xd, to_dev(ow["packed"], dev), to_dev(ow["iscale"], dev), 1024, N)
    oq, os_ = orc.quant_sym_i8(xw)
    np.testing.assert_array_equal(qx.cpu().numpy(), oq)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.int32), os_.view(np.int32))
    _, oy, _ = orc.w4a8_gemm_is(oq, os_, ow["codes"], ow["iscale"], 1024)
    _check_y(orc, y, oy, kind)


@pytest.mark.parametrize("case", range(8))
def test_random_w8a8_zp(bgt, orc, dev, case):
    g = np.random.default_rng(17000 + case)
    M, K, N = _draw_shape(g, 64 if case % 2 else 600, 48, 128)
    relu = bool(case % 3 == 0)
    say(f"random w8a8_zp #{case}: M={M} K={K} N={N} relu={relu}")
    x, w = synth.w8a8_inputs(18000 + case, M, K, N, relu=relu)
    qx, sx, zx, rx = bgt.quantize_act(to_dev(x, dev), mode="asym")
    qw, sw, zw, cw = bgt.quantize_act(to_dev(np.ascontiguousarray(w.T), dev), mode="asym")
    oqx, osx, ozx, orx = orc.quant_asym_u8(x)
    oqw, osw, ozw, ocw = orc.quant_asym_u8(np.ascontiguousarray(w.T))
    for got, want in ((qx, oqx), (zx, ozx), (rx, orx), (qw, oqw), (zw, ozw), (cw, ocw)):
        np.testing.assert_array_equal(got.cpu().numpy(), want)
    for got, want in ((sx, osx), (sw, osw)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.int32), want.view(np.int32))
    acc = torch.full((M, N), -1, dtype=torch.int32, device=dev)
    y = bgt.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw, acc_out=acc)
    oA, oy, ov = orc.w8a8_gemm_zp(oqx, osx, ozx, orx, oqw, osw, ozw, ocw)
    assert ov == 0
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oA)
    _check_y(orc, y, oy, "f32")


@pytest.mark.parametrize("case", range(12))
def test_random_quantize(bgt, orc, dev, case):
    # any row count, any column count (vector and scalar paths), padded rows, three input types
    g = np.random.default_rng(19000 + case)
    rows = int(g.integers(1, 300))
    cols = int(g.integers(1, 5000)) if case % 2 else 16 * int(g.integers(1, 600))
    pad = int(g.choice([0, 0, 4, 7]))
    kind = str(g.choice(["f32", "f16", "bf16"]))
    asym = bool(case % 3 == 0)
    say(f"random quantize #{case}: rows={rows} cols={cols} pad={pad} x={kind} asym={asym}")
    x = synth.activations(20000 + case, rows, cols, outlier_frac=0.0 if asym else 0.01,
                          mean=0.5 if asym else 0.0)
    if kind == "f32":
        xh, xw = x, x
    elif kind == "f16":
        xh = x.astype(np.float16)
        xw = xh.astype(np.float32)
    else:
        xh = orc.f32_to_bf16_bits(x)
        xw = orc.bf16_bits_to_f32(xh)
    buf = np.zeros((rows, cols + pad), xh.dtype)
    buf[:, :cols] = xh
    xd = to_dev(buf if kind != "bf16" else buf.view(np.int16), dev)
    if kind == "bf16":
        xd = xd.view(torch.bfloat16)
    xd = xd[:, :cols]
    if asym:
        q, s, z, r = bgt.quantize_act(xd, mode="asym")
        oq, os_, oz, orow = orc.quant_asym_u8(xw)
        np.testing.assert_array_equal(z.cpu().numpy(), oz)
        np.testing.assert_array_equal(r.cpu().numpy(), orow)
    else:
        q, s, _ = bgt.quantize_act(xd)
        oq, os_ = orc.quant_sym_i8(xw)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.int32), os_.view(np.int32))
