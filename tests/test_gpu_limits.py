"""GPU parity at the sizes where 32-bit offsets would wrap.

The boundary accepts M and K up to 65536 and N up to 2^24, so activation byte
offsets (row * K), output element offsets (row * N + col) and token offsets of
the grouped GEMM pass 2^31 well inside the limits. Each case builds its rows by
repeating a seeded block of P = 61 rows on the device (row i is base row
i % P; 61 is prime and does not divide 2^32 / K, so an offset that wrapped
would land on a row with other data), runs the entry point at full size, and
compares sampled rows -- among them rows whose offsets pass 2^31 -- with the
oracle's result for those rows, bit for bit.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

P = 61          # period of the repeated base rows
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


def say(*a):
    print(*a, flush=True)


def repeat_rows(base, M, dev):
    """M x cols device tensor whose row i is base row i % P."""
    b = torch.from_numpy(np.ascontiguousarray(base)).to(dev)
    return b.repeat((M + P - 1) // P, *([1] * (b.dim() - 1)))[:M].contiguous()


def base_codes(orc, seed, K):
    """P rows of activation codes and scales, quantized by the oracle."""
    return orc.quant_sym_i8(synth.activations(seed, P, K))


def wrap32(a):
    return ((a + 2 ** 31) % 2 ** 32) - 2 ** 31


def check_rows(rows, y_rows, acc_rows, oA, oy, what):
    for n, i in enumerate(rows):
        if acc_rows is not None:
            np.testing.assert_array_equal(acc_rows[n].astype(np.int64), wrap32(oA[n]),
                                          err_msg=f"{what}: accumulators of row {i}")
        assert not np.isnan(y_rows[n]).any(), f"{what}: unwritten outputs in row {i}"
        np.testing.assert_array_equal(y_rows[n].view(np.int32), oy[n].view(np.int32),
                                      err_msg=f"{what}: outputs of row {i}")


def test_quantize_rows_past_2_31_bytes(bgt, orc, dev):
    M, K = 33000, 65536                      # q: 2.16e9 bytes; x: 8.65e9 bytes
    say(f"quantize_act sym M={M} K={K} (byte offsets past 2^31)")
    x = synth.activations(71, P, K)
    xd = repeat_rows(x, M, dev)
    q, s, _ = bgt.quantize_act(xd)
    torch.cuda.synchronize()
    oq, os_ = orc.quant_sym_i8(x)
    rows = [0, 1, 32767, 32768, 32769, 32768 + 100, M - 2, M - 1]
    got_q = q[rows].cpu().numpy()
    got_s = s[rows].cpu().numpy()
    for n, i in enumerate(rows):
        np.testing.assert_array_equal(got_q[n], oq[i % P], err_msg=f"codes of row {i}")
        assert got_s[n].view(np.int32) == os_[i % P].view(np.int32), f"scale of row {i}"
    del xd, q, s
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_x(orc, dev):
    """33000 x 65536 activation codes (2.16e9 bytes) and their scales."""
    M, K = 33000, 65536
    bq, bs = base_codes(orc, 72, K)
    return M, K, bq, bs, repeat_rows(bq, M, dev), repeat_rows(bs, M, dev)


ROWS_BIG = [0, 1, 255, 256, 32767, 32768, 32769, 32999 - 300, 32998, 32999]


def test_w4a8_is_activation_offsets_past_2_31(bgt, orc, dev, big_x):
    M, K, bq, bs, qx, sx = big_x
    N = 48
    say(f"w4a8_gemm_is M={M} K={K} N={N} kernel={bgt.w4a8_kernel_name(M, N, K)}")
    w = synth.weights(73, K, N, std=0.02, outlier_prob=0.001)
    ow = orc.pack_weights(w, 128, ALPHA)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=ALPHA)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w4a8_gemm_is(qx, sx, pw["packed"], pw["iscale"], ALPHA, N, y=y, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pw["packed"].cpu().numpy(), ow["packed"])
    np.testing.assert_array_equal(pw["iscale"].cpu().numpy(), ow["iscale"])
    assert not torch.isnan(y).any().item(), "unwritten outputs"
    idx = [i % P for i in ROWS_BIG]
    oA, oy, _ = orc.w4a8_gemm_is(bq[idx], bs[idx], ow["codes"], ow["iscale"], ALPHA)
    check_rows(ROWS_BIG, y[ROWS_BIG].cpu().numpy(), acc[ROWS_BIG].cpu().numpy(), oA, oy, "w4a8_is")


def test_w8a8_is_activation_offsets_past_2_31(bgt, orc, dev, big_x):
    M, K, bq, bs, qx, sx = big_x
    N = 256
    say(f"w8a8_gemm_is M={M} K={K} N={N} kernel={bgt.w8a8_is_kernel_name(M, N, K)}")
    w = synth.weights(74, K, N, std=0.02, outlier_prob=0.001)
    ow = orc.pack_weights_int8(w, 128, 1 << 16)
    pw = bgt.pack_weights_int8(torch.from_numpy(w).to(dev), alpha=1 << 16)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w8a8_gemm_is(qx, sx, pw["qw"], pw["iscale"], 1 << 16, N, y=y, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pw["iscale"].cpu().numpy(), ow["iscale"])
    assert not torch.isnan(y).any().item(), "unwritten outputs"
    idx = [i % P for i in ROWS_BIG]
    oA, oy, _ = orc.w8a8_gemm_is(bq[idx], bs[idx], ow["codes"], ow["iscale"], 1 << 16)
    check_rows(ROWS_BIG, y[ROWS_BIG].cpu().numpy(), acc[ROWS_BIG].cpu().numpy(), oA, oy, "w8a8_is")


def test_moe_token_offsets_past_2_31(bgt, orc, dev, big_x):
    T, K, bq, bs, qx, sx = big_x
    E, N = 2, 32
    offs, tok = synth.route_by_expert(synth.moe_routing(75, T, E, 1), E)
    say(f"w4a8_moe_gemm_is T={T} E={E} R={len(tok)} K={K} N={N} kernel={bgt.w4a8_moe_kernel_name(T, E, len(tok), K)}")
    ws = synth.expert_weights(75, E, K, N)
    ows = [orc.pack_weights(ws[e], 128, ALPHA) for e in range(E)]
    pws = [bgt.pack_weights_int4(torch.from_numpy(ws[e]).to(dev), alpha=ALPHA) for e in range(E)]
    packed = torch.stack([p["packed"] for p in pws])
    isc = torch.stack([p["iscale"] for p in pws])
    R = len(tok)
    y = torch.full((R, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.empty((R, N), dtype=torch.int32, device=dev)
    bgt.w4a8_moe_gemm_is(qx, sx, torch.from_numpy(offs).to(dev), torch.from_numpy(tok).to(dev),
                         packed, isc, ALPHA, N, y=y, acc_out=acc)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item(), "unwritten outputs"
    # slots of both experts, among them slots whose token offset passes 2^31
    slots = []
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        far = [r for r in range(a, b) if tok[r] >= 32768]
        slots += [a, b - 1] + far[:2] + far[-2:]
    got_y = y[slots].cpu().numpy()
    got_a = acc[slots].cpu().numpy()
    for n, r in enumerate(slots):
        e = int(np.searchsorted(offs, r, side="right")) - 1
        i = int(tok[r])
        oA, oy, _ = orc.w4a8_gemm_is(bq[[i % P]], bs[[i % P]], ows[e]["codes"], ows[e]["iscale"], ALPHA)
        check_rows([r], got_y[n:n + 1], got_a[n:n + 1], oA, oy, f"moe expert {e} token {i}")


def test_w4a8_is_output_offsets_past_2_31(bgt, orc, dev):
    M, K, N = 65536, 128, 32784               # y: 2^31 + 2^20 elements
    say(f"w4a8_gemm_is M={M} K={K} N={N} (output element offsets past 2^31) "
        f"kernel={bgt.w4a8_kernel_name(M, N, K)}")
    bq, bs = base_codes(orc, 76, K)
    qx, sx = repeat_rows(bq, M, dev), repeat_rows(bs, M, dev)
    w = synth.weights(77, K, N, std=0.02, outlier_prob=0.001)
    ow = orc.pack_weights(w, 128, ALPHA)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=ALPHA)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    bgt.w4a8_gemm_is(qx, sx, pw["packed"], pw["iscale"], ALPHA, N, y=y)
    torch.cuda.synchronize()
    rows = [0, 65503, 65504, 65520, 65534, 65535]   # rows from 65504 on pass 2^31
    idx = [i % P for i in rows]
    oA, oy, _ = orc.w4a8_gemm_is(bq[idx], bs[idx], ow["codes"], ow["iscale"], ALPHA)
    check_rows(rows, y[rows].cpu().numpy(), None, oA, oy, "w4a8_is wide output")
    assert not torch.isnan(y[-64:]).any().item(), "unwritten outputs in the last rows"
    del y, qx, sx
    torch.cuda.empty_cache()


def test_w8a8_zp_weight_offsets_past_2_31(bgt, orc, dev):
    M, K, N = 16, 32768, 65600               # W^T codes: 2.15e9 bytes (K is the control's limit)
    say(f"w8a8_gemm_zp M={M} K={K} N={N} (weight byte offsets past 2^31)")
    x = synth.activations(78, M, K, mean=0.5)
    wt = np.ascontiguousarray(synth.weights(79, K, P).T)       # P rows of W^T
    qx, sx, zx, rx = bgt.quantize_act(torch.from_numpy(x).to(dev), mode="asym")
    wtd = repeat_rows(wt, N, dev)                              # 8.6e9 bytes of fp32
    qw, sw, zw, cw = bgt.quantize_act(wtd, mode="asym")
    del wtd
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    bgt.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw, y=y, acc_out=acc)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item(), "unwritten outputs"
    oqx, osx, ozx, orx = orc.quant_asym_u8(x)
    oqw, osw, ozw, ocw = orc.quant_asym_u8(wt)
    cols = [0, 1, 63, 64, 65535, 65536, 65537, N - 17, N - 1]  # from 65536 on: past 2^31
    idx = [n % P for n in cols]
    np.testing.assert_array_equal(qw[cols].cpu().numpy(), oqw[idx])
    np.testing.assert_array_equal(cw[cols].cpu().numpy(), ocw[idx])
    oA, oy, ov = orc.w8a8_gemm_zp(oqx, osx, ozx, orx, oqw[idx], osw[idx], ozw[idx], ocw[idx])
    assert ov == 0
    np.testing.assert_array_equal(acc[:, cols].cpu().numpy().astype(np.int64), oA)
    got = np.ascontiguousarray(y[:, cols].cpu().numpy())
    np.testing.assert_array_equal(got.view(np.int32), oy.view(np.int32))
    del qw, y, acc
    torch.cuda.empty_cache()
