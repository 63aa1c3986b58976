"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU. Each one is chosen so that a plausible mistake
in the oracle (a dropped term, a wrong sign or index, half-even instead of
half-away rounding, truncation, a transposed operand, a wrong clip range)
fails it. Pages: [IS] Integer Scale summary page, [QB] "量化基礎" blog,
[QN] "Quantization" notes.
"""
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (t.strip() for t in line.split("="))
                out[k] = int(v)
    return out


# ------------------------------------------------------------------ O1 symmetric int8

def test_sym_hand_vector_ties_round_half_away(orc):
    # absmax 127 -> s = 1 exactly; ties +-0.5 and 2.5 go away from zero ("四舍五入",
    # [QB] §2.2); half-even would give 0, 0, 2 instead.
    x = np.array([[127.0, 0.5, -0.5, 2.5, -63.5, 1.49, -126.6]], np.float32)
    q, s = orc.quant_sym_i8(x)
    assert s[0] == np.float32(1.0)
    assert q.tolist() == [[127, 1, -1, 3, -64, 1, -127]]


def test_sym_range_and_absmax_maps_to_qmax(orc):
    r = golden("quant_ranges.txt")
    x = synth.activations(3, 33, 1000)
    x[5, 17] = -1e3      # the row's absmax is negative
    q, s = orc.quant_sym_i8(x)
    assert q.min() >= r["sym_int8_qmin"] and q.max() <= r["sym_int8_qmax"]
    am = np.abs(x).argmax(axis=1)
    picked = q[np.arange(33), am].astype(int)
    assert np.all(np.abs(picked) == 127)
    assert picked[5] == -127
    np.testing.assert_array_equal(s, (np.abs(x).max(axis=1) / np.float32(127.0)).astype(np.float32))


def test_sym_rounding_error_bound_and_sign(orc):
    # |x - s q| <= s/2 (plus one float rounding of x/s); truncation would break it.
    x = synth.activations(4, 64, 512)
    q, s = orc.quant_sym_i8(x)
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -20))
    assert np.all((q == 0) | (np.sign(q) == np.sign(x)))


def test_sym_error_variance_is_s2_over_12(orc):
    # [QB] §2.2 quantization error: sigma^2 ~ s^2/12 for round-to-nearest.
    # A uniform row makes the rounding error uniform on [-s/2, s/2].
    g = synth.rng(11, 99)
    x = g.uniform(-1.0, 1.0, size=(1, 1_000_000)).astype(np.float32)
    q, s = orc.quant_sym_i8(x)
    mse = np.mean((x.astype(np.float64) - float(s[0]) * q) ** 2)
    assert abs(mse / (float(s[0]) ** 2 / 12.0) - 1.0) < 0.05


def test_sym_zero_row(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = 2.0
    q, s = orc.quant_sym_i8(x)
    assert s[0] == 0 and not q[0].any()
    assert q[1, 3] == 127 and s[1] == np.float32(2.0) / np.float32(127.0)


# ----------------------------------------------------------------- O5 asymmetric uint8

def test_asym_hand_vector(orc):
    # x_min = -1, x_max = 254: s = 255/255 = 1, z = round(0 - (-1)/1) = 1.
    x = np.array([[-1.0, 254.0, 0.0, 0.5, -0.5, 100.4]], np.float32)
    q, s, z, rs = orc.quant_asym_u8(x)
    assert s[0] == 1.0 and z[0] == 1
    # round(x/s) + z: 0.5 -> 1+1, -0.5 -> -1+1 (half away from zero, then add z)
    assert q.tolist() == [[0, 255, 1, 2, 0, 101]]
    assert rs[0] == sum(q[0].astype(int))


def test_asym_min_max_map_to_ends(orc):
    r = golden("quant_ranges.txt")
    x = synth.activations(5, 40, 777, outlier_frac=0.0, mean=0.5)
    q, s, z, rs = orc.quant_asym_u8(x)
    assert q.min() >= r["asym_uint8_qmin"] and q.max() <= r["asym_uint8_qmax"]
    i = np.arange(40)
    assert np.all(q[i, x.argmin(axis=1)] == 0)
    assert np.all(q[i, x.argmax(axis=1)] >= 254)
    np.testing.assert_array_equal(rs, q.astype(np.int64).sum(axis=1))
    # dequantization s(q - z) is within half a step of x, except clipped top codes
    xh = s[:, None].astype(np.float64) * (q.astype(np.int64) - z[:, None])
    err = np.abs(x - xh)
    ok = err <= s[:, None] * (0.5 + 2.0 ** -18)
    assert np.all(ok | (q == 255))


def test_asym_one_sided_row_saturates(orc):
    # the raw-range reading: a row whose values are all positive gets s = (max - min)/255
    # and z = clip(round(-min/s), 0, 255) = 0, so codes above (max - min)/s saturate at 255;
    # the header states the precondition (the row range must contain 0) for the W8A8 control
    x = np.array([[1.0, 2.0, 3.0, 4.0]], np.float32)
    q, s, z, rs = orc.quant_asym_u8(x)
    assert s[0] == np.float32(3.0) / np.float32(255.0) and z[0] == 0
    assert q.tolist() == [[85, 170, 255, 255]]
    xh = s[0] * (q.astype(np.float64) - z[0])
    assert abs(xh[0, 3] - 4.0) > 0.5                     # not representable: saturated


def test_asym_degenerate_row(orc):
    x = np.full((1, 16), 3.0, np.float32)
    q, s, z, rs = orc.quant_asym_u8(x)
    assert s[0] == 0 and z[0] == 0 and rs[0] == 0 and not q.any()


# --------------------------------------------------------------- O2 int4 group quant

def test_group_scale_count_matches_page():
    f = golden("is_method_facts.txt")
    G = f["layer_k"] // f["group"]
    assert G * f["layer_n"] == f["float_scale_count"]


def test_group_quant_shapes_and_count(orc):
    f = golden("is_method_facts.txt")
    w = synth.weights(0, 512, 64)
    codes, fs = orc.group_quant_int4(w, 128)
    assert fs.shape == (4, 64) and codes.shape == (512, 64)
    # the page's 4096x4096 count, from the oracle's own shape rule
    assert (f["layer_k"] // f["group"]) * f["layer_n"] == f["float_scale_count"]


def test_group_quant_hand_group(orc):
    # one column, one group of 128: absmax 7 -> s = 1; ties away from zero; clip [-7,7]
    w = np.zeros((128, 16), np.float32)
    w[:8, 0] = [7.0, 3.5, -3.5, 0.5, -0.49, -7.0, 6.6, 2.5]
    w[:, 1] = np.linspace(-1, 1, 128)
    codes, fs = orc.group_quant_int4(w, 128)
    assert fs[0, 0] == 1.0
    assert codes[:8, 0].tolist() == [7, 4, -4, 1, 0, -7, 7, 3]
    assert fs[0, 2] == 0 and not codes[:, 2].any()          # all-zero group
    assert codes[:, 1].min() == -7 and codes[:, 1].max() == 7


def test_group_quant_bound_and_grouping(orc):
    w = synth.weights(1, 384, 48, outlier_prob=0.01)
    codes, fs = orc.group_quant_int4(w, 128)
    for l in range(3):
        blk = w[128 * l:128 * (l + 1)]
        np.testing.assert_array_equal(fs[l], (np.abs(blk).max(axis=0) / np.float32(7)).astype(np.float32))
        err = np.abs(blk.astype(np.float64) - fs[l].astype(np.float64) * codes[128 * l:128 * (l + 1)])
        assert np.all(err <= fs[l] * (0.5 + 2.0 ** -20))
    assert codes.min() >= -7 and codes.max() <= 7


# ------------------------------------------------------------------ packed layout

def test_pack_unpack_roundtrip_all_codes(orc):
    K, N = 256, 32
    g = synth.rng(7, 1)
    codes = g.integers(-8, 8, size=(K, N)).astype(np.int8)
    codes[0, :16] = np.arange(-8, 8)
    p = orc.pack_int4(codes)
    assert p.size == N * K // 2
    np.testing.assert_array_equal(orc.unpack_int4(p, K, N), codes)


@pytest.mark.parametrize("k,j,byte,high", [
    (0, 0, 0, False), (4, 0, 0, True), (1, 0, 1, False), (7, 0, 3, True),
    (8, 0, 4, False), (12, 0, 4, True), (15, 0, 7, True),
    (64, 0, 8, False), (16, 0, 256, False), (0, 1, 16, False), (48, 15, 3 * 256 + 15 * 16, False),
    (128, 0, 1024, False), (0, 16, 2 * 1024, False), (127, 31, 2048 + 1023, True),
    (255, 31, 2048 + 1024 + 1023, True),
])
def test_pack_layout_positions(orc, k, j, byte, high):
    # K=256 (G=2), N=32 (2 column tiles): single code 5 at (k, j), all others 0
    K, N = 256, 32
    codes = np.zeros((K, N), np.int8)
    codes[k, j] = 5
    p = orc.pack_int4(codes)
    nz = np.flatnonzero(p)
    assert nz.tolist() == [byte]
    assert p[byte] == (0x50 if high else 0x05)


def test_pack_twos_complement(orc):
    codes = np.zeros((128, 16), np.int8)
    codes[0, 0], codes[4, 0] = -1, -8
    p = orc.pack_int4(codes)
    assert p[0] == 0x8F


def test_canonical_layout_byte_positions(orc):
    # byte (j*K + k)/2, even k low nibble, odd k high nibble, two's complement
    K, N = 256, 32
    for (k, j, v) in [(0, 0, 1), (1, 0, -1), (2, 1, 7), (255, 31, -8), (128, 5, 3), (77, 9, -2)]:
        codes = np.zeros((K, N), np.int8)
        codes[k, j] = v
        p = orc.pack_int4_canonical(codes)
        b = (j * K + k) // 2
        nz = np.flatnonzero(p)
        assert nz.tolist() == [b]
        want = (v & 0xF) << 4 if k % 2 else v & 0xF
        assert int(p[b]) == want


def test_canonical_layout_round_trip_and_native(orc):
    g = synth.rng(11, 3)
    codes = g.integers(-8, 8, size=(384, 48)).astype(np.int8)
    can = orc.pack_int4_canonical(codes)
    assert can.size == 384 * 48 // 2
    np.testing.assert_array_equal(orc.unpack_int4_canonical(can, 384, 48), codes)
    # both layouts hold the same codes: unpacking either gives the matrix back
    np.testing.assert_array_equal(orc.unpack_int4(orc.pack_int4(codes), 384, 48), codes)
    # a column's 16-code runs are contiguous 8-byte runs in the canonical layout
    j, k0 = 7, 192
    run = can[(j * 384 + k0) // 2:(j * 384 + k0) // 2 + 8]
    lo, hi = (run & 0xF).astype(np.int8), (run >> 4).astype(np.int8)
    vals = np.empty(16, np.int8)
    vals[0::2], vals[1::2] = lo, hi
    vals = np.where(vals >= 8, vals - 16, vals)
    np.testing.assert_array_equal(vals, codes[k0:k0 + 16, j])


# --------------------------------------------------------------- amplifier search

@pytest.mark.parametrize("smin", [0.3, 2.0 ** -10, 0.001, 0.0009, 0.5, 0.75, 2.0 ** -20 * 1.5, 0.999])
def test_amplifier_follows_search_rule(orc, smin):
    # the rule the page states: the smallest power of two, from 2^0 up, that brings the
    # smallest (nonzero) scale to at least 1
    rule = golden("amplifier_rule.txt")
    f = np.array([[smin, 0.9, 5.0], [0.0, 1.0, 0.4 + smin]], np.float32)
    n = orc.amplifier_log2(f)
    s = float(np.float32(smin))
    assert n >= rule["min_exponent"]
    assert s * 2 ** n >= rule["stop_threshold"]
    assert n == rule["min_exponent"] or s * 2 ** (n - 1) < rule["stop_threshold"]


def test_amplifier_closed_form_sweep(orc):
    g = synth.rng(3, 3)
    for v in g.uniform(1e-7, 0.999, 500).astype(np.float32):
        m, e = math.frexp(float(v))                     # v = m 2^e, m in [0.5, 1)
        assert orc.amplifier_log2(np.array([v], np.float32)) == 1 - e


def test_amplifier_edges(orc):
    # scales already >= 1: the search starts from 2^0, so the amplifier is 1.
    # Zero scales are ignored.
    assert orc.amplifier_log2(np.array([1.0, 3.0], np.float32)) == 0
    assert orc.amplifier_log2(np.array([0.0, 0.0], np.float32)) == 0
    assert orc.amplifier_log2(np.array([0.0, 0.25], np.float32)) == 2
    assert orc.amplifier_log2(np.array([2.0 ** -40], np.float32), 30) == -1


def test_default_amplifier_and_iscale_width(orc):
    f = golden("is_method_facts.txt")
    assert f["default_amplifier"] == 2 ** f["amplifier_log2"]
    w = synth.weights(0, 1024, 512, outlier_prob=0.001)
    _, fs = orc.group_quant_int4(w, 128)
    isc = orc.integer_scales(fs, f["default_amplifier"])
    assert isc.min() >= 0 and int(isc.max()) < 2 ** f["iscale_bits_max"]
    # round half away on s*alpha, exact product
    prod = fs.astype(np.float64) * f["default_amplifier"]
    assert np.all(np.abs(isc - prod) <= 0.5)
    ties = np.array([[0.5 / 1024, 1.5 / 1024, 2.5 / 1024]], np.float32)
    assert orc.integer_scales(ties, 1024).tolist() == [[1, 2, 3]]


# ------------------------------------------- narrow integer scales, weight MSE

@pytest.mark.parametrize("width,top", [(1, 255), (2, 65535)])
def test_narrow_iscale_bounds_and_identity(orc, width, top):
    # the element holds exactly [0, 2^(8 width) - 1]; stored values are unchanged
    ok = np.array([[0, 1, top - 1, top]], np.int32)
    out, bad = orc.narrow_iscale(ok, width)
    assert bad == 0 and out.dtype == (np.uint8 if width == 1 else np.uint16)
    assert out.astype(np.int64).tolist() == ok.astype(np.int64).tolist()
    for v in (top + 1, -1, 2 ** 23 - 1):
        out, bad = orc.narrow_iscale(np.array([[3, v, 5]], np.int32), width)
        assert out is None and bad == 1
    with pytest.raises(ValueError):
        orc.narrow_iscale(ok, 3)


def test_default_amplifier_scales_fit_8_bits_on_synthetic_layers(orc):
    # the pages find the alpha = 2^10 scales of LLaMA-2-7B within 16 bits, most
    # within 8; the synthetic N(0, 0.02) layers (with 0.1% x10 outliers) fit 8 bits
    w = synth.weights(4, 1024, 512, std=0.02, outlier_prob=0.001, outlier_scale=10.0)
    _, fs = orc.group_quant_int4(w, 128)
    isc = orc.integer_scales(fs, 1024)
    out, bad = orc.narrow_iscale(isc, 1)
    assert bad == 0 and out.max() <= 255


def _mse_case(orc, seed=12, K=512, N=64):
    w = synth.weights(seed, K, N, std=0.02, outlier_prob=0.001, outlier_scale=10.0)
    codes, fs = orc.group_quant_int4(w, 128)
    return codes, fs


def test_weight_mse_zero_when_scales_are_exact(orc):
    # weights built so that s * alpha is an integer: both dequantizations agree exactly
    K, N, alpha = 384, 16, 1024
    g = synth.rng(21, 9)
    m = g.integers(1, 200, size=(K // 128, N))
    w = g.uniform(-1, 1, size=(K, N)).astype(np.float32)
    for l in range(K // 128):
        blk = w[128 * l:128 * (l + 1)]
        blk /= np.abs(blk).max(axis=0)
        blk *= (7.0 * m[l] / alpha).astype(np.float32)
        blk[0] = (7.0 * m[l] / alpha).astype(np.float32)
    codes, fs = orc.group_quant_int4(w, 128)
    isc = orc.integer_scales(fs, alpha)
    mse, mx, wide = orc.weight_mse_is_fs(codes, fs, isc, alpha)
    assert mse == 0.0 and mx == m.max() and wide == 0


@pytest.mark.parametrize("log2a", [4, 8, 10, 14])
def test_weight_mse_rounding_bound(orc, log2a):
    # |S/alpha - s| <= 1/(2 alpha), so MSE <= sum q^2 / (4 alpha^2 K N)
    codes, fs = _mse_case(orc)
    alpha = 1 << log2a
    isc = orc.integer_scales(fs, alpha)
    mse, _, _ = orc.weight_mse_is_fs(codes, fs, isc, alpha)
    q2 = float((codes.astype(np.float64) ** 2).sum())
    bound = q2 / (4.0 * alpha * alpha * codes.size)
    assert 0.0 < mse <= bound * (1 + 1e-12)


def test_weight_mse_scales_as_alpha_squared(orc):
    # once alpha * s spans many integers the rounding errors are uniform on
    # [-1/2, 1/2]: MSE -> E[q^2]/(12 alpha^2), a quarter per doubling of alpha
    codes, fs = _mse_case(orc, K=1024, N=256)
    q2 = float((codes.astype(np.float64) ** 2).mean())
    for log2a in (14, 16, 18):
        alpha = 1 << log2a
        mse, _, _ = orc.weight_mse_is_fs(codes, fs, orc.integer_scales(fs, alpha), alpha)
        assert mse * alpha * alpha == pytest.approx(q2 / 12.0, rel=0.1)


def test_weight_mse_alpha_one_drops_small_scales(orc):
    # alpha = 1 and every s < 1/2: every integer scale rounds to 0, so the
    # integer-scale weights vanish and the MSE is the mean square of q*s
    codes, fs = _mse_case(orc)
    assert fs.max() < 0.5
    isc = orc.integer_scales(fs, 1)
    assert (isc == 0).all()
    mse, mx, _ = orc.weight_mse_is_fs(codes, fs, isc, 1)
    wfs = codes.astype(np.float64) * np.repeat(fs.astype(np.float64), 128, axis=0)
    assert mx == 0
    assert mse == pytest.approx(float((wfs ** 2).mean()), rel=1e-12)


def test_weight_mse_reports_wide_scales(orc):
    codes, fs = _mse_case(orc)
    alpha = 1 << 14
    isc = orc.integer_scales(fs, alpha)
    _, mx, wide = orc.weight_mse_is_fs(codes, fs, isc, alpha)
    assert mx == int(isc.max()) and wide == int((isc > 255).sum()) and wide > 0


def test_scale_table_fixture_relations():
    # the analysis table written from the oracle by tests/golden/make_scale_table.py:
    # each searched amplifier is the smallest 2^n lifting the smallest scale to >= 1,
    # the weight MSE falls as alpha grows (by ~16x per 4x once rounding is uniform),
    # and at alpha = 2^10 every integer scale of these layers fits 8 bits
    path = os.path.join(os.path.dirname(__file__), "golden", "scale_table_synthetic.txt")
    rows = [ln.split("|") for ln in open(path, encoding="utf-8") if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 8
    for r in rows:
        smin, n, mx, wide = float(r[2]), int(r[3]), int(r[4]), int(r[5])
        mse = [float(v) for v in r[6].split()]
        assert smin * 2.0 ** n >= 1.0 > smin * 2.0 ** (n - 1)
        assert all(a >= b for a, b in zip(mse, mse[1:]))
        assert 12.0 < mse[-2] / mse[-1] < 20.0
        assert wide == 0 and mx <= 255


def test_int8_scale_table_fixture_relations():
    # the int8-weight table written from the oracle by tests/golden/make_scale_table.py:
    # the searched amplifier rule holds, the largest integer scale doubles with alpha
    # (round(2x) = 2 round(x) or differs by one), the weight MSE falls as alpha grows,
    # and the output error falls towards the float-scale error
    path = os.path.join(os.path.dirname(__file__), "golden", "scale_table_int8_synthetic.txt")
    lines = open(path, encoding="utf-8").read().splitlines()
    head = [ln for ln in lines if ln.startswith("# scales")][0]
    fields = dict(f.strip().rsplit(" ", 1) for f in head[2:].split("|"))
    smin, n = float(fields["min float scale"]), int(fields["searched log2(alpha)"])
    err_fs = float(fields["float-scale output error"])
    assert smin * 2.0 ** n >= 1.0 > smin * 2.0 ** (n - 1)
    rows = [[float(v) for v in ln.split("|")] for ln in lines if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 6
    for (la0, mx0, _, mse0, e0), (la1, mx1, _, mse1, e1) in zip(rows, rows[1:]):
        assert abs(mx1 - mx0 * 2 ** (la1 - la0)) <= 2 ** (la1 - la0)
        assert mse1 < mse0 and e1 <= e0
    assert rows[-1][4] >= err_fs * 0.999 and rows[-1][4] < err_fs * 1.01
    assert rows[0][4] > 5 * err_fs                # alpha = 2^10 is far too coarse for int8


# ----------------------------------------------------- bf16 output rounding

def test_bf16_ties_to_even_and_exact_values(orc):
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20,
                  2.0 ** -130, 0.0, -0.0], np.float32)
    got = orc.f32_to_bf16_bits(v)
    assert [int(b) for b in got] == [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81, 0x0008, 0x0000, 0x8000]
    # values already representable in bfloat16 are unchanged
    g = np.random.default_rng(3)
    b = g.integers(0, 0x7F80, size=5000).astype(np.uint16)
    b = np.concatenate([b, b | 0x8000]).astype(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits(orc.bf16_bits_to_f32(b)), b)


def test_bf16_half_ulp_bound_monotone_overflow_nan(orc):
    g = np.random.default_rng(4)
    x = (g.standard_normal(20000) * 10.0 ** g.uniform(-30, 30, 20000)).astype(np.float32)
    r = orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(x)).astype(np.float64)
    xd = x.astype(np.float64)
    normal = np.abs(xd) >= 2.0 ** -126
    assert np.all(np.abs(r - xd)[normal] <= np.abs(xd)[normal] * 2.0 ** -8)   # half an ulp of 8 bits
    xs = np.sort(x)
    rs = orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(xs))
    assert np.all(np.diff(rs.astype(np.float64)) >= 0)
    big = np.array([3.4e38, -3.4e38, np.float32(np.finfo(np.float32).max)], np.float32)
    assert [int(b) for b in orc.f32_to_bf16_bits(big)] == [0x7F80, 0xFF80, 0x7F80]
    nan = orc.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(orc.bf16_bits_to_f32(nan)[0])


# -------------------------------------------------------------------- O3 IS GEMM

def _tiny_case(seed, M, K, N, iscale_hi=300):
    g = synth.rng(seed, 50)
    qx = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = g.integers(-7, 8, size=(K, N)).astype(np.int8)
    isc = g.integers(0, iscale_hi, size=(K // 128, N)).astype(np.int32)
    sx = g.uniform(0.001, 0.1, size=M).astype(np.float32)
    return qx, qw, isc, sx


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (2, 256, 3), (3, 256, 2), (3, 384, 5)])
def test_is_brute_force_ungrouped(orc, M, K, N):
    # distributivity: sum_l iscale_l sum_{k in l} qx qw == sum_k qx qw iscale_{l(k)}
    qx, qw, isc, sx = _tiny_case(M * 7 + K + N, M, K, N)
    A, y, ov = orc.w4a8_gemm_is(qx, sx, qw, isc, 1024)
    ref = np.zeros((M, N), np.int64)
    for i in range(M):
        for j in range(N):
            ref[i, j] = sum(int(qx[i, k]) * int(qw[k, j]) * int(isc[k // 128, j]) for k in range(K))
    np.testing.assert_array_equal(A, ref)
    assert ov == 0


def test_is_unit_scales_is_int_matmul(orc):
    qx, qw, _, sx = _tiny_case(1, 9, 512, 20)
    isc = np.ones((4, 20), np.int32)
    A, _, _ = orc.w4a8_gemm_is(qx, sx, qw, isc, 1)
    np.testing.assert_array_equal(A, qx.astype(np.int64) @ qw.astype(np.int64))


def test_is_single_group_is_per_channel(orc):
    qx, qw, isc, sx = _tiny_case(2, 5, 128, 12)
    A, y, _ = orc.w4a8_gemm_is(qx, sx, qw, isc, 1024)
    np.testing.assert_array_equal(A, (qx.astype(np.int64) @ qw.astype(np.int64)) * isc[0][None, :])


def test_is_output_closed_form(orc):
    # y = RN(float(A) * s) * 2^-10; the double product of two floats is exact,
    # so float32(double product) is the single rounding.
    qx, qw, isc, sx = _tiny_case(3, 7, 512, 33, iscale_hi=130)
    A, y, _ = orc.w4a8_gemm_is(qx, sx, qw, isc, 1024)
    Af = A.astype(np.int32).astype(np.float32).astype(np.float64)
    ref = (Af * sx[:, None].astype(np.float64)).astype(np.float32) * np.float32(2.0 ** -10)
    np.testing.assert_array_equal(y, ref)


def test_is_row_col_selection(orc):
    qx, qw, isc, sx = _tiny_case(4, 6, 256, 10)
    A, y, _ = orc.w4a8_gemm_is(qx, sx, qw, isc, 1024)
    rows, cols = [5, 0, 3], [9, 2]
    A2, y2, _ = orc.w4a8_gemm_is(qx, sx, qw, isc, 1024, rows=rows, cols=cols)
    np.testing.assert_array_equal(A2, A[np.ix_(rows, cols)])
    np.testing.assert_array_equal(y2, y[np.ix_(rows, cols)])


def test_is_overflow_flag_and_wrap(orc):
    r = golden("quant_ranges.txt")
    # int32 accumulator ([QB] §1.4); crafted maximal codes push A past 2^31
    M, K, N = 2, 4096, 3
    qx = np.full((M, K), 127, np.int8)
    qw = np.full((K, N), 7, np.int8)
    isc = np.full((K // 128, N), 600, np.int32)
    isc[:, 2] = 500
    sx = np.ones(M, np.float32)
    A, y, ov = orc.w4a8_gemm_is(qx, sx, qw, isc, 1)
    assert A[0, 0] == 32 * 128 * 127 * 7 * 600 and A[0, 0] >= 2 ** (r["accumulator_bits"] - 1)
    assert A[0, 2] < 2 ** 31
    assert ov == M * 2
    wrapped = ((A[0, 0] + 2 ** 31) % 2 ** 32) - 2 ** 31
    assert y[0, 0] == np.float32(wrapped)


def test_is_equals_fs_when_scales_are_exact(orc):
    # weights built so that s * alpha is an integer: then integer and float scales agree
    # exactly (every partial float sum is a multiple of 2^-10 below 2^24 * 2^-10)
    M, K, N = 4, 512, 24
    g = synth.rng(9, 9)
    m = g.integers(1, 200, size=(K // 128, N))
    w = g.uniform(-1, 1, size=(K, N)).astype(np.float32)
    for l in range(K // 128):
        blk = w[128 * l:128 * (l + 1)]
        blk /= np.abs(blk).max(axis=0)
        blk *= (7.0 * m[l] / 1024.0).astype(np.float32)
        blk[0] = (7.0 * m[l] / 1024.0).astype(np.float32)
    codes, fs = orc.group_quant_int4(w, 128)
    np.testing.assert_array_equal(fs.astype(np.float64) * 1024, m)
    isc = orc.integer_scales(fs, 1024)
    x = synth.activations(9, M, K)
    qx, sx = orc.quant_sym_i8(x)
    _, y_is, _ = orc.w4a8_gemm_is(qx, sx, codes, isc, 1024)
    y_fs = orc.w4a8_gemm_fs(qx, sx, codes, fs)
    np.testing.assert_array_equal(y_is, y_fs)


def _dequant_matmul(qx, sx, codes, fs):
    wq = codes.astype(np.float64) * np.repeat(fs.astype(np.float64), 128, axis=0)
    return (qx.astype(np.float64) * sx[:, None].astype(np.float64)) @ wq


def test_is_error_bound_vs_float_scales(orc):
    # |y_IS - y_exact| <= s_i/alpha * sum_l |p_l| |iscale - alpha s_l| + fp32 rounding
    x, w = synth.single_gemm_inputs(0)
    x, w = x[:4], w[:, :96]
    codes, fs = orc.group_quant_int4(w)
    isc = orc.integer_scales(fs, 1024)
    qx, sx = orc.quant_sym_i8(x)
    _, y, _ = orc.w4a8_gemm_is(qx, sx, codes, isc, 1024)
    exact = _dequant_matmul(qx, sx, codes, fs)
    G = fs.shape[0]
    p = np.stack([qx[:, 128 * l:128 * (l + 1)].astype(np.int64) @ codes[128 * l:128 * (l + 1)].astype(np.int64)
                  for l in range(G)])                       # G x M x N
    dev = np.abs(isc.astype(np.float64) - 1024 * fs.astype(np.float64))   # G x N
    bound = sx[:, None] / 1024.0 * np.einsum("lmn,ln->mn", np.abs(p), dev)
    bound += np.abs(exact) * 2.0 ** -22 + 1e-30
    assert np.all(np.abs(y - exact) <= bound)


def test_is_full_path_approximates_matmul(orc):
    # the method approximates Y = X W ([IS] 方法 Fig. 3): relative Frobenius error of the
    # W4A8 integer-scale path against the float64 product stays at int4 rounding level
    x, w = synth.single_gemm_inputs(0)
    x, w = x[:8], w[:, :256]
    pw = orc.pack_weights(w, 128, 1024)
    qx, sx = orc.quant_sym_i8(x)
    _, y, _ = orc.w4a8_gemm_is(qx, sx, pw["codes"], pw["iscale"], pw["alpha"])
    ref = x.astype(np.float64) @ w.astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.2          # int4 weights: a few percent, never exact


# -------------------------------------------------------------------- O4 FS GEMM

def test_fs_fma_chain_small_case(orc):
    # two groups, hand-checkable: p0 = 3, p1 = -2 with scales 0.5, 0.25 -> 1.0, times s=2
    qx = np.zeros((1, 256), np.int8)
    qw = np.zeros((256, 16), np.int8)
    qx[0, 0], qw[0, 0] = 3, 1
    qx[0, 130], qw[130, 0] = -2, 1
    fs = np.full((2, 16), 0.5, np.float32)
    fs[1, 0] = 0.25
    y = orc.w4a8_gemm_fs(qx, np.array([2.0], np.float32), qw, fs)
    assert y[0, 0] == np.float32(2.0) and not y[0, 1:].any()


def test_fs_close_to_exact(orc):
    x, w = synth.single_gemm_inputs(1)
    x, w = x[:3], w[:, :64]
    codes, fs = orc.group_quant_int4(w)
    qx, sx = orc.quant_sym_i8(x)
    y = orc.w4a8_gemm_fs(qx, sx, codes, fs)
    exact = _dequant_matmul(qx, sx, codes, fs)
    G = fs.shape[0]
    mag = _dequant_matmul(np.abs(qx), sx, np.abs(codes), fs)
    assert np.all(np.abs(y - exact) <= (G + 2) * 2.0 ** -24 * mag + 1e-30)


# ------------------------------------------------------------------- O5 W8A8 ZP

def _w8a8_case(orc, seed, M, K, N, relu=False):
    x, w = synth.w8a8_inputs(seed, M, K, N, relu=relu)
    qx, sx, zx, rx = orc.quant_asym_u8(x)
    qw, sw, zw, cw = orc.quant_asym_u8(np.ascontiguousarray(w.T))
    return x, w, (qx, sx, zx, rx, qw, sw, zw, cw)


def test_w8a8_expansion_identity(orc):
    # [QN] 矩阵乘法中的量化计算: the expanded four-term form equals the direct
    # product of zero-point-shifted codes, exactly in integers
    _, _, (qx, sx, zx, rx, qw, sw, zw, cw) = _w8a8_case(orc, 0, 7, 384, 21)
    A, y, ov = orc.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw)
    direct = (qx.astype(np.int64) - zx[:, None]) @ (qw.astype(np.int64) - zw[:, None]).T
    np.testing.assert_array_equal(A, direct)
    assert ov == 0
    assert zx.min() > 0 and zw.min() > 0                      # all four terms live
    ref = (A.astype(np.float32) * (sx[:, None] * sw[None, :])).astype(np.float32)
    np.testing.assert_array_equal(y, ref)


def test_w8a8_zero_points_zero_reduce_to_plain_product(orc):
    g = synth.rng(2, 2)
    qx = g.integers(0, 256, size=(5, 256)).astype(np.uint8)
    qw = g.integers(0, 256, size=(6, 256)).astype(np.uint8)
    z5, z6 = np.zeros(5, np.int32), np.zeros(6, np.int32)
    A, _, _ = orc.w8a8_gemm_zp(qx, np.ones(5, np.float32), z5, qx.sum(1).astype(np.int32),
                               qw, np.ones(6, np.float32), z6, qw.sum(1).astype(np.int32))
    np.testing.assert_array_equal(A, qx.astype(np.int64) @ qw.astype(np.int64).T)


def test_w8a8_recentred_codes_same_accumulator(orc):
    # shifting codes and zero points by 128 leaves every (q - z) unchanged
    _, _, (qx, sx, zx, rx, qw, sw, zw, cw) = _w8a8_case(orc, 1, 4, 256, 9)
    A, _, _ = orc.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw)
    sx_ = (qx.astype(np.int64) - 128)
    sw_ = (qw.astype(np.int64) - 128)
    direct = (sx_ - (zx[:, None] - 128)) @ (sw_ - (zw[:, None] - 128)).T
    np.testing.assert_array_equal(A, direct)
    assert np.abs(A).max() <= 256 * 255 ** 2


def test_w8a8_relu_activations_zero_point_zero(orc):
    x, w, (qx, sx, zx, rx, qw, sw, zw, cw) = _w8a8_case(orc, 0, 16, 256, 8, relu=True)
    assert np.all(zx == 0)
    A, y, _ = orc.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.05


def test_w8a8_approximates_matmul(orc):
    x, w, (qx, sx, zx, rx, qw, sw, zw, cw) = _w8a8_case(orc, 3, 16, 512, 32)
    _, y, _ = orc.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.05


# ------------------------------------------------- fine-grained W8A8 integer scale
# [IS] 5.4 (the LLaMA-3 scheme): 8-bit group-wise weights for the down projection,
# with the same integer-scale epilogue.

def test_group_quant_int8_hand_group(orc):
    # absmax 127 -> s = 1; ties away from zero; clip [-127, 127]
    w = np.zeros((128, 16), np.float32)
    w[:8, 0] = [127.0, 63.5, -63.5, 0.5, -0.49, -127.0, 126.6, 2.5]
    w[:, 1] = np.linspace(-1, 1, 128)
    codes, fs = orc.group_quant_int8(w, 128)
    assert fs[0, 0] == 1.0
    assert codes[:8, 0].tolist() == [127, 64, -64, 1, 0, -127, 127, 3]
    assert fs[0, 2] == 0 and not codes[:, 2].any()          # all-zero group
    assert codes[:, 1].min() == -127 and codes[:, 1].max() == 127
    # the int4 quantizer on the same group differs (q_max 7): not a shared constant
    c4, f4 = orc.group_quant_int4(w, 128)
    assert f4[0, 0] == np.float32(127.0 / 7.0) and c4[:8, 0].max() == 7


def test_group_quant_int8_bound_and_grouping(orc):
    w = synth.weights(2, 384, 48, outlier_prob=0.01)
    codes, fs = orc.group_quant_int8(w, 128)
    for l in range(3):
        blk = w[128 * l:128 * (l + 1)]
        np.testing.assert_array_equal(fs[l], (np.abs(blk).max(axis=0) / np.float32(127)).astype(np.float32))
        err = np.abs(blk.astype(np.float64) - fs[l].astype(np.float64) * codes[128 * l:128 * (l + 1)])
        assert np.all(err <= fs[l] * (0.5 + 2.0 ** -20))
        # the group's absmax element maps to +-127
        assert np.all(np.abs(codes[128 * l:128 * (l + 1)]).max(axis=0) == 127)
    assert codes.min() >= -127 and codes.max() <= 127


def test_int8_layout_roundtrip_and_permutation(orc):
    K, N = 384, 48
    codes = synth.rng(11, 3).integers(-127, 128, size=(K, N)).astype(np.int8)
    qw = orc.layout_int8(codes)
    assert qw.size == N * K
    np.testing.assert_array_equal(np.sort(qw), np.sort(codes.ravel()))
    np.testing.assert_array_equal(orc.unlayout_int8(qw, K, N), codes)


@pytest.mark.parametrize("k,j,byte", [
    (0, 0, 0), (1, 0, 1), (15, 0, 15), (16, 0, 256), (0, 1, 16), (64, 0, 1024),
    (128, 0, 2048), (0, 16, 4096), (100, 5, 1620), (255, 31, 8191),
])
def test_int8_layout_positions(orc, k, j, byte):
    # K=256 (G=2), N=32 (2 column tiles): a single code 9 at (k, j)
    K, N = 256, 32
    codes = np.zeros((K, N), np.int8)
    codes[k, j] = 9
    qw = orc.layout_int8(codes)
    assert np.flatnonzero(qw).tolist() == [byte]


def test_w8is_brute_force_ungrouped(orc):
    # full int8 weight range; distributivity against a per-k brute force
    M, K, N = 3, 384, 4
    g = synth.rng(12, 5)
    qx = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = g.integers(-127, 128, size=(K, N)).astype(np.int8)
    isc = g.integers(0, 70, size=(K // 128, N)).astype(np.int32)
    sx = g.uniform(0.001, 0.1, size=M).astype(np.float32)
    A, _, ov = orc.w8a8_gemm_is(qx, sx, qw, isc, 1 << 14)
    ref = np.zeros((M, N), np.int64)
    for i in range(M):
        for j in range(N):
            ref[i, j] = sum(int(qx[i, k]) * int(qw[k, j]) * int(isc[k // 128, j]) for k in range(K))
    np.testing.assert_array_equal(A, ref)
    assert ov == 0


def test_w8is_unit_scales_is_int_matmul_and_group_bound(orc):
    g = synth.rng(13, 5)
    qx = g.integers(-127, 128, size=(5, 512)).astype(np.int8)
    qw = g.integers(-127, 128, size=(512, 20)).astype(np.int8)
    A, _, _ = orc.w8a8_gemm_is(qx, np.ones(5, np.float32), qw, np.ones((4, 20), np.int32), 1)
    np.testing.assert_array_equal(A, qx.astype(np.int64) @ qw.astype(np.int64))
    # one group's |p| stays below 2^23 even at the extreme codes
    ext = np.full((1, 128), -127, np.int8)
    A1, _, _ = orc.w8a8_gemm_is(ext, np.ones(1, np.float32), np.full((128, 16), 127, np.int8),
                                np.ones((1, 16), np.int32), 1)
    assert A1[0, 0] == -128 * 127 * 127 and abs(A1[0, 0]) < 2 ** 23


def test_w8is_overflow_flag(orc):
    K, N = 1024, 2
    qx = np.full((1, K), 127, np.int8)
    qw = np.full((K, N), 127, np.int8)
    isc = np.full((K // 128, N), 200, np.int32)
    isc[:, 1] = 100
    A, y, ov = orc.w8a8_gemm_is(qx, np.ones(1, np.float32), qw, isc, 1)
    assert A[0, 0] == 8 * 128 * 127 * 127 * 200 and A[0, 0] >= 2 ** 31
    assert A[0, 1] < 2 ** 31 and ov == 1


def test_w8is_error_bound_and_accuracy(orc):
    # |y_IS - y_FS-exact| <= s_i/alpha * sum_l |p_l| |iscale - alpha s_l| + rounding; at
    # alpha = 2^18 the integer scales (still below 2^8 here) cost almost nothing over the
    # float scales, and the int8 path is much closer to X W than the int4 one
    x, w = synth.single_gemm_inputs(0)
    x, w = x[:4], w[:, :96]
    alpha = 1 << 18
    pw = orc.pack_weights_int8(w, 128, alpha)
    codes, fs, isc = pw["codes"], pw["fscale"], pw["iscale"]
    qx, sx = orc.quant_sym_i8(x)
    _, y, ov = orc.w8a8_gemm_is(qx, sx, codes, isc, alpha)
    assert ov == 0
    exact = _dequant_matmul(qx, sx, codes, fs)
    G = fs.shape[0]
    p = np.stack([qx[:, 128 * l:128 * (l + 1)].astype(np.int64) @ codes[128 * l:128 * (l + 1)].astype(np.int64)
                  for l in range(G)])
    dev = np.abs(isc.astype(np.float64) - alpha * fs.astype(np.float64))
    bound = sx[:, None] / alpha * np.einsum("lmn,ln->mn", np.abs(p), dev)
    bound += np.abs(exact) * 2.0 ** -22 + 1e-30
    assert np.all(np.abs(y - exact) <= bound)
    assert isc.max() <= 255
    ref = x.astype(np.float64) @ w.astype(np.float64)
    rel8 = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    relfs = np.linalg.norm(orc.w4a8_gemm_fs(qx, sx, codes, fs) - ref) / np.linalg.norm(ref)
    p4 = orc.pack_weights(w, 128, 1024)
    _, y4, _ = orc.w4a8_gemm_is(qx, sx, p4["codes"], p4["iscale"], 1024)
    rel4 = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    assert rel8 <= 1.02 * relfs and rel8 < rel4 / 2


def test_w8is_searched_alpha_rule(orc):
    # alpha 0 runs the same search as for int4: smallest 2^n with min scale * 2^n >= 1
    w = synth.weights(3, 256, 32, outlier_prob=0.001)
    pw = orc.pack_weights_int8(w, 128, 0)
    smin = pw["fscale"][pw["fscale"] > 0].min()
    a = pw["alpha"]
    assert smin * a >= 1 and smin * (a // 2) < 1
    assert pw["iscale"].min() >= 1


# ------------------------------------------- grouped (mixture-of-experts) IS GEMM
# [IS] 5.3: the integer-scale W4A8 layer applied to the experts of Mixtral 8x7B.

def _moe_case(seed, T, E, K, N, topk=2):
    g = synth.rng(seed, 60)
    qx = g.integers(-127, 128, size=(T, K)).astype(np.int8)
    sx = g.uniform(0.001, 0.1, size=T).astype(np.float32)
    codes = g.integers(-7, 8, size=(E, K, N)).astype(np.int8)
    isc = g.integers(0, 300, size=(E, K // 128, N)).astype(np.int32)
    offs, tok = synth.route_by_expert(synth.moe_routing(seed, T, E, topk), E)
    return qx, sx, codes, isc, offs, tok


def test_moe_routing_is_a_valid_top_k(orc):
    ex = synth.moe_routing(3, 50, 8, 2)
    assert ex.shape == (50, 2) and ex.min() >= 0 and ex.max() < 8
    assert np.all(ex[:, 0] != ex[:, 1])
    offs, tok = synth.route_by_expert(ex, 8)
    assert offs[0] == 0 and offs[-1] == 100 and np.all(np.diff(offs) >= 0)
    np.testing.assert_array_equal(np.bincount(tok, minlength=50), np.full(50, 2))
    for e in range(8):
        t = tok[offs[e]:offs[e + 1]]
        assert np.all(np.diff(t) > 0)                      # tokens ascending, no repeats
        assert all(e in ex[i] for i in t)


def test_moe_single_expert_is_the_dense_gemm(orc):
    qx, sx, codes, isc, _, _ = _moe_case(4, 9, 1, 256, 32, topk=1)
    offs = np.array([0, 9], np.int32)
    tok = np.arange(9, dtype=np.int32)
    A, y, ov = orc.moe_w4a8_gemm_is(qx, sx, codes, isc, 1024, offs, tok)
    A0, y0, ov0 = orc.w4a8_gemm_is(qx, sx, codes[0], isc[0], 1024)
    np.testing.assert_array_equal(A, A0)
    np.testing.assert_array_equal(y, y0)
    assert ov == ov0 == 0


def test_moe_each_slot_is_its_token_times_its_expert(orc):
    T, E, K, N = 6, 4, 256, 16
    qx, sx, codes, isc, offs, tok = _moe_case(5, T, E, K, N)
    A, y, _ = orc.moe_w4a8_gemm_is(qx, sx, codes, isc, 1024, offs, tok)
    for e in range(E):
        for r in range(offs[e], offs[e + 1]):
            t = tok[r]
            # brute force with Python integers over k (independent of the grouping code)
            for j in range(N):
                ref = sum(int(qx[t, k]) * int(codes[e, k, j]) * int(isc[e, k // 128, j]) for k in range(K))
                assert A[r, j] == ref
            Ar, yr, _ = orc.w4a8_gemm_is(qx[t:t + 1], sx[t:t + 1], codes[e], isc[e], 1024)
            np.testing.assert_array_equal(y[r], yr[0])


def test_moe_token_permutation_permutes_rows(orc):
    # relabelling the tokens (and the routing with them) leaves each slot's row unchanged
    T, E, K, N = 12, 8, 128, 32
    qx, sx, codes, isc, offs, tok = _moe_case(6, T, E, K, N)
    _, y, _ = orc.moe_w4a8_gemm_is(qx, sx, codes, isc, 1024, offs, tok)
    perm = synth.rng(6, 61).permutation(T)
    inv = np.argsort(perm)
    _, y2, _ = orc.moe_w4a8_gemm_is(qx[perm], sx[perm], codes, isc, 1024, offs, inv[tok].astype(np.int32))
    np.testing.assert_array_equal(y, y2)


def test_moe_experts_without_tokens(orc):
    T, E, K, N = 1, 8, 128, 16
    qx, sx, codes, isc, offs, tok = _moe_case(7, T, E, K, N)
    assert (np.diff(offs) > 0).sum() == 2                  # one token reaches two experts
    A, y, _ = orc.moe_w4a8_gemm_is(qx, sx, codes, isc, 1024, offs, tok)
    assert A.shape == (2, N)
