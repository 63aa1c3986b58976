"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

A separate build of oracle/oracle.c with -fsanitize=address,undefined runs
the pins' tiny cases in a child process (the sanitizer runtime must be
loaded first, so the child preloads it); any out-of-bounds access, leak or
undefined operation aborts the child and fails the test. CPU only.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.timeout(300)
def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("ASan runtime not available")
    so = tmp_path / "liborc_san.so"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(so), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import oracle
        oracle._LIB = {str(so)!r}
        import numpy as np, synth
        x = synth.activations(1, 5, 384)
        q, s = oracle.quant_sym_i8(x)
        qa, sa, za, ra = oracle.quant_asym_u8(x)
        w = synth.weights(2, 384, 48, outlier_prob=0.01)
        pw = oracle.pack_weights(w, 128, 0)
        codes = oracle.unpack_int4(pw["packed"], 384, 48)
        assert (codes == pw["codes"]).all()
        can = oracle.pack_int4_canonical(pw["codes"])
        assert (oracle.unpack_int4_canonical(can, 384, 48) == pw["codes"]).all()
        A, y, ov = oracle.w4a8_gemm_is(q, s, pw["codes"], pw["iscale"], pw["alpha"])
        yf = oracle.w4a8_gemm_fs(q, s, pw["codes"], pw["fscale"])
        p8 = oracle.pack_weights_int8(w, 128, 1 << 16)
        A8, y8, _ = oracle.w8a8_gemm_is(q, s, p8["codes"], p8["iscale"], 1 << 16)
        wt = np.ascontiguousarray(w.T)
        qw, sw, zw, cw = oracle.quant_asym_u8(wt)
        Az, yz, _ = oracle.w8a8_gemm_zp(qa, sa, za, ra, qw, sw, zw, cw)
        offs = np.array([0, 3, 3, 7], np.int32)
        tok = np.array([0, 4, 2, 1, 1, 3, 0], np.int32)
        cs = np.stack([pw["codes"]] * 3)
        isc = np.stack([pw["iscale"]] * 3)
        Am, ym, _ = oracle.moe_w4a8_gemm_is(q, s, cs, isc, pw["alpha"], offs, tok)
        n = oracle.narrow_iscale(pw["iscale"], 2)
        b = oracle.f32_to_bf16_bits(y.astype(np.float32))
        mse = oracle.weight_mse_is_fs(pw["codes"], pw["fscale"], pw["iscale"], pw["alpha"])
        assert oracle._lib._name == {str(so)!r}
        print("sanitized oracle ok", flush=True)
    """)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + ((" " + _runtime("libubsan.so")) if _runtime("libubsan.so") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
