"""Writes scale_table_synthetic.txt: the integer-scale analysis of the
"Integer Scale" page's Fig. 4 (amplified-scale width, amplifier search per
layer, weight MSE between integer and float scales under several amplifiers)
on the synthetic layers; and scale_table_int8_synthetic.txt, the same for the
fine-grained int8 weights of the page's LLaMA-3 scheme (5.4), with the relative
error of the whole W8A8 path against X.W. Calls only the CPU oracle and the
seeded generators.

    python tests/golden/make_scale_table.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

LOG2_ALPHAS = (4, 6, 8, 10, 12, 14)


def layers():
    for li, (name, k, n) in enumerate(synth.LLAMA2_7B_BLOCK):
        yield (f"llama2-7b {name} {k}x{n}",
               lambda k=k, n=n, li=li: synth.weights(0, k, n, std=0.02, stream=synth.STREAM_LAYER + li))
    yield (f"decode layer {synth.K_LAYER}x{synth.N_LAYER} (0.1% x10)",
           lambda: synth.layer_inputs(0, M=1)[1])


def main():
    oracle.build()
    rows = []
    for name, make in layers():
        w = make()
        codes, fs = oracle.group_quant_int4(w, synth.GROUP)
        del w
        smin = float(fs[fs > 0].min())
        n = oracle.amplifier_log2(fs)
        isc = oracle.integer_scales(fs, 1024)
        _, mx, wide = oracle.weight_mse_is_fs(codes, fs, isc, 1024)
        mses = []
        for la in LOG2_ALPHAS:
            a = 1 << la
            mses.append(oracle.weight_mse_is_fs(codes, fs, oracle.integer_scales(fs, a), a)[0])
        rows.append((name, fs.size, smin, n, mx, wide, mses))
        print(name, "done", flush=True)
    out = os.path.join(HERE, "scale_table_synthetic.txt")
    with open(out, "w") as f:
        f.write("# Integer-scale analysis of the synthetic layers (the Fig. 4 analogue of the\n"
                "# \"Integer Scale\" page, 方法): written by tests/golden/make_scale_table.py from the\n"
                "# CPU oracle; weights N(0, 0.02) (decode layer: with 0.1% of elements x10), group 128.\n"
                "# columns: layer | scales | min float scale | searched log2(alpha) |\n"
                "#          max integer scale at alpha=2^10 | scales above 255 at 2^10 |\n"
                "#          weight MSE (integer vs float scales) at alpha = "
                + ", ".join(f"2^{la}" for la in LOG2_ALPHAS) + "\n")
        for name, cnt, smin, n, mx, wide, mses in rows:
            f.write(f"{name} | {cnt} | {smin:.6g} | {n} | {mx} | {wide} | "
                    + " ".join(f"{m:.4g}" for m in mses) + "\n")
    print("wrote", out)
    int8_table()


LOG2_ALPHAS_8 = (10, 12, 14, 15, 16, 18)


def int8_table():
    """The int8-weight analogue on 512 columns of the synthetic LLaMA-3-8B down
    projection (14336 x 4096, 0.1% of weights x10) with 16 tokens of the
    synthetic activations: per amplifier, the largest integer scale, how many
    exceed 8 bits, the weight MSE against float scales, and the relative
    Frobenius error of the integer-scale W8A8 output against X.W (float
    scales: the last column of the header line)."""
    K, N, M = 14336, 512, 16
    w = synth.weights(901, K, N, std=0.02, outlier_prob=0.001)
    x = synth.activations(900, M, K)
    codes, fs = oracle.group_quant_int8(w, synth.GROUP)
    qx, sx = oracle.quant_sym_i8(x)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    nref = np.linalg.norm(ref)
    y_fs = oracle.w4a8_gemm_fs(qx, sx, codes, fs)
    rel_fs = np.linalg.norm(y_fs - ref) / nref
    n = oracle.amplifier_log2(fs)
    smin = float(fs[fs > 0].min())
    out = os.path.join(HERE, "scale_table_int8_synthetic.txt")
    with open(out, "w") as f:
        f.write("# Integer scales for fine-grained int8 weights (q_max 127), the W8A8 scheme of the\n"
                "# \"Integer Scale\" page (5.4 LLaMA-3): written by tests/golden/make_scale_table.py from\n"
                "# the CPU oracle; 512 columns of a synthetic 14336x4096 down projection, N(0, 0.02)\n"
                "# with 0.1% of elements x10, group 128; 16 synthetic tokens.\n"
                f"# scales {fs.size} | min float scale {smin:.6g} | searched log2(alpha) {n} | "
                f"float-scale output error {rel_fs:.5f}\n"
                "# columns: log2(alpha) | max integer scale | scales above 255 | "
                "weight MSE (integer vs float scales) | output error vs X.W\n")
        for la in LOG2_ALPHAS_8:
            a = 1 << la
            isc = oracle.integer_scales(fs, a)
            mse, mx, wide = oracle.weight_mse_is_fs(codes, fs, isc, a)
            _, y, ov = oracle.w8a8_gemm_is(qx, sx, codes, isc, a)
            assert ov == 0
            rel = np.linalg.norm(y - ref) / nref
            f.write(f"{la} | {mx} | {wide} | {mse:.4g} | {rel:.5f}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
