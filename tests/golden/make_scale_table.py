"""Writes scale_table_synthetic.txt: the integer-scale analysis of the
"Integer Scale" page's Fig. 4 (amplified-scale width, amplifier search per
layer, weight MSE between integer and float scales under several amplifiers)
on the synthetic layers. Calls only the CPU oracle and the seeded generators.

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


if __name__ == "__main__":
    main()
