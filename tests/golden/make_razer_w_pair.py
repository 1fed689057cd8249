"""Offline search for the second special-value pair of RaZeR for weights.

"RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
Remapping", technical summary sec. 2.2: with the two bits freed by an E3M3
block scale, a weight block chooses one of four special values, two pairs
computed offline; special values are multiples of 0.5, and +-5 is the best
single pair. The pages do not give the second pair, so it is searched here:
every multiple of 0.5 that is neither an E2M1 magnitude nor 5 and lies below
the largest scaled magnitude (about 6.4), on the synthetic Llama-70B-shaped
weights (0.02 N(0,1) with 0.1% outliers x20, 512 rows of each of the seven
tensors, seeds 400 + t). The pair with the highest SQNR is written to
razer_w_pair.txt. Calls only the oracle.

    python tests/golden/make_razer_w_pair.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from block_scaled_fp4_absmax_amd import inputs  # noqa: E402

CANDIDATES = [2.5, 3.5, 4.5, 5.5]
ROWS = 512


def main():
    oracle.build(force=False)
    oracle.set_threads(os.cpu_count() or 1)
    xs = [inputs.gen_c5(t, rows=ROWS) for t in range(len(inputs.C5_SHAPES))]
    xf = [inputs.bf16_bits_to_f32(x).astype(np.float64) for x in xs]
    energy = sum(float((v * v).sum()) for v in xf)

    def sqnr(decode):
        err = sum(float(((v - decode(x)) ** 2).sum()) for x, v in zip(xs, xf))
        return 10 * np.log10(energy / err)

    rows = []

    def nv(razer):
        def dec(x):
            c, s, t = oracle.nv_quantize(x, razer)
            return oracle.dequantize_f64(c, s, 1, int(razer), t)
        return dec

    rows.append(("nvfp4 e4m3, plain", sqnr(nv(False))))
    rows.append(("nvfp4 e4m3, razer +-5", sqnr(nv(True))))
    results = {}
    for p in CANDIDATES:
        def dec(x, p=p):
            c, s, t = oracle.nvw_quantize(x, p)
            return oracle.dequantize_f64(c, s, 1, 2, t, p)
        results[p] = sqnr(dec)
        rows.append((f"e3m3, razer +-5 and +-{p}", results[p]))
    best = max(CANDIDATES, key=lambda p: (results[p], -p))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "razer_w_pair.txt")
    with open(out, "w") as f:
        f.write("# Second special-value pair of RaZeR for weights (E3M3 block scale, 2-bit\n"
                "# selector over {+5, -5, +p, -p}). Not on the pages: chosen offline by\n"
                "# tests/golden/make_razer_w_pair.py (oracle only) as the multiple of 0.5\n"
                f"# with the best SQNR on {ROWS} rows of each synthetic Llama-70B-shaped\n"
                "# weight tensor (0.02 N(0,1), 0.1% outliers x20, seeds 400 + t).\n"
                "# SQNR dB over all seven tensors:\n")
        for name, v in rows:
            f.write(f"#   {name}: {v:.4f}\n")
        f.write(f"pair {best}\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
