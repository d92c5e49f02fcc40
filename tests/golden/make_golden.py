"""Writes the golden fixtures in this directory.  Calls only oracle/ (and the
seeded input generator), never the HIP library.

    python tests/golden/make_golden.py

codec_tables.txt  frequency / cumulative / fp16 reconstruction tables of the
                  four default codecs (levels 8 and 6 at 34 and 29 bytes).
small_encode.txt  containers and fp16 norms of a small seeded K and V batch
                  (8 tokens, 2 kv heads, outlier-channel data) under the
                  34-byte codecs, as hex.
The pages print no worked example, so these files are regression fixtures of
the oracle itself (they freeze its behaviour; the mathematical pins live in
tests/test_oracle_pins.py).
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import synth  # noqa: E402


def tables_text():
    lines = ["# levels C step64 | freq | cum | recon_f16_hex"]
    for (levels, C), step in sorted(O.DEFAULT_STEP64.items()):
        t = O.Codec(levels, C, seed=0, hkv=1).tables()
        lines.append(f"{levels} {C} {step} | {' '.join(map(str, t['freq']))} | "
                     f"{' '.join(map(str, t['cum']))} | "
                     f"{' '.join(f'{int(r):04x}' for r in t['recon_f16'])}")
    return "\n".join(lines) + "\n"


def small_encode_text():
    lines = ["# stream levels C seed | head token | norm_f16_hex | container_hex"]
    K = synth.kv_tensor("outlier", 8, 2, seed=42)
    V = synth.kv_tensor("outlier", 8, 2, seed=43)
    for name, x, levels in (("K", K, 8), ("V", V, 6)):
        codec = O.Codec(levels, 34, seed=7, hkv=2)
        cont, norm, _ = O.encode(codec, x)
        for g in range(2):
            for t in range(8):
                lines.append(f"{name} {levels} 34 7 | {g} {t} | {int(norm[g, t]):04x} | "
                             f"{bytes(cont[g, t]).hex()}")
    return "\n".join(lines) + "\n"


def main():
    with open(os.path.join(HERE, "codec_tables.txt"), "w") as f:
        f.write(tables_text())
    with open(os.path.join(HERE, "small_encode.txt"), "w") as f:
        f.write(small_encode_text())


if __name__ == "__main__":
    main()
