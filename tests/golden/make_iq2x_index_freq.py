"""Writes iq2x_index_freq.txt: how often the oracle's iq2x quantizer picks each row of the seeded codebook
(synth.codebook(0)) on N(0, 0.02) weights.  The full-size workloads draw their codebook indices from these
frequencies (synth.random_blocks), so their lookup patterns are those of quantized weights.

    python tests/golden/make_iq2x_index_freq.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth   # noqa: E402


def main():
    cb = synth.codebook(0)
    w = (np.random.default_rng([2024, 7]).standard_normal(1024 * 4096) * 0.02).astype(np.float32)
    blocks = oracle.quantize(oracle.FMT_IQ2X, w, cb).reshape(-1, 66)
    idx = blocks[:, 2:].reshape(-1, 8, 8)[:, :, 0:4].reshape(-1)      # idx[4] of each 8-byte group record
    counts = np.bincount(idx, minlength=256)
    with open(os.path.join(HERE, "iq2x_index_freq.txt"), "w") as f:
        f.write("# Codebook-row counts of the oracle's iq2x quantizer on 1024 x 4096 N(0, 0.02) weights (seed [2024, 7])\n")
        f.write("# with the seeded codebook synth.codebook(0); written by make_iq2x_index_freq.py.  Row r's count is\n")
        f.write("# on line r (0-based, after these comments).\n")
        for c in counts:
            f.write(f"{int(c)}\n")


if __name__ == "__main__":
    main()
