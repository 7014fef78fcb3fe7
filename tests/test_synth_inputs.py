"""The seeded input generators (synth/): fixed draws, so the workloads the parity tests and the benchmark use are
the same from run to run and machine to machine."""
import hashlib
import os

import numpy as np

import synth


def _golden():
    out = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "codebook.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def test_codebook_is_the_recorded_draw():
    cb = np.ascontiguousarray(synth.codebook(0))
    g = _golden()
    assert cb.shape == (256, 8) and cb.dtype == np.uint8
    assert hashlib.sha256(cb.tobytes()).hexdigest() == g["sha256"][0]
    counts = {int(k): int(v) for k, v in (c.split(":") for c in g["counts"])}
    assert {m: int((cb == m).sum()) for m in (1, 2, 3)} == counts


def test_codebook_entries_are_exact_fp4_magnitudes():
    cb = synth.codebook(0)
    assert set(np.unique(cb).tolist()) <= {1, 2, 3}


def test_activations_are_reproducible():
    a = synth.activations("decode", 4, 4096, True)
    b = synth.activations("decode", 4, 4096, True)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
