"""Pins for the oracle's number conversions and block formats (CPU only).

The conversions are checked against library casts (numpy float16, torch
bfloat16) over every 16-bit pattern; the formats against hand-worked blocks in
tests/golden/format_blocks.txt and against properties every decoded weight
must have.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

FMT = {"iq2x": oracle.FMT_IQ2X, "q2k": oracle.FMT_Q2K, "q4k": oracle.FMT_Q4K}


def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy_cast():
    rng = np.random.default_rng(0)
    # every finite f16 value, the midpoints between neighbours (ties), and random doubles
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    h = h[np.isfinite(h)]
    hs = np.sort(np.unique(h))
    mids = (hs[1:] + hs[:-1]) / 2
    rnd = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                          rng.uniform(-70000, 70000, 2000)])
    xs = np.concatenate([hs, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), rnd, [65519.9, 65520.0, 1e9]])
    for x in xs:
        want = np.array([x]).astype(np.float16).view(np.uint16)[0]
        got = oracle.f64_to_f16(float(x))
        assert got == want, (x, hex(got), hex(want))


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.int32).astype(np.int16)
    ref = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(b) & 0xFFFF) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("name,fmt", [("iq2x_A", "iq2x"), ("q2k_B", "q2k"), ("q4k_C", "q4k")])
def test_golden_blocks(golden_blocks, name, fmt):
    sec = golden_blocks[name]
    blk = np.array(sec["bytes"], dtype=np.uint8)
    assert blk.size == oracle.BLOCK_BYTES[FMT[fmt]]
    assert len(sec["expect"]) == 256
    cb = None
    if fmt == "iq2x":
        cb = np.ones((256, 8), dtype=np.uint8)
        for r, row in sec["codebook"].items():
            cb[r] = row
    got = oracle.dequantize(FMT[fmt], blk, cb)
    assert np.array_equal(got, np.array(sec["expect"])), np.nonzero(got != np.array(sec["expect"]))


@pytest.mark.parametrize("fmt", [oracle.FMT_IQ2X, oracle.FMT_Q2K, oracle.FMT_Q4K])
def test_dequant_values_exact_in_fp32(fmt):
    """Every decoded weight is a product of small integers and fp16 scales (plus
    one subtraction for q2k/q4k): it must be exactly representable in fp32, so the
    value does not depend on how a kernel orders or fuses that arithmetic."""
    blocks = synth.random_blocks(fmt, 4096, 7, 99)
    w = oracle.dequantize(fmt, blocks, synth.codebook())
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


def test_iq2x_even_negatives_and_scale_identity():
    """Each 8-group decodes with an even number of negative weights, and |w|/d is
    an integer between 1 and 93."""
    cb = synth.codebook()
    blocks = synth.random_blocks(oracle.FMT_IQ2X, 512, 3, 5)
    w = oracle.dequantize(oracle.FMT_IQ2X, blocks, cb).reshape(-1, 32, 8)
    assert np.all((w < 0).sum(-1) % 2 == 0)
    blk = blocks.reshape(-1, 66)
    d = blk[:, :2].copy().view(np.float16).astype(np.float64).reshape(-1)
    q = np.abs(w.reshape(512, 256)) / d[:, None]
    assert np.array_equal(q, np.rint(q))
    assert q.min() >= 1 and q.max() <= 93          # (2s+1) * C with s < 16, C in {1,2,3}


def test_codebook_alphabet():
    cb = synth.codebook()
    assert cb.shape == (256, 8) and set(np.unique(cb)) <= {1, 2, 3}
    assert np.array_equal(cb, synth.codebook())   # seeded, reproducible
