"""Pins for the oracle's reference encoders (CPU only).

Encoders are offline tools (not on the layer's hot path); they give the test
layers their N(0,0.02)-quantized weights.  Pins: a closed-form error bound for
q2k/q4k, brute-force nearest-codebook search for iq2x, the parity invariant,
exact round trips of representable blocks, sign and power-of-two symmetries.
"""
import numpy as np
import pytest

import oracle
import synth


def _w(n_blocks, seed, std=0.02):
    return synth.normal_f32(seed, 77, (n_blocks * 256,), std)


def _fields_kq(blocks, fmt):
    """Read d, dmin, sc, m back from canonical bytes (test-side reader)."""
    if fmt == oracle.FMT_Q2K:
        b = blocks.reshape(-1, 84)
        sc = (b[:, 4:20] & 15).astype(np.float64)
        m = (b[:, 4:20] >> 4).astype(np.float64)
    else:
        b = blocks.reshape(-1, 144)
        bits = np.unpackbits(b[:, 4:16], bitorder="little").reshape(-1, 16, 6)
        v = (bits * (1 << np.arange(6))).sum(-1).astype(np.float64)
        sc, m = v[:, :8], v[:, 8:]
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64)
    dmin = b[:, 2:4].copy().view(np.float16).astype(np.float64)
    return d, dmin, sc, m


@pytest.mark.parametrize("fmt,nsub,L", [(oracle.FMT_Q2K, 16, 1.5), (oracle.FMT_Q4K, 8, 7.5)])
def test_kquant_roundtrip_bound(fmt, nsub, L):
    """|w - w^| <= max(d*sc/2, L*d + dmin/2) + 2^-9 (hi - lo) per sub-block:
    half a grid step inside the range, plus the end mismatch from rounding the
    step and offset to integer multiples of d and dmin (fp16 rounding of d and
    dmin is covered by the last term)."""
    w = _w(2000, 1).astype(np.float64)
    blocks = oracle.quantize(fmt, w.astype(np.float32))
    wh = oracle.dequantize(fmt, blocks)
    d, dmin, sc, m = _fields_kq(blocks, fmt)
    ws = w.reshape(-1, nsub, 256 // nsub)
    err = np.abs(ws - wh.reshape(ws.shape)).max(-1)
    lo = np.minimum(0, ws.min(-1))
    hi = np.maximum(0, ws.max(-1))
    bound = np.maximum(d * sc / 2, L * d + dmin / 2) + 2.0 ** -9 * (hi - lo)
    assert np.all(err <= bound), float((err / bound).max())
    # relative error is what a 2/4-bit grid gives
    rel = np.linalg.norm(w - wh) / np.linalg.norm(w)
    assert rel < (0.40 if fmt == oracle.FMT_Q2K else 0.10)


def test_iq2x_index_is_bruteforce_argmin():
    """Each stored index is the lowest codebook row minimising the squared error
    of the magnitudes at the group's scale S = d (2s+1), found by brute force."""
    cb = synth.codebook()
    w = _w(64, 2).astype(np.float64)
    blocks = oracle.quantize(oracle.FMT_IQ2X, w.astype(np.float32), cb)
    b = blocks.reshape(-1, 66)
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64)[:, 0]
    rec = b[:, 2:].reshape(-1, 8, 8)
    aux = rec[:, :, 4:].copy().view(np.uint32)[..., 0]
    s = (aux >> 28).astype(np.float64)
    S = d[:, None] * (2 * s + 1)                                  # [blocks][groups]
    mag = np.abs(w.reshape(-1, 8, 4, 8))                          # [blocks][group][sub][8]
    err = ((mag[..., None, :] - S[:, :, None, None, None] * cb[None, None, None].astype(np.float64)) ** 2).sum(-1)
    want = err.argmin(-1)                                         # numpy argmin takes the first (lowest) index
    assert np.array_equal(rec[:, :, :4], want.astype(np.uint8))


def test_iq2x_scale_rule():
    """The block scale d is the fp16 value nearest max|w| / 93 (no neighbouring fp16 value is closer), and each
    group's scale s is, by search over all sixteen values, the one whose largest magnitude 3(2s+1)d lies closest to
    the group's largest |w|."""
    cb = synth.codebook()
    w = _w(64, 3).astype(np.float64)
    b = oracle.quantize(oracle.FMT_IQ2X, w.astype(np.float32), cb).reshape(-1, 66)
    d16 = b[:, 0:2].copy().view(np.float16)[:, 0]
    d = d16.astype(np.float64)
    target = np.abs(w.reshape(-1, 256)).max(-1) / 93
    for di, ti in zip(d16, target):
        up, down = np.nextafter(di, np.float16(np.inf)), np.nextafter(di, np.float16(0))
        assert abs(float(di) - ti) <= abs(float(up) - ti) and abs(float(di) - ti) <= abs(float(down) - ti)
    aux = b[:, 2:].reshape(-1, 8, 8)[:, :, 4:].copy().view(np.uint32)[..., 0]
    G = np.abs(w.reshape(-1, 8, 32)).max(-1)
    cand = 3.0 * (2 * np.arange(16) + 1)[None, None, :] * d[:, None, None]   # [block][group][s]
    want_s = np.abs(cand - G[..., None]).argmin(-1)
    assert np.array_equal((aux >> 28).astype(np.int64), want_s)


def test_iq2x_parity_and_sign_choice():
    """Decoded signs agree with the input's except for at most one weight per
    8-group, and the number of negatives is even."""
    cb = synth.codebook()
    w = _w(256, 4)
    wh = oracle.dequantize(oracle.FMT_IQ2X, oracle.quantize(oracle.FMT_IQ2X, w, cb), cb)
    sw = (w < 0).reshape(-1, 8)
    sh = (wh < 0).reshape(-1, 8)
    assert np.all(sh.sum(-1) % 2 == 0)
    flips = (sw != sh).sum(-1)
    assert np.all(flips == (sw.sum(-1) % 2))


def test_iq2x_representable_block_roundtrips():
    """A block whose groups each contain a codebook magnitude 3 decodes to weights
    that the encoder maps back to the same weights."""
    cb = synth.codebook()
    g = np.random.default_rng(5)
    blocks = synth.random_blocks(oracle.FMT_IQ2X, 200, 9, 9).reshape(-1, 66).copy()
    rows3 = np.nonzero((cb == 3).any(1))[0]
    rec = blocks[:, 2:].reshape(-1, 8, 8)
    rec[:, :, 0] = g.choice(rows3, size=rec.shape[:2])          # sub-group 0 of every group uses a row with a 3
    blocks[:, 2:] = rec.reshape(-1, 64)
    blocks[:, 0:2] = np.array([0.01], np.float16).view(np.uint8)  # d exact, far from fp16 limits
    aux = rec[:, :, 4:].copy().view(np.uint32)[..., 0]
    s = g.integers(0, 15, size=aux.shape).astype(np.uint32)
    s[:, 0] = 15                                                  # group 0 sets the block scale
    aux = (aux & np.uint32(0x0FFFFFFF)) | (s << np.uint32(28))
    rec[:, :, 4:] = aux.view(np.uint8).reshape(rec.shape[0], 8, 4)
    blocks[:, 2:] = rec.reshape(-1, 64)
    w = oracle.dequantize(oracle.FMT_IQ2X, blocks.reshape(-1), cb)
    w2 = oracle.dequantize(oracle.FMT_IQ2X, oracle.quantize(oracle.FMT_IQ2X, w.astype(np.float32), cb), cb)
    assert np.array_equal(w, w2)


def test_iq2x_negation_symmetry():
    cb = synth.codebook()
    w = _w(128, 6)
    w[w == 0] = 1e-3
    a = oracle.dequantize(oracle.FMT_IQ2X, oracle.quantize(oracle.FMT_IQ2X, w, cb), cb)
    b = oracle.dequantize(oracle.FMT_IQ2X, oracle.quantize(oracle.FMT_IQ2X, -w, cb), cb)
    assert np.array_equal(a, -b)


@pytest.mark.parametrize("fmt", [oracle.FMT_IQ2X, oracle.FMT_Q2K, oracle.FMT_Q4K])
@pytest.mark.parametrize("k", [-2, 3])
def test_power_of_two_scaling(fmt, k):
    """quant(2^k w) is quant(w) with d and dmin multiplied by 2^k while d and dmin
    stay in fp16's normal range (weights N(0, 0.2) so that q4k's d stays normal)."""
    cb = synth.codebook()
    w = _w(128, 7, std=0.2)
    a = oracle.dequantize(fmt, oracle.quantize(fmt, w, cb), cb)
    b = oracle.dequantize(fmt, oracle.quantize(fmt, (w * 2.0 ** k).astype(np.float32), cb), cb)
    assert np.array_equal(a * 2.0 ** k, b)


@pytest.mark.parametrize("fmt", [oracle.FMT_IQ2X, oracle.FMT_Q2K, oracle.FMT_Q4K])
def test_zero_block(fmt):
    w = np.zeros(512, np.float32)
    assert np.array_equal(oracle.dequantize(fmt, oracle.quantize(fmt, w, synth.codebook()), synth.codebook()), np.zeros(512))
