"""Seeded synthetic inputs for the routed 2-bit MoE FFN layer.

This module is the only code shared by the GPU library's tests/benchmark and
the CPU oracle.  It draws random numbers and lays them out as inputs; it holds
none of the layer's arithmetic (no dequantization, quantization, routing or
FFN).  Where a test wants expert weights that were really quantized from
N(0, 0.02) masters it passes a quantizer in (``make_layer(quantizer=...)``).

Workloads (layer shapes; all inputs seeded):
  tiny      hidden 256, 8 routed experts, top-2, intermediate 128, 4 tokens,
            fp32 activations N(0,1), fp32 router N(0,0.02), experts N(0,0.02)
            quantized (gate/up iq2x, down q2k), no shared expert, seed 0.
  decode    hidden 4096, 256 experts, top-8, intermediate 2048, one bf16
            shared expert (intermediate 2048), bf16 activations N(0,1), bf16
            router N(0,0.02); 1000 tokens, one per call.
  verify    the decode layer, 3 tokens per step (1 accepted + 2 drafts).
  prefill   the decode layer, 512 tokens, router bias N(0,0.5) per expert.
  long      the decode layer, 11,709 tokens in 2048-token chunks, routed
            experts in 2-bit form and in a q4k (4.5 bpw) form.
  steering  one unit-length fp32 direction per layer (normalised N(0,1)
            draws), strength 1.

Full-size routed experts (1.8 GB of blocks per layer) are drawn field by field
("random blocks"): every bit pattern of the formats decodes to a valid block,
so scales are drawn from distributions measured once on N(0,0.02) weights
quantized by the oracle's quantizers (block scale, group/sub-block scales and
mins), codes and signs are uniform random bits, and the iq2x block scale is
set so that the decoded weights have mean ~0 and RMS ~0.02-0.026 like
N(0,0.02) weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import os

import numpy as np

FMT_IQ2X, FMT_Q2K, FMT_Q4K, FMT_BF16 = 1, 2, 3, 4
BLOCK_BYTES = {FMT_IQ2X: 66, FMT_Q2K: 84, FMT_Q4K: 144}
QK = 256

# tensor ids for per-tensor random streams
_T_X, _T_ROUTER, _T_BIAS, _T_SG, _T_SU, _T_SD, _T_G, _T_U, _T_D, _T_CB, _T_STEER = range(1, 12)


def rng(seed: int, tensor: int, part: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tensor), int(part)])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (the input's storage type)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, tensor: int, shape, std: float, part: int = 0) -> np.ndarray:
    return (rng(seed, tensor, part).standard_normal(size=shape, dtype=np.float64) * std).astype(np.float32)


def codebook(seed: int = 0) -> np.ndarray:
    """The seeded 256 x 8 codebook of iq2x magnitudes, entries in {1, 2, 3}."""
    return rng(seed, _T_CB).integers(1, 4, size=(256, 8), dtype=np.uint8)


# ----------------------------------------------------------------------------
# random blocks (field-level draws)
# ----------------------------------------------------------------------------
def _fp16_bits(v: np.ndarray) -> np.ndarray:
    return v.astype(np.float16).view(np.uint16)


def _clip_round(g: np.random.Generator, n: int, mean: float, std: float, lo: int, hi: int) -> np.ndarray:
    return np.clip(np.rint(g.normal(mean, std, size=n)), lo, hi).astype(np.uint8)


_IQ2X_ROWS = None


def _iq2x_row_table() -> np.ndarray:
    """65536-entry table taking a uniform 16-bit draw to a codebook row, with the row frequencies recorded in
    tests/golden/iq2x_index_freq.txt (those of quantized N(0, 0.02) weights with the seeded codebook)."""
    global _IQ2X_ROWS
    if _IQ2X_ROWS is None:
        path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                            "iq2x_index_freq.txt")
        counts = np.loadtxt(path, dtype=np.int64)
        assert counts.shape == (256,)
        cdf = np.cumsum(counts) / counts.sum()
        u = (np.arange(65536) + 0.5) / 65536.0
        _IQ2X_ROWS = np.minimum(np.searchsorted(cdf, u, side="right"), 255).astype(np.uint8)
    return _IQ2X_ROWS


def random_blocks(fmt: int, nblocks: int, seed: int, tensor: int, part: int = 0) -> np.ndarray:
    """`nblocks` canonical blocks drawn field by field (uint8, nblocks*block_bytes)."""
    g = rng(seed, tensor, part)
    bb = BLOCK_BYTES[fmt]
    out = np.frombuffer(bytearray(g.bytes(nblocks * bb)), dtype=np.uint8).reshape(nblocks, bb)
    if fmt == FMT_IQ2X:
        d = np.clip(g.normal(6.56e-4, 7.9e-5, size=nblocks), 4.7e-4, 1.02e-3)
        out[:, 0:2] = _fp16_bits(d).view(np.uint8).reshape(nblocks, 2)
        # codebook rows with the quantizer's frequencies (bytes 0..3 of each 8-byte group record)
        rows = _iq2x_row_table()[g.integers(0, 65536, size=(nblocks, 8, 4), dtype=np.uint16)]
        out[:, 2:].reshape(nblocks, 8, 8)[:, :, 0:4] = rows
        s = _clip_round(g, nblocks * 8, 11.5, 2.3, 0, 15).reshape(nblocks, 8)
        aux_hi = out[:, 2:].reshape(nblocks, 8, 8)[:, :, 7]          # byte holding bits 24..31 of aux
        out[:, 2:].reshape(nblocks, 8, 8)[:, :, 7] = (aux_hi & 0x0F) | (s << 4)
    elif fmt == FMT_Q2K:
        d = np.clip(g.normal(2.21e-3, 2.2e-4, size=nblocks), 1.2e-3, 3.5e-3)
        dm = np.clip(g.normal(3.76e-3, 5.1e-4, size=nblocks), 1.5e-3, 6.5e-3)
        out[:, 0:2] = _fp16_bits(d).view(np.uint8).reshape(nblocks, 2)
        out[:, 2:4] = _fp16_bits(dm).view(np.uint8).reshape(nblocks, 2)
        sc = _clip_round(g, nblocks * 16, 10.5, 2.4, 0, 15)
        m = _clip_round(g, nblocks * 16, 9.5, 2.8, 0, 15)
        out[:, 4:20] = (sc | (m << 4)).reshape(nblocks, 16)
        # 2-bit codes: the uniform random bytes already drawn
    elif fmt == FMT_Q4K:
        d = np.clip(g.normal(1.094e-4, 1.08e-5, size=nblocks), 6e-5, 1.8e-4)
        dm = np.clip(g.normal(8.95e-4, 1.22e-4, size=nblocks), 4e-4, 1.5e-3)
        out[:, 0:2] = _fp16_bits(d).view(np.uint8).reshape(nblocks, 2)
        out[:, 2:4] = _fp16_bits(dm).view(np.uint8).reshape(nblocks, 2)
        sc = _clip_round(g, nblocks * 8, 50.0, 9.0, 0, 63).reshape(nblocks, 8)
        m = _clip_round(g, nblocks * 8, 44.0, 11.0, 0, 63).reshape(nblocks, 8)
        fields = np.concatenate([sc, m], axis=1).astype(np.uint64)          # 16 six-bit fields
        bits = np.zeros(nblocks, dtype=np.uint64)
        hi = np.zeros(nblocks, dtype=np.uint64)
        for f in range(16):                                                 # 96-bit little-endian string
            pos = 6 * f
            if pos + 6 <= 64:
                bits |= fields[:, f] << np.uint64(pos)
            elif pos >= 64:
                hi |= fields[:, f] << np.uint64(pos - 64)
            else:                                                           # straddles bit 64
                bits |= (fields[:, f] << np.uint64(pos)) & np.uint64(0xFFFFFFFFFFFFFFFF)
                hi |= fields[:, f] >> np.uint64(64 - pos)
        out[:, 4:12] = bits.view(np.uint8).reshape(nblocks, 8)
        out[:, 12:16] = hi.astype(np.uint32).view(np.uint8).reshape(nblocks, 4)
        # 4-bit codes: the uniform random bytes already drawn
    else:
        raise ValueError(fmt)
    return out.reshape(-1)


# ----------------------------------------------------------------------------
# layers
# ----------------------------------------------------------------------------
@dataclass
class LayerSpec:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    shared_inter: int          # 0 = no shared expert
    x_bf16: bool               # activations (and router weight) in bf16, else fp32
    layer_seed: int
    gate_up_fmt: int = FMT_IQ2X
    down_fmt: int = FMT_Q2K
    bias_std: float = 0.0      # router bias N(0, bias_std) per expert, 0 = none


@dataclass
class Layer:
    spec: LayerSpec
    w_router: np.ndarray                       # [E][H] bf16 bits (uint16) or fp32
    bias: Optional[np.ndarray]                 # [E] fp32 or None
    codebook: np.ndarray                       # [256][8] uint8
    gate: np.ndarray                           # canonical blocks, experts stacked, [E][I][H]
    up: np.ndarray
    down: np.ndarray                           # [E][H][I]
    shared: Optional[tuple] = None             # (Wg [Is][H], Wu [Is][H], Wd [H][Is]) bf16 bits
    masters: dict = field(default_factory=dict)


SPECS = {
    "tiny": LayerSpec("tiny", 256, 128, 8, 2, 0, False, 0),
    "decode": LayerSpec("decode", 4096, 2048, 256, 8, 2048, True, 1),
    "verify": LayerSpec("verify", 4096, 2048, 256, 8, 2048, True, 1),
    "prefill": LayerSpec("prefill", 4096, 2048, 256, 8, 2048, True, 1, bias_std=0.5),
    "long": LayerSpec("long", 4096, 2048, 256, 8, 2048, True, 1),
    "long_q4k": LayerSpec("long_q4k", 4096, 2048, 256, 8, 2048, True, 1, FMT_Q4K, FMT_Q4K),
    # reduced layers that the oracle finishes in seconds; several tiles and a ragged tail
    "small": LayerSpec("small", 512, 256, 16, 4, 256, True, 101),
    "small_q4k": LayerSpec("small_q4k", 512, 256, 16, 4, 256, True, 101, FMT_Q4K, FMT_Q4K),
    "small_mix_a": LayerSpec("small_mix_a", 512, 256, 16, 4, 256, True, 101, FMT_IQ2X, FMT_Q4K),
    "small_mix_b": LayerSpec("small_mix_b", 512, 256, 16, 4, 256, True, 101, FMT_Q4K, FMT_Q2K),
    "mid": LayerSpec("mid", 1024, 512, 32, 8, 512, True, 102, bias_std=0.5),
    "mid_fp32": LayerSpec("mid_fp32", 1024, 512, 32, 8, 0, False, 103),
    # top-16 routing: the one-ballot slot lookup of the decode kernels covers T*k <= 64 slots
    "mid_k16": LayerSpec("mid_k16", 1024, 512, 32, 16, 512, True, 104),
}

# activation seeds per workload
X_SEEDS = {"tiny": 0, "decode": 11, "verify": 12, "prefill": 13, "long": 14, "long_q4k": 14,
           "small": 201, "small_q4k": 201, "small_mix_a": 201, "small_mix_b": 201, "mid": 202, "mid_fp32": 203,
           "mid_k16": 204}
BIAS_SEEDS = {"prefill": 23, "mid": 24}
TOKENS = {"tiny": 4, "decode": 1000, "verify": 3 * 334, "prefill": 512, "long": 11709, "long_q4k": 11709}


def activations(name: str, n_tokens: int, hidden: int, bf16: bool, seed: Optional[int] = None) -> np.ndarray:
    """x [T][H] ~ N(0,1): fp32, or bf16 bit patterns (uint16)."""
    s = X_SEEDS[name] if seed is None else seed
    x = normal_f32(s, _T_X, (n_tokens, hidden), 1.0)
    return to_bf16_bits(x) if bf16 else x


def steer_direction(hidden: int, seed: int = 0) -> np.ndarray:
    """A unit-length fp32 direction [hidden] for directional steering (N(0,1) draws, normalised)."""
    v = rng(seed, _T_STEER).standard_normal(size=hidden, dtype=np.float64)
    return (v / np.linalg.norm(v)).astype(np.float32)


def make_router(spec: LayerSpec | str):
    """(w_router, bias) of a layer without its experts (same draws as make_layer)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    s = spec.layer_seed
    wr = normal_f32(s, _T_ROUTER, (spec.n_experts, spec.hidden), 0.02)
    wr = to_bf16_bits(wr) if spec.x_bf16 else wr
    bias = None
    if spec.bias_std > 0:
        bias = normal_f32(BIAS_SEEDS.get(spec.name, s + 7), _T_BIAS, (spec.n_experts,), spec.bias_std)
    return wr, bias


def make_layer(spec: LayerSpec | str, quantizer: Optional[Callable] = None, keep_masters: bool = False) -> Layer:
    """Build a seeded layer.

    quantizer(fmt, w_f32_flat, codebook) -> canonical blocks.  When given, routed
    experts are N(0,0.02) fp32 masters encoded by it; otherwise random blocks.
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    H, I, E = spec.hidden, spec.inter, spec.n_experts
    s = spec.layer_seed
    cb = codebook(0)
    wr, bias = make_router(spec)
    masters = {}
    if quantizer is not None:
        blocks = {}
        for name, tid, fmt, shape in (("gate", _T_G, spec.gate_up_fmt, (E, I, H)), ("up", _T_U, spec.gate_up_fmt, (E, I, H)),
                                      ("down", _T_D, spec.down_fmt, (E, H, I))):
            w = normal_f32(s, tid, shape, 0.02)
            blocks[name] = quantizer(fmt, w.reshape(-1), cb)
            if keep_masters:
                masters[name] = w
        gate, up, down = blocks["gate"], blocks["up"], blocks["down"]
    else:
        ngu = E * I * H // QK
        gate = random_blocks(spec.gate_up_fmt, ngu, s, _T_G)
        up = random_blocks(spec.gate_up_fmt, ngu, s, _T_U)
        down = random_blocks(spec.down_fmt, ngu, s, _T_D)
    shared = None
    if spec.shared_inter:
        Is = spec.shared_inter
        shared = (to_bf16_bits(normal_f32(s, _T_SG, (Is, H), 0.02)),
                  to_bf16_bits(normal_f32(s, _T_SU, (Is, H), 0.02)),
                  to_bf16_bits(normal_f32(s, _T_SD, (H, Is), 0.02)))
    return Layer(spec, wr, bias, cb, gate, up, down, shared, masters)
