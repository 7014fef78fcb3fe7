"""Pins for the oracle's router, permutation, expert FFN and combine (CPU only).

Routing is pinned by exact (correctly rounded) sums, a library sort of the
logits, closed forms for the degenerate cases and library softmax; the
permutation by numpy's stable argsort; the FFN by a textbook dense SwiGLU with
numpy matmuls on the dequantized weights (brute force on small layers); the
combine by linearity and a numpy contraction; the whole layer by per-token
independence (chunking, permutation and duplication of tokens).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16_to_f64(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def _as_f64(a):
    return _bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.fixture(scope="module")
def tiny():
    return synth.make_layer("tiny", quantizer=oracle.quantize)


@pytest.fixture(scope="module")
def small():
    return synth.make_layer("small", quantizer=oracle.quantize)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [False, True])
def test_router_logits_are_correctly_rounded_sums(bf16):
    """The binary64 fixed-order sum of exact products, rounded once to fp32, equals
    the exactly computed (rational) dot product rounded to fp32."""
    H, E, T = 512, 16, 6
    x = synth.normal_f32(1, 1, (T, H), 1.0)
    w = synth.normal_f32(1, 2, (E, H), 0.02)
    if bf16:
        x, w = synth.to_bf16_bits(x), synth.to_bf16_bits(w)
    logits, _, _ = oracle.route(x, w, 4)
    xf, wf = _as_f64(x), _as_f64(w)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wf[e], xf[t]))
            assert np.float32(float(exact)) == logits[t, e] or \
                np.float32(math.fsum(float(a) * float(b) for a, b in zip(wf[e], xf[t]))) == logits[t, e]


def test_topk_matches_library_sort(small):
    x = synth.activations("small", 37, 512, True)
    logits, idx, w = oracle.route(x, small.w_router, 4)
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(16), -logits[t].astype(np.float64)))   # by (-logit, index)
        assert np.array_equal(idx[t], order[:4])
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_topk_weights_are_library_softmax(small):
    x = synth.activations("small", 37, 512, True)
    logits, idx, w = oracle.route(x, small.w_router, 4)
    sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
    want = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    assert np.allclose(w, want, rtol=1e-14, atol=0)


def test_full_softmax_when_k_equals_E(small):
    x = synth.activations("small", 5, 512, True)
    logits, idx, w = oracle.route(x, small.w_router, 16)
    full = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    assert np.allclose(np.take_along_axis(full, idx, 1), w, rtol=1e-14, atol=0)


def test_zero_input_ties_go_to_lower_index(small):
    x = np.zeros((3, 512), np.uint16)
    _, idx, w = oracle.route(x, small.w_router, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    assert np.array_equal(w, np.full((3, 4), 0.25))


def test_power_of_two_input_scaling_keeps_selection(small):
    x = synth.activations("small", 20, 512, True)
    x4 = synth.to_bf16_bits(synth.bf16_bits_to_f32(x) * 4.0)        # exact
    _, i1, _ = oracle.route(x, small.w_router, 4)
    _, i2, _ = oracle.route(x4, small.w_router, 4)
    assert np.array_equal(i1, i2)


def test_bias_enters_logits():
    spec = synth.SPECS["mid"]
    L = synth.make_layer(spec, quantizer=oracle.quantize)
    x = synth.activations("mid", 8, spec.hidden, True)
    l0, _, _ = oracle.route(x, L.w_router, 8)
    lb, idx, _ = oracle.route(x, L.w_router, 8, L.bias)
    assert np.array_equal(lb, (l0.astype(np.float64) + L.bias.astype(np.float64)).astype(np.float32))
    for t in range(8):
        assert np.array_equal(idx[t], np.lexsort((np.arange(32), -lb[t].astype(np.float64)))[:8])


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (3, 8, 256), (37, 4, 16), (512, 8, 256), (5, 2, 8)])
def test_permutation_is_stable_argsort(T, k, E):
    g = np.random.default_rng(T)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, perm, active = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(cnt)]))
    nz = np.nonzero(cnt)[0]
    assert active[0] == nz.size and np.array_equal(active[1:1 + nz.size], nz)


# ----------------------------------------------------------------------------
# FFN and combine
# ----------------------------------------------------------------------------
def _silu(g):
    return g / (1.0 + np.exp(-g))


def _dense(layer, fmt, blocks, E, rows, cols):
    return oracle.dequantize(fmt, blocks, layer.codebook).reshape(E, rows, cols)


def test_expert_ffn_equals_dense_swiglu(tiny):
    """Every slot's output is the textbook SwiGLU FFN of its expert, evaluated with
    numpy matmuls on the dequantized matrices (gate/up [I][H], down [H][I])."""
    sp = tiny.spec
    x = synth.activations("tiny", 4, sp.hidden, False)
    _, idx, _ = oracle.route(x, tiny.w_router, sp.top_k)
    out = oracle.expert_ffn(x, idx, sp.gate_up_fmt, tiny.gate, tiny.up, sp.down_fmt, tiny.down, tiny.codebook,
                            sp.n_experts, sp.inter)
    G = _dense(tiny, sp.gate_up_fmt, tiny.gate, sp.n_experts, sp.inter, sp.hidden)
    U = _dense(tiny, sp.gate_up_fmt, tiny.up, sp.n_experts, sp.inter, sp.hidden)
    D = _dense(tiny, sp.down_fmt, tiny.down, sp.n_experts, sp.hidden, sp.inter)
    xf = x.astype(np.float64)
    for s in range(idx.size):
        t, e = s // sp.top_k, idx.reshape(-1)[s]
        h = _silu(G[e] @ xf[t]) * (U[e] @ xf[t])
        want = D[e] @ h
        assert np.allclose(out[s], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_top1_single_expert_layer_is_dense_ffn(small):
    """With one expert and top-1 the routing weight is exactly 1 and the layer is
    that expert's dense FFN (plus the shared expert, dense too)."""
    sp = small.spec
    H, I = sp.hidden, sp.inter
    per_gu = I * H // 256 * 66
    per_d = H * I // 256 * 84
    gate, up, down = small.gate[:per_gu], small.up[:per_gu], small.down[:per_d]
    wr = small.w_router[:1]
    x = synth.activations("small", 9, H, True)
    res = oracle.layer(x, wr, 1, 1, I, sp.gate_up_fmt, gate, up, sp.down_fmt, down, small.codebook,
                       shared=small.shared)
    assert np.array_equal(res["topk_idx"], np.zeros((9, 1), np.int32)) and np.array_equal(res["topk_w"], np.ones((9, 1)))
    G = oracle.dequantize(sp.gate_up_fmt, gate, small.codebook).reshape(I, H)
    U = oracle.dequantize(sp.gate_up_fmt, up, small.codebook).reshape(I, H)
    D = oracle.dequantize(sp.down_fmt, down).reshape(H, I)
    Sg, Su, Sd = (_bf16_to_f64(a) for a in small.shared)
    xf = _bf16_to_f64(x)
    want = (D @ (_silu(G @ xf.T) * (U @ xf.T))).T + (Sd @ (_silu(Sg @ xf.T) * (Su @ xf.T))).T
    assert np.allclose(res["y"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_combine_is_weighted_sum():
    g = np.random.default_rng(3)
    T, k, H = 5, 3, 64
    o = g.standard_normal((T * k, H))
    w = g.random((T, k))
    s = g.standard_normal((T, H))
    y = oracle.combine(o, w, s)
    want = np.einsum("tk,tkh->th", w, o.reshape(T, k, H)) + s
    assert np.allclose(y, want, rtol=1e-14, atol=1e-14)
    # linear in the slot outputs, shared output optional
    y2 = oracle.combine(2 * o, w, None)
    assert np.allclose(y2, 2 * (want - s), rtol=1e-14, atol=1e-13)


# directional steering of the FFN output: y' = y - F v (v . y)

def test_steer_zero_strength_and_basis_direction():
    g = np.random.default_rng(11)
    T, H = 4, 48
    y = g.standard_normal((T, H))
    v = g.standard_normal(H)
    assert np.array_equal(oracle.steer(y, v, 0.0), y)
    # along a basis vector the map scales that one column by (1 - F), exactly
    for i, F in ((0, 1.0), (17, 0.5), (47, 2.0)):
        e = np.zeros(H)
        e[i] = 1.0
        out = oracle.steer(y, e, F)
        want = y.copy()
        want[:, i] = (1.0 - F) * y[:, i]
        assert np.array_equal(out, want)


def test_steer_unit_direction_projects_and_reflects():
    g = np.random.default_rng(12)
    T, H = 6, 4096
    y = g.standard_normal((T, H))
    v = g.standard_normal(H)
    v /= np.linalg.norm(v)
    p = oracle.steer(y, v, 1.0)
    # F = 1 removes the component along v: orthogonal to v, and a projection (idempotent)
    assert np.abs(p @ v).max() <= 1e-12 * np.abs(y).sum(axis=1).max()
    assert np.allclose(oracle.steer(p, v, 1.0), p, rtol=0, atol=1e-13)
    assert np.allclose(y - p, np.outer(y @ v, v), rtol=0, atol=1e-12)
    # F = 2 is the Householder reflection: norm-preserving and its own inverse
    r = oracle.steer(y, v, 2.0)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(y, axis=1), rtol=1e-13)
    assert np.allclose(oracle.steer(r, v, 2.0), y, rtol=0, atol=1e-12)
    assert np.allclose(r @ v, -(y @ v), rtol=1e-12, atol=1e-12)


def test_steer_is_per_token_linear_and_unnormalised():
    g = np.random.default_rng(13)
    T, H = 5, 96
    y1, y2 = g.standard_normal((T, H)), g.standard_normal((T, H))
    v = g.standard_normal(H)
    F = 0.75
    out = oracle.steer(y1, v, F)
    # rows are independent: reversing the tokens reverses the output rows bit for bit
    assert np.array_equal(oracle.steer(y1[::-1], v, F), out[::-1])
    # linear in y
    assert np.allclose(oracle.steer(2 * y1 - 3 * y2, v, F), 2 * out - 3 * oracle.steer(y2, v, F), rtol=0, atol=1e-12)
    # v is used as given: scaling it by c scales the strength by c^2
    assert np.allclose(oracle.steer(y1, 3.0 * v, F), oracle.steer(y1, v, 9.0 * F), rtol=0, atol=1e-11)


def test_layer_is_per_token(small):
    """Splitting the tokens into chunks, reordering them or duplicating one leaves
    every token's output bit-identical (the layer has no cross-token arithmetic)."""
    sp = small.spec
    x = synth.activations("small", 12, sp.hidden, True)
    args = (sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, small.gate, small.up, sp.down_fmt, small.down,
            small.codebook)
    full = oracle.layer(x, small.w_router, *args, shared=small.shared)["y"]
    parts = [oracle.layer(x[a:b], small.w_router, *args, shared=small.shared)["y"] for a, b in ((0, 5), (5, 6), (6, 12))]
    assert np.array_equal(np.concatenate(parts), full)
    p = np.random.default_rng(0).permutation(12)
    assert np.array_equal(oracle.layer(x[p], small.w_router, *args, shared=small.shared)["y"], full[p])
    xd = np.concatenate([x, x[3:4]])
    yd = oracle.layer(xd, small.w_router, *args, shared=small.shared)["y"]
    assert np.array_equal(yd[12], yd[3])


def test_shared_expert_is_dense_bf16_ffn(small):
    x = synth.activations("small", 4, small.spec.hidden, True)
    s = oracle.shared_ffn(x, *small.shared)
    Sg, Su, Sd = (_bf16_to_f64(a) for a in small.shared)
    xf = _bf16_to_f64(x)
    want = (Sd @ (_silu(Sg @ xf.T) * (Su @ xf.T))).T
    assert np.allclose(s, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def _router_order_cases():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "router_order.txt")
    cases = []
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line.startswith("case"):
            continue
        head, want = line.split("->")
        toks = head.split()
        name, H = toks[1], int(toks[2].rstrip(":"))
        entries = [(int(a), float(b)) for a, b in (t.split(":") for t in toks[3:])]
        cases.append((name, H, entries, float(want)))
    return cases


@pytest.mark.parametrize("case", _router_order_cases(), ids=lambda c: c[0])
def test_router_fixed_summation_order(case):
    """Hand-worked cancellation cases (tests/golden/router_order.txt) where the order
    of the binary64 additions decides the fp32 logit."""
    name, H, entries, want = case
    x = np.ones((1, H), np.float32)
    w = np.zeros((2, H), np.float32)
    for h, v in entries:
        w[0, h] = v
    logits, _, _ = oracle.route(x, w, 1)
    assert logits[0, 0] == np.float32(want), (name, logits[0, 0])
