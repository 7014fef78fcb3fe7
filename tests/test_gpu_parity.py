"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: dequantized weights, logits, routing indices, offsets, permutation and
active lists bit-exact; routing weights within 1e-6; slot, shared and layer
outputs within a per-token relative L2 error of 1e-3 (the layer's stated
tolerance with fp32 accumulation).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


def note(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import bit_quantized_moe_permute_amd as m
    return m


def dev_x(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def rel_l2_rows(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    got = got.reshape(want.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1)
    den = np.linalg.norm(want, axis=1)
    return np.linalg.norm(got - want, axis=1) / np.where(den > 0, den, 1.0)


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [oracle.FMT_IQ2X, oracle.FMT_Q2K, oracle.FMT_Q4K])
@pytest.mark.parametrize("kind", ["quantized", "random"])
def test_dequant_bit_exact(m, fmt, kind):
    note(f"dequant fmt={fmt} kind={kind}")
    cb = synth.codebook()
    if kind == "quantized":
        w = synth.normal_f32(3, 50, (6, 96, 256), 0.02)         # 6 matrices [96][256]
        blocks = oracle.quantize(fmt, w.reshape(-1), cb)
    else:
        blocks = synth.random_blocks(fmt, 6 * 96, 4, 51)
    n_mats, rows, cols = 6, 96, 256
    canon = torch.from_numpy(blocks).cuda()
    prep = torch.empty_like(canon)
    m.moe_prepare_weights(fmt, n_mats, rows, cols, canon, prep)
    dcb = torch.from_numpy(cb.reshape(-1)).cuda()
    want = oracle.dequantize(fmt, blocks, cb).reshape(n_mats, rows, cols)
    out = torch.empty(n_mats, rows, cols, dtype=torch.float32, device="cuda")
    m.moe_dequantize(fmt, prep, n_mats, rows, cols, 0, n_mats, dcb, out)
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    # a sub-range of matrices
    out2 = torch.empty(2, rows, cols, dtype=torch.float32, device="cuda")
    m.moe_dequantize(fmt, prep, n_mats, rows, cols, 3, 2, dcb, out2)
    assert np.array_equal(out2.cpu().numpy().astype(np.float64), want[3:5])


def test_dequant_rows_shorter_than_a_block(m):
    """The tiny layer's down matrices are [256][128] q2k: blocks span two rows."""
    note("dequant tiny down")
    L = synth.make_layer("tiny", quantizer=oracle.quantize)
    canon = torch.from_numpy(L.down).cuda()
    prep = torch.empty_like(canon)
    m.moe_prepare_weights(oracle.FMT_Q2K, 8, 256, 128, canon, prep)
    out = torch.empty(8, 256, 128, dtype=torch.float32, device="cuda")
    m.moe_dequantize(oracle.FMT_Q2K, prep, 8, 256, 128, 0, 8, None, out)
    assert np.array_equal(out.cpu().numpy().astype(np.float64).reshape(-1), oracle.dequantize(oracle.FMT_Q2K, L.down))


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def _route_gpu(m, x, w_router, E, k, bias=None):
    T = x.shape[0]
    xd = dev_x(x)
    wd = dev_x(w_router)
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    idx = torch.empty(T, k, **i32)
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, **i32)
    perm = torch.empty(T * k, **i32)
    act = torch.full((E + 1,), -7, **i32)
    ws = torch.empty(max(m.moe_route_workspace(T, E, k), 256), dtype=torch.uint8, device="cuda")
    m.moe_route(xd, wd, E, k, idx, tw, off, perm, act, ws, bias=bd, logits=lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), idx.cpu().numpy(), tw.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy(), act.cpu().numpy()


def _route_gpu_no_logits(m, x, w_router, E, k, bias=None):
    """moe_route without the logits output: above 8 tokens with bf16 inputs this takes the bounded matrix-core
    router (exact binary64 sums only for the experts near each token's selection boundary)."""
    T = x.shape[0]
    i32 = dict(dtype=torch.int32, device="cuda")
    idx = torch.empty(T, k, **i32)
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, **i32)
    perm = torch.empty(T * k, **i32)
    act = torch.full((E + 1,), -7, **i32)
    ws = torch.empty(max(m.moe_route_workspace(T, E, k), 256), dtype=torch.uint8, device="cuda")
    m.moe_route(dev_x(x), dev_x(w_router), E, k, idx, tw, off, perm, act, ws,
                bias=None if bias is None else torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tw.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy(), act.cpu().numpy()


def _check_route(m, x, w_router, E, k, bias=None):
    lg, idx, tw, off, perm, act = _route_gpu(m, x, w_router, E, k, bias)
    ol, oi, ow = oracle.route(x, w_router, k, bias)
    assert np.array_equal(lg.view(np.uint32), ol.view(np.uint32)), np.argwhere(lg != ol)[:5]
    assert np.array_equal(idx, oi)
    assert np.abs(tw.astype(np.float64) - ow).max() <= 1e-6
    oo, op, oa = oracle.permute(oi, E)
    assert np.array_equal(off, oo)
    assert np.array_equal(perm, op)
    assert np.array_equal(act[: oa[0] + 1], oa[: oa[0] + 1])
    # without the logits output: the same bits (indices, weights, offsets, permutation, active list)
    idx2, tw2, off2, perm2, act2 = _route_gpu_no_logits(m, x, w_router, E, k, bias)
    assert np.array_equal(idx2, idx)
    assert np.array_equal(tw2.view(np.uint32), tw.view(np.uint32))
    assert np.array_equal(off2, off)
    assert np.array_equal(perm2, perm)
    assert np.array_equal(act2[: oa[0] + 1], oa[: oa[0] + 1])


ROUTE_CASES = [
    ("tiny", 4), ("small", 1), ("small", 2), ("small", 3), ("small", 8), ("small", 37), ("mid", 6), ("mid", 70), ("decode", 1),
    ("decode", 3), ("decode", 5), ("decode", 8), ("decode", 9), ("decode", 64), ("prefill", 512), ("long", 2048), ("long", 2500),
]


@pytest.mark.parametrize("name,T", ROUTE_CASES, ids=[f"{a}-{b}" for a, b in ROUTE_CASES])
def test_route_matches_oracle(m, name, T):
    note(f"route {name} T={T}")
    sp = synth.SPECS[name]
    wr, bias = synth.make_router(sp)
    x = synth.activations(name, T, sp.hidden, sp.x_bf16)
    _check_route(m, x, wr, sp.n_experts, sp.top_k, bias)


@pytest.mark.parametrize("k", [1, 16])
@pytest.mark.parametrize("T", [1, 4, 8, 9])
def test_route_k_extremes(m, k, T):
    note(f"route k={k} T={T}")
    wr, _ = synth.make_router("small")
    x = synth.activations("small", T, 512, True)
    _check_route(m, x, wr, 16, k)


@pytest.mark.parametrize("T", [1, 3, 5, 8])
def test_route_zero_input_ties(m, T):
    note(f"route zero input T={T}")
    wr, _ = synth.make_router("small")
    x = np.zeros((T, 512), np.uint16)
    _, idx, tw, _, _, _ = _route_gpu(m, x, wr, 16, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (T, 1)))
    assert np.array_equal(tw, np.full((T, 4), 0.25, np.float32))


def test_route_full_size_decode_tokens(m):
    """The decode router (4096 x 256, bf16) on 64 separate one-token calls, 16 three-token calls and 8
    eight-token calls."""
    sp = synth.SPECS["decode"]
    wr, _ = synth.make_router(sp)
    x = synth.activations("decode", 176, sp.hidden, True, seed=977)
    for i in range(64):
        _check_route(m, x[i:i + 1], wr, sp.n_experts, sp.top_k)
    for i in range(16):
        _check_route(m, x[64 + 3 * i: 67 + 3 * i], wr, sp.n_experts, sp.top_k)
    for i in range(8):
        _check_route(m, x[112 + 8 * i: 120 + 8 * i], wr, sp.n_experts, sp.top_k)
    note("route decode tokens: 64 x T=1, 16 x T=3, 8 x T=8")


def _near_tie_router(H, E, seed):
    """A bf16 router with duplicated rows (exact logit ties, broken by the lower index) and rows that differ from
    another in one small entry (logits a few ulps apart)."""
    wr, _ = synth.make_router("decode")
    w = synth.bf16_bits_to_f32(wr[:E, :H]).copy()
    g = np.random.default_rng(seed)
    for a, b in ((5, 200), (17, 18), (0, 255), (100, 40)):
        if max(a, b) < E:
            w[b] = w[a]
    for a, b in ((7, 8), (90, 91), (150, 30)):
        if max(a, b) < E:
            w[b] = w[a]
            w[b, g.integers(H)] += np.float32(2.0 ** -12)
    return synth.to_bf16_bits(w)


@pytest.mark.parametrize("T", [9, 64, 300])
def test_route_many_tokens_near_ties(m, T):
    """Many-token routing on a router with duplicated and nearly duplicated expert rows, tokens built to sit near
    the selection boundary (copies of a few tokens, a zero token), with and without a bias: the bounded
    matrix-core router must give the full binary64 router's indices and weights bit for bit."""
    note(f"route near ties T={T}")
    H, E, k = 4096, 256, 8
    w = _near_tie_router(H, E, T)
    x = synth.activations("decode", T, H, True, seed=3100 + T).copy()
    x[1] = 0
    if T > 4:
        x[3] = x[2]
        x[4] = synth.to_bf16_bits(synth.bf16_bits_to_f32(x[2]) * np.float32(2.0 ** 9))
    for bias in (None, synth.normal_f32(5, 9, (E,), 0.5)):
        _check_route(m, x, w, E, k, bias)


def test_route_many_tokens_subnormal_and_large_inputs(m):
    """Tokens and router rows holding subnormal bf16 values (which matrix cores may flush: those tokens and experts
    take the exact sum for every expert), tokens scaled by 2^40 and 2^-60, and a top-k of 1 and of 64."""
    note("route subnormal / large inputs")
    H, E, T = 2048, 96, 40
    wr, _ = synth.make_router("small")
    wf = synth.bf16_bits_to_f32(synth.make_router("decode")[0][:E, :H]).copy()
    wf[3, 10] = np.float32(2.0 ** -130)                   # subnormal in bf16 (and fp32)
    w = synth.to_bf16_bits(wf)
    xf = synth.bf16_bits_to_f32(synth.activations("decode", T, H, True, seed=3200)).copy()
    xf[5, 7] = np.float32(2.0 ** -128)
    xf[6] *= np.float32(2.0 ** 40)
    xf[7] *= np.float32(2.0 ** -60)
    x = synth.to_bf16_bits(xf)
    for k in (1, 8, 64):
        _check_route(m, x, w, E, k)


@pytest.mark.parametrize("T", [1, 3, 300])
def test_route_inputs_only_4_byte_aligned(m, T):
    """x and the router at addresses that are 4-byte but not 16-byte aligned (views 2 bf16 values into larger
    buffers): the routers that read rows with 16-byte loads are skipped, and the result is the same bits as from
    aligned inputs, and the oracle's."""
    note(f"route unaligned T={T}")
    H, E, k = 4096, 256, 8
    w, _ = synth.make_router("decode")
    x = synth.activations("decode", T, H, True, seed=3300 + T)
    bias = synth.normal_f32(5, 11, (E,), 0.5)

    def unaligned(a):
        buf = torch.empty(a.size + 8, dtype=torch.bfloat16, device="cuda")
        v = buf[2: 2 + a.size].view(a.shape)
        v.copy_(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16))
        assert v.data_ptr() % 16 != 0 and v.data_ptr() % 4 == 0
        return v

    i32 = dict(dtype=torch.int32, device="cuda")
    outs = []
    for xd, wd in ((dev_x(x), dev_x(w)), (unaligned(x), unaligned(w))):
        idx = torch.empty(T, k, **i32)
        tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
        off = torch.empty(E + 1, **i32)
        perm = torch.empty(T * k, **i32)
        act = torch.full((E + 1,), -7, **i32)
        ws = torch.empty(max(m.moe_route_workspace(T, E, k), 256), dtype=torch.uint8, device="cuda")
        m.moe_route(xd, wd, E, k, idx, tw, off, perm, act, ws, bias=torch.from_numpy(bias).cuda())
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), tw.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    _, oi, ow = oracle.route(x, w, k, bias)
    assert np.array_equal(outs[1][0], oi)
    assert np.abs(outs[1][1].astype(np.float64) - ow).max() <= 1e-6


def test_route_summation_order_golden(m):
    """tests/golden/router_order.txt: cancellation cases where the fixed order decides the logit."""
    from test_oracle_layer import _router_order_cases
    for name, H, entries, want in _router_order_cases():
        # also zero-padded to 256 columns (padding adds exact zeros to the partials), which takes the
        # small-batch router kernel
        for Hp in (H, 256):
            note(f"route order {name} H={Hp}")
            x = np.ones((1, Hp), np.float32)
            w = np.zeros((2, Hp), np.float32)
            for h, v in entries:
                w[0, h] = v
            lg, _, _, _, _, _ = _route_gpu(m, x, w, 2, 1)
            assert lg[0, 0] == np.float32(want), (name, Hp, lg[0, 0])


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------
_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        sp = synth.SPECS[name]
        _LAYERS[name] = synth.make_layer(sp) if sp.hidden >= 4096 else synth.make_layer(sp, quantizer=oracle.quantize)
    return _LAYERS[name]


_DEV = {}


def _run_layer(m, L, x, path):
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    key = (L.spec.name, path)
    if key not in _DEV:
        if len(_DEV) > 3:
            _DEV.clear()
        _DEV[key] = DeviceLayer.from_synth(L, path=path)
    DL = _DEV[key]
    b = LayerBuffers.allocate(DL, x.shape[0])
    forward(DL, dev_x(x), b)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in
            dict(y=b.y, slot_out=b.slot_out, shared_out=b.shared_out, topk_idx=b.topk_idx).items()}


def _oracle_layer(L, x):
    sp = L.spec
    return oracle.layer(x, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up, sp.down_fmt,
                        L.down, L.codebook, bias=L.bias, shared=L.shared)


LAYER_CASES = [
    ("tiny", 4, 0), ("small", 1, 0), ("small", 3, 0), ("small", 4, 0), ("small", 1, 1), ("small", 37, 1),
    ("mid", 2, 0), ("mid", 9, 1), ("mid_fp32", 3, 0),
    # grouped-GEMM kernels: auto path above 4 tokens, and forced at the degenerate sizes
    ("small", 37, 0), ("small", 1, 3), ("small", 3, 3), ("small", 5, 3), ("mid", 70, 0), ("mid", 130, 0),
    ("mid", 300, 0),
    # several tokens per call on the decode kernels (speculative verify micro-batch, up to 8 tokens, T*k <= 64)
    ("small", 2, 0), ("small", 5, 0), ("small", 6, 0), ("small", 8, 0), ("small", 8, 2), ("mid", 5, 0),
    ("mid", 8, 0), ("small", 9, 0),
    # q4k routed experts (4.5 bpw) and mixed formats: decode sizes and grouped GEMM
    ("small_q4k", 1, 0), ("small_q4k", 3, 0), ("small_q4k", 4, 0), ("small_q4k", 3, 1), ("small_q4k", 37, 0),
    ("small_q4k", 3, 3), ("small_q4k", 70, 0),
    ("small_mix_a", 2, 0), ("small_mix_a", 37, 0), ("small_mix_b", 2, 0), ("small_mix_b", 37, 0),
    # one token on each down shape
    ("mid", 1, 0), ("small_mix_b", 1, 0), ("mid", 1, 2),
    # top-16: 16, 32 and 64 slots on the decode kernels, 80 slots on the grouped GEMM
    ("mid_k16", 1, 0), ("mid_k16", 2, 0), ("mid_k16", 4, 0), ("mid_k16", 5, 0),
]


@pytest.mark.parametrize("name,T,path", LAYER_CASES, ids=[f"{a}-T{b}-p{c}" for a, b, c in LAYER_CASES])
def test_layer_matches_oracle(m, name, T, path):
    note(f"layer {name} T={T} path={path}")
    L = _layer(name)
    sp = L.spec
    x = synth.activations(name, T, sp.hidden, sp.x_bf16)
    got = _run_layer(m, L, x, path)
    ref = _oracle_layer(L, x)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    assert rel_l2_rows(got["slot_out"], ref["slot_out"]).max() <= TOL
    if ref["shared_out"] is not None:
        assert rel_l2_rows(got["shared_out"], ref["shared_out"]).max() <= TOL
    err = rel_l2_rows(got["y"], ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL


def test_two_streams_at_once_match_sequential_calls(m):
    """The library keeps no state between calls: two layer calls (grouped GEMM at 37 tokens, verify kernels at 3)
    running at once on two streams, each with its own buffers, give the bits of the same calls run one after the
    other."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note("two streams at once")
    L = _layer("small")
    sp = L.spec
    DL = DeviceLayer.from_synth(L)
    xa = dev_x(synth.activations("small", 37, sp.hidden, True, seed=1400))
    xb = dev_x(synth.activations("small", 3, sp.hidden, True, seed=1401))
    ra, rb = LayerBuffers.allocate(DL, 37), LayerBuffers.allocate(DL, 3)
    forward(DL, xa, ra)
    forward(DL, xb, rb)
    torch.cuda.synchronize()
    ba, bb = LayerBuffers.allocate(DL, 37), LayerBuffers.allocate(DL, 3)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()           # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(4):
        with torch.cuda.stream(s1):
            forward(DL, xa, ba)
        with torch.cuda.stream(s2):
            forward(DL, xb, bb)
    torch.cuda.synchronize()
    assert torch.equal(ba.y, ra.y)
    assert torch.equal(bb.y, rb.y)


@pytest.mark.parametrize("name,T,path", [("small", 1, 0), ("small", 3, 0), ("small", 37, 0), ("small_q4k", 3, 0),
                                         ("small", 5, 3), ("tiny", 4, 0)])
def test_split_ffn_calls_match_the_fused_call(m, name, T, path):
    """moe_expert_gate_up then moe_expert_down, with their own workspace, give the same bits as moe_expert_ffn
    (decode, verify, grouped-GEMM and generic kernels): the halves carry h and its per-token scale exponents
    through the workspace."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers
    note(f"split FFN calls {name} T={T} path={path}")
    L = _layer(name)
    sp = L.spec
    DL = DeviceLayer.from_synth(L, path=path)
    x = dev_x(synth.activations(name, T, sp.hidden, sp.x_bf16, seed=1300 + T))
    b1, b2 = LayerBuffers.allocate(DL, T), LayerBuffers.allocate(DL, T)
    m.moe_route(x, DL.w_router, DL.E, DL.k, b1.topk_idx, b1.topk_w, b1.offsets, b1.perm, b1.active, b1.ws_route,
                bias=DL.bias)
    m.moe_expert_ffn(DL.desc, x, b1.topk_idx, b1.offsets, b1.perm, b1.active, b1.slot_out, b1.shared_out, b1.ws_ffn)
    m.moe_expert_gate_up(DL.desc, x, b1.topk_idx, b1.offsets, b1.perm, b1.active, b2.ws_ffn)
    m.moe_expert_down(DL.desc, x, b1.topk_idx, b1.offsets, b1.perm, b1.active, b2.slot_out, b2.shared_out, b2.ws_ffn)
    torch.cuda.synchronize()
    assert torch.equal(b1.slot_out, b2.slot_out)
    if b1.shared_out is not None:
        assert torch.equal(b1.shared_out, b2.shared_out)


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 3), ("decode", 8), ("long_q4k", 1),
                                    ("long_q4k", 3)])
def test_decode_layer_full_size(m, name, T):
    """Full-size decode layer (hidden 4096, 256 experts, top-8, intermediate
    2048, bf16 shared expert), 2-bit or q4k routed experts, on several
    independent calls of 1 or 3 tokens."""
    L = _layer(name)
    sp = L.spec
    xs = synth.activations("decode", 4 * T, sp.hidden, True, seed=901 + T)
    for c in range(4):
        note(f"decode full size {name} T={T} call {c}")
        x = xs[c * T:(c + 1) * T]
        got = _run_layer(m, L, x, 0)
        ref = _oracle_layer(L, x)
        assert np.array_equal(got["topk_idx"], ref["topk_idx"])
        err = rel_l2_rows(got["y"], ref["y"])
        note(f"  max per-token rel L2 = {err.max():.3e}")
        assert err.max() <= TOL


@pytest.mark.parametrize("name,T", [("small", 8), ("mid", 6), ("decode", 8)])
def test_verify_batch_of_one_repeated_token(m, name, T):
    """T copies of one token: every selected expert gets all T tokens (T / 2 passes over its weights in the
    several-token kernels); every row must match the oracle's single-token output."""
    note(f"repeated token {name} T={T}")
    L = _layer(name)
    sp = L.spec
    x1 = synth.activations(name, 1, sp.hidden, sp.x_bf16, seed=907)
    x = np.repeat(x1, T, axis=0)
    got = _run_layer(m, L, x, 0)
    ref = _oracle_layer(L, x1)
    assert np.array_equal(got["topk_idx"], np.repeat(ref["topk_idx"], T, axis=0))
    err = rel_l2_rows(got["y"], np.repeat(ref["y"], T, axis=0))
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL
    assert np.array_equal(got["y"], np.repeat(got["y"][:1], T, axis=0))


@pytest.mark.parametrize("name,T,chunk", [("prefill", 512, 512), ("long", 2048, 2048), ("long", 2600, 2048),
                                          ("long_q4k", 2048, 2048)])
def test_prefill_layer_full_size(m, name, T, chunk):
    """Full-size prefill layers through the grouped-GEMM kernels, every token of every chunk against one batched
    oracle call on that chunk: routing (indices, offsets, permutation, active list) bit-exact, weights within
    1e-6, and the slot outputs, shared-expert outputs and layer outputs within a per-token relative L2 error of
    1e-3.  This
    covers every (expert, row tile, token tile) work item of the launches at the real shapes: hidden 4096, 256
    experts (the E == 256 tile-offset end), thousands of items remapped over the 8 XCDs, experts with one to
    more than 64 tokens, and a ragged last chunk (2600 = 2048 + 552)."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    # prefill and long share the decode layer's weights; long_q4k has its own 4-bit experts
    L = _layer("long_q4k" if name == "long_q4k" else "decode")
    sp = synth.SPECS[name]
    _, bias = synth.make_router(sp)
    x = synth.activations(name, T, sp.hidden, True)
    DL = DeviceLayer.from_synth(L, path=0)
    DL.bias = None if bias is None else torch.from_numpy(bias).cuda()
    for c0 in range(0, T, chunk):
        xc = x[c0:c0 + chunk]
        n = xc.shape[0]
        note(f"prefill {name} tokens {c0}..{c0 + n}: GPU")
        b = LayerBuffers.allocate(DL, n)
        forward(DL, dev_x(xc), b)
        torch.cuda.synchronize()
        note(f"prefill {name} tokens {c0}..{c0 + n}: oracle")
        ref = oracle.layer(xc, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up,
                           sp.down_fmt, L.down, L.codebook, bias=bias, shared=L.shared)
        assert np.array_equal(b.topk_idx.cpu().numpy(), ref["topk_idx"])
        assert np.abs(b.topk_w.cpu().numpy().astype(np.float64) - ref["topk_w"]).max() <= 1e-6
        assert np.array_equal(b.offsets.cpu().numpy(), ref["offsets"])
        assert np.array_equal(b.perm.cpu().numpy(), ref["perm"])
        act = b.active.cpu().numpy()
        assert np.array_equal(act[: ref["active"][0] + 1], ref["active"][: ref["active"][0] + 1])
        counts = np.diff(ref["offsets"])
        e_slot = rel_l2_rows(b.slot_out.cpu().numpy(), ref["slot_out"])
        e_sh = rel_l2_rows(b.shared_out.cpu().numpy(), ref["shared_out"])
        err = rel_l2_rows(b.y.cpu().numpy(), ref["y"])
        note(f"  {n} tokens, {int((counts > 0).sum())} experts with 1..{counts.max()} tokens: max per-token rel L2 "
             f"y {err.max():.3e}, slots {e_slot.max():.3e}, shared {e_sh.max():.3e}")
        assert e_slot.max() <= TOL
        assert e_sh.max() <= TOL
        assert err.max() <= TOL


def test_combine_matches_numpy(m):
    note("combine")
    g = np.random.default_rng(0)
    for T, k, H, shared in ((1, 8, 4096, True), (7, 3, 100, False), (5, 2, 256, True)):
        o = g.standard_normal((T * k, H)).astype(np.float32)
        w = g.random((T, k)).astype(np.float32)
        s = g.standard_normal((T, H)).astype(np.float32) if shared else None
        y = torch.empty(T, H, dtype=torch.float32, device="cuda")
        m.moe_combine(torch.from_numpy(o).cuda(), torch.from_numpy(w).cuda(),
                      None if s is None else torch.from_numpy(s).cuda(), T, k, H, y)
        want = oracle.combine(o.astype(np.float64), w.astype(np.float64), None if s is None else s.astype(np.float64))
        assert rel_l2_rows(y.cpu().numpy(), want).max() <= 1e-6


def test_binding_rejects_strided_and_mistyped_tensors(m):
    """The binding hands raw device pointers to the library, so it refuses tensors the kernels would misread."""
    note("binding argument checks")
    o = torch.zeros(8, 64, device="cuda")
    w = torch.ones(1, 8, device="cuda")
    y = torch.empty(1, 64, device="cuda")
    with pytest.raises(ValueError):
        m.moe_combine(o.t().contiguous().t(), w, None, 1, 8, 64, y)      # transposed view: not contiguous
    with pytest.raises(TypeError):
        m.moe_combine(o, w.double(), None, 1, 8, 64, y)                  # weights must be fp32
    with pytest.raises(TypeError):
        m.moe_combine(o.cpu(), w, None, 1, 8, 64, y)                     # host memory
    idx64 = torch.zeros(1, 8, dtype=torch.int64, device="cuda")
    with pytest.raises(TypeError):
        m.moe_route(torch.zeros(1, 256, device="cuda"), torch.zeros(8, 256, device="cuda"), 8, 8, idx64, w,
                    torch.zeros(9, dtype=torch.int32, device="cuda"), torch.zeros(8, dtype=torch.int32, device="cuda"),
                    torch.zeros(9, dtype=torch.int32, device="cuda"), torch.zeros(1024, dtype=torch.uint8,
                                                                                  device="cuda"))


# ----------------------------------------------------------------------------
# directional steering fused into the combine
# ----------------------------------------------------------------------------
STEER_CASES = [
    # T, k, H, shared, offset (floats; a nonzero offset makes the rows unaligned -> the any-shape kernel)
    (1, 8, 4096, True, 0),       # decode shape, 4 outputs per thread, one group per thread
    (6, 8, 7168, True, 0),       # two groups of 4 per thread
    (5, 4, 256, True, 0),
    (3, 6, 4096, False, 0),      # top-k without a compiled specialisation
    (4, 8, 8196, True, 0),       # longer than the register-resident kernel holds
    (7, 3, 100, False, 0),       # H % 4 != 0
    (2, 8, 4096, True, 1),       # unaligned rows
]


@pytest.mark.parametrize("T,k,H,shared,off", STEER_CASES)
def test_combine_steer_matches_oracle(m, T, k, H, shared, off):
    note(f"combine_steer T={T} k={k} H={H} shared={shared} off={off}")
    g = np.random.default_rng(1000 + T * 31 + H)
    o = g.standard_normal((T * k, H)).astype(np.float32)
    w = g.random((T, k)).astype(np.float32)
    s = g.standard_normal((T, H)).astype(np.float32) if shared else None
    v = g.standard_normal(H).astype(np.float32)
    vu = (v / np.linalg.norm(v)).astype(np.float32)

    def dev(a):
        if a is None:
            return None
        buf = torch.empty(a.size + off, dtype=torch.float32, device="cuda")
        buf[off:] = torch.from_numpy(a.reshape(-1)).cuda()
        return buf[off:]

    od, wd, sd = dev(o), dev(w), dev(s)
    y = torch.empty(T * H + off, dtype=torch.float32, device="cuda")[off:]
    plain = torch.empty(T, H, dtype=torch.float32, device="cuda")
    m.moe_combine(od, wd, sd, T, k, H, plain)
    comb = oracle.combine(o.astype(np.float64), w.astype(np.float64), None if s is None else s.astype(np.float64))
    for vec, F in ((vu, 1.0), (vu, 2.0), (v, 0.01), (vu, -0.5)):
        m.moe_combine_steer(od, wd, sd, T, k, H, dev(vec), F, y)
        want = oracle.steer(comb, vec.astype(np.float64), F)
        err = rel_l2_rows(y.cpu().numpy(), want)
        assert err.max() <= 1e-5, (F, err.max())
    # strength 0 leaves the plain combine's values untouched
    m.moe_combine_steer(od, wd, sd, T, k, H, dev(vu), 0.0, y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().reshape(T, H), plain.cpu().numpy())
    # unit direction and F = 1: the component along v is gone
    m.moe_combine_steer(od, wd, sd, T, k, H, dev(vu), 1.0, y)
    yy = y.cpu().numpy().reshape(T, H).astype(np.float64)
    assert np.abs(yy @ vu.astype(np.float64)).max() <= 1e-5 * np.linalg.norm(comb, axis=1).max()


@pytest.mark.parametrize("name,T", [("small", 37), ("mid", 9), ("decode", 1)])
def test_layer_with_steering_matches_oracle(m, name, T):
    """The whole layer with a unit steering direction at strength 1, against the oracle's layer + steering."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note(f"layer with steering {name} T={T}")
    L = _layer(name)
    sp = L.spec
    x = synth.activations(name, T, sp.hidden, sp.x_bf16)
    v = synth.steer_direction(sp.hidden)
    DL = DeviceLayer.from_synth(L)
    DL.set_steering(v, 1.0)
    b = LayerBuffers.allocate(DL, T)
    forward(DL, dev_x(x), b)
    ref = oracle.layer(x, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up, sp.down_fmt,
                       L.down, L.codebook, bias=L.bias, shared=L.shared, steering=(v, 1.0))
    err = rel_l2_rows(b.y.cpu().numpy(), ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL
    # the routed part is unchanged by steering: same slot outputs as without it
    DL.set_steering(None)
    b2 = LayerBuffers.allocate(DL, T)
    forward(DL, dev_x(x), b2)
    torch.cuda.synchronize()
    assert torch.equal(b.slot_out, b2.slot_out)


# ----------------------------------------------------------------------------
# HIP graph capture of the whole layer
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name,T,steer", [("mid", 1, False), ("mid", 3, True), ("mid", 8, False),
                                          ("mid", 37, True)])
def test_layer_graph_replay_matches_eager(m, name, T, steer):
    """route -> expert FFN -> combine captured once in a HIP graph and replayed on new inputs (copied into the
    captured input buffer between replays, with eager work and synchronizations in between): every replay equals
    an eager run on the same input bit for bit."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note(f"graph replay {name} T={T} steer={steer}")
    L = _layer(name)
    sp = L.spec
    DL = DeviceLayer.from_synth(L)
    if steer:
        DL.set_steering(synth.steer_direction(sp.hidden), 1.0)
    xs = [dev_x(synth.activations(name, T, sp.hidden, sp.x_bf16, seed=600 + r)) for r in range(3)]
    xin = torch.empty_like(xs[0])
    xin.copy_(xs[0])
    bg, be = LayerBuffers.allocate(DL, T), LayerBuffers.allocate(DL, T)
    forward(DL, xin, bg)                                       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            forward(DL, xin, bg)
    torch.cuda.synchronize()
    for r in range(3):
        xin.copy_(xs[r])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        forward(DL, xs[r], be)
        torch.cuda.synchronize()
        assert torch.equal(bg.topk_idx, be.topk_idx)
        assert torch.equal(bg.y, be.y), f"replay {r}"


# ----------------------------------------------------------------------------
# degenerate blocks: zero scales
# ----------------------------------------------------------------------------
def _zero_scales(blocks: np.ndarray, fmt: int, frac: float, seed: int) -> np.ndarray:
    """A copy of canonical blocks with the fp16 scale d (and dmin for q2k/q4k) of a random fraction of blocks
    set to +0: such blocks decode to zeros, and the grouped GEMM must keep its running block scale across them."""
    bb = oracle.BLOCK_BYTES[fmt]
    b = blocks.copy().reshape(-1, bb)
    pick = np.random.default_rng(seed).random(b.shape[0]) < frac
    b[pick, 0:2] = 0
    if fmt != oracle.FMT_IQ2X:
        b[pick, 2:4] = 0
    return b.reshape(-1)


@pytest.mark.parametrize("name,T,path", [("small", 1, 0), ("small", 3, 0), ("small", 6, 0), ("small", 37, 0),
                                         ("small", 3, 3), ("small", 2, 1), ("small_q4k", 1, 0), ("small_q4k", 37, 0)])
def test_layer_with_zero_scale_blocks(m, name, T, path):
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note(f"zero-scale blocks {name} T={T} path={path}")
    L = _layer(name)
    sp = L.spec
    gate = _zero_scales(L.gate, sp.gate_up_fmt, 0.2, 1)
    up = _zero_scales(L.up, sp.gate_up_fmt, 0.2, 2)
    down = _zero_scales(L.down, sp.down_fmt, 0.2, 3)
    DL = DeviceLayer(sp.hidden, sp.inter, sp.n_experts, sp.top_k, sp.gate_up_fmt, sp.down_fmt, gate, up, down,
                     L.codebook, L.w_router, L.bias, L.shared, path=path)
    x = synth.activations(name, T, sp.hidden, sp.x_bf16, seed=950 + T)
    b = LayerBuffers.allocate(DL, T)
    forward(DL, dev_x(x), b)
    torch.cuda.synchronize()
    ref = oracle.layer(x, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, gate, up, sp.down_fmt, down,
                       L.codebook, bias=L.bias, shared=L.shared)
    assert np.array_equal(b.topk_idx.cpu().numpy(), ref["topk_idx"])
    assert rel_l2_rows(b.slot_out.cpu().numpy(), ref["slot_out"]).max() <= TOL
    err = rel_l2_rows(b.y.cpu().numpy(), ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL


# ----------------------------------------------------------------------------
# activation range: the per-group scaling of the e4m3 pieces and the fp16 tiles
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("scale_exp", [-20, -10, -6, 6, 12, 16])
@pytest.mark.parametrize("T,path", [(1, 0), (3, 0), (37, 0), (37, 3), (5, 3)])
def test_layer_activation_scales(m, scale_exp, T, path):
    """x scaled by powers of two from 2^-20 to 2^16 (exact in bf16): routing, slot and layer outputs still match
    the oracle on the decode, verify and grouped-GEMM kernels.  The routed SwiGLU output h grows as |x|^2 and is
    carried in fp16 as h * 2^-s with s from the token's largest |x|; without that scale 2^-10 falls into fp16's
    subnormals and 2^8 overflows.  The grouped GEMM also reads x in fp16 after a power-of-two prescale of each
    token's row: without it 2^16 would overflow fp16 (65504) and 2^-20 would fall into its subnormals."""
    note(f"activation scale 2^{scale_exp} T={T} path={path}")
    L = _layer("small")
    sp = L.spec
    x = synth.to_bf16_bits(synth.bf16_bits_to_f32(synth.activations("small", T, sp.hidden, True, seed=970 + T))
                           * np.float32(2.0 ** scale_exp))
    got = _run_layer(m, L, x, path)
    ref = _oracle_layer(L, x)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    assert rel_l2_rows(got["slot_out"], ref["slot_out"]).max() <= TOL
    err = rel_l2_rows(got["y"], ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL


@pytest.mark.parametrize("name", ["small", "small_q4k"])
@pytest.mark.parametrize("T,path", [(1, 0), (3, 0), (3, 3), (37, 0)])
def test_layer_zero_spike_and_mixed_scale_tokens(m, name, T, path):
    """One call mixing an all-zero token, a one-hot spike token (a single 64.0) and tokens scaled by 2^-10 and
    2^12 next to unit-scale ones: each token carries its own h scale, also inside a shared grouped-GEMM token
    tile, and the zero token's output is exactly zero."""
    note(f"zero / spike / mixed-scale tokens {name} T={T} path={path}")
    L = _layer(name)
    sp = L.spec
    xf = synth.bf16_bits_to_f32(synth.activations(name, T, sp.hidden, True, seed=990 + T)).copy()
    xf[0] = 0.0
    if T > 1:
        xf[1] = 0.0
        xf[1, 7] = 64.0
    if T > 2:
        xf[2] *= np.float32(2.0 ** -10)
    if T > 3:
        xf[3] *= np.float32(2.0 ** 12)
    x = synth.to_bf16_bits(xf)
    got = _run_layer(m, L, x, path)
    ref = _oracle_layer(L, x)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    assert not np.any(got["y"][0]), "an all-zero token must give an all-zero output"
    assert rel_l2_rows(got["slot_out"], ref["slot_out"]).max() <= TOL
    err = rel_l2_rows(got["y"], ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL


# ----------------------------------------------------------------------------
# the single-call layer (moe_layer): same bits as the three calls
# ----------------------------------------------------------------------------
LAYER_CALL_CASES = [
    # one token: routing selected inside the gate/up launch (MFMA iq2x kernel; VALU q4k kernel; top-16)
    ("small", 1, False), ("decode", 1, False), ("decode", 1, True), ("small_q4k", 1, False),
    ("small_mix_a", 1, False), ("small_mix_b", 1, False), ("mid_k16", 1, False), ("mid", 1, True),
    # several tokens: the three calls inside one (2..8 tokens on the verify kernels, with one wave per workgroup
    # at hidden 512 and eight at 4096, top-16 with 64 slots, a bias, steering; then the grouped GEMM)
    ("small", 3, False), ("small", 8, True), ("decode", 2, False), ("decode", 3, True), ("decode", 8, False),
    ("mid", 5, False), ("mid_k16", 4, False), ("small", 37, True), ("mid", 70, False), ("tiny", 4, False),
]


@pytest.mark.parametrize("name,T,steer", LAYER_CALL_CASES, ids=[f"{a}-T{b}-s{int(c)}" for a, b, c in LAYER_CALL_CASES])
def test_layer_call_matches_the_three_calls(m, name, T, steer):
    """moe_layer writes the same routing outputs (indices, weights, offsets, permutation, active list, optional
    logits), slot and shared outputs and layer output, bit for bit, as moe_route + moe_expert_ffn + moe_combine
    (or moe_combine_steer); the one-token calls select their experts inside the gate/up launch."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward, forward_layer
    L = _layer(name)
    sp = L.spec
    DL = DeviceLayer.from_synth(L)
    if steer:
        DL.set_steering(synth.steer_direction(sp.hidden), 1.0)
    for r in range(3 if T == 1 else 1):
        note(f"layer call {name} T={T} steer={steer} input {r}")
        x = dev_x(synth.activations(name, T, sp.hidden, sp.x_bf16, seed=1700 + 10 * T + r))
        for with_logits in (False, True):
            b1 = LayerBuffers.allocate(DL, T, with_logits=with_logits)
            b2 = LayerBuffers.allocate(DL, T, with_logits=with_logits)
            b2.active.fill_(-5)
            b2.offsets.fill_(-5)
            forward(DL, x, b1)
            forward_layer(DL, x, b2)
            torch.cuda.synchronize()
            n_act = int(b1.active[0])
            assert torch.equal(b1.topk_idx, b2.topk_idx)
            assert torch.equal(b1.topk_w, b2.topk_w)
            assert torch.equal(b1.offsets, b2.offsets)
            assert torch.equal(b1.perm, b2.perm)
            assert torch.equal(b1.active[: n_act + 1], b2.active[: n_act + 1])
            if with_logits:
                assert torch.equal(b1.logits, b2.logits)
            assert torch.equal(b1.slot_out, b2.slot_out)
            if b1.shared_out is not None:
                assert torch.equal(b1.shared_out, b2.shared_out)
            assert torch.equal(b1.y, b2.y)
    # and against the oracle once
    xo = synth.activations(name, T, sp.hidden, sp.x_bf16, seed=1700 + 10 * T)
    b = LayerBuffers.allocate(DL, T)
    forward_layer(DL, dev_x(xo), b)
    ref = oracle.layer(xo, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up, sp.down_fmt,
                       L.down, L.codebook, bias=L.bias, shared=L.shared,
                       steering=(synth.steer_direction(sp.hidden), 1.0) if steer else None)
    assert np.array_equal(b.topk_idx.cpu().numpy(), ref["topk_idx"])
    err = rel_l2_rows(b.y.cpu().numpy(), ref["y"])
    note(f"  max per-token rel L2 = {err.max():.3e}")
    assert err.max() <= TOL


@pytest.mark.parametrize("name,T", [("mid", 1), ("decode", 1), ("decode", 3), ("small", 5)])
def test_layer_call_graph_replay_matches_eager(m, name, T):
    """moe_layer at one token (selection in the decode gate/up launch) or a few (the verify kernels) captured once
    in a HIP graph: every replay on new inputs equals an eager call."""
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward_layer
    note(f"layer call graph replay {name} T={T}")
    L = _layer(name)
    sp = L.spec
    DL = DeviceLayer.from_synth(L)
    xs = [dev_x(synth.activations(name, T, sp.hidden, sp.x_bf16, seed=1800 + r)) for r in range(3)]
    xin = torch.empty_like(xs[0])
    xin.copy_(xs[0])
    bg, be = LayerBuffers.allocate(DL, T), LayerBuffers.allocate(DL, T)
    forward_layer(DL, xin, bg)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            forward_layer(DL, xin, bg)
    torch.cuda.synchronize()
    for r in range(3):
        xin.copy_(xs[r])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        forward_layer(DL, xs[r], be)
        torch.cuda.synchronize()
        assert torch.equal(bg.topk_idx, be.topk_idx)
        assert torch.equal(bg.y, be.y), f"replay {r}"


# ----------------------------------------------------------------------------
# the approximate fast mode (MOE_PRECISION_FAST): grouped-GEMM kernels only
# ----------------------------------------------------------------------------
FAST_TOL = 5e-3


@pytest.mark.parametrize("name,T", [("small", 37), ("mid", 300), ("small_mix_a", 37), ("small_mix_b", 37),
                                    ("prefill", 512), ("long", 2048)])
def test_fast_mode_within_its_tolerance(m, name, T):
    """The opt-in fast mode (q2k down weights as one fp16 fused multiply-add each, the shared expert's h in one bf16
    plane) against the oracle at its stated 5e-3 per-token relative L2, with routing unchanged; it must differ from
    the exact mode (it is a different computation) on the layers it applies to."""
    from bit_quantized_moe_permute_amd import PRECISION_FAST
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note(f"fast mode {name} T={T}")
    L = _layer("decode" if name in ("prefill", "long") else name)
    sp = synth.SPECS[name]
    _, bias = synth.make_router(sp)
    x = synth.activations(name, T, sp.hidden, True)
    DL = DeviceLayer.from_synth(L)
    DL.bias = None if bias is None else torch.from_numpy(bias).cuda()
    fast = DL.make_desc(precision=PRECISION_FAST)
    b_ex, b_fa = LayerBuffers.allocate(DL, T), LayerBuffers.allocate(DL, T)
    forward(DL, dev_x(x), b_ex)
    forward(DL, dev_x(x), b_fa, desc=fast)
    torch.cuda.synchronize()
    ref = oracle.layer(x, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up, sp.down_fmt,
                       L.down, L.codebook, bias=bias, shared=L.shared)
    assert torch.equal(b_fa.topk_idx, b_ex.topk_idx)
    err = rel_l2_rows(b_fa.y.cpu().numpy(), ref["y"])
    err_ex = rel_l2_rows(b_ex.y.cpu().numpy(), ref["y"])
    note(f"  fast max per-token rel L2 = {err.max():.3e} (exact {err_ex.max():.3e})")
    assert err.max() <= FAST_TOL
    assert err_ex.max() <= TOL
    assert not torch.equal(b_fa.y, b_ex.y)


@pytest.mark.parametrize("name,T", [("small", 1), ("small", 3), ("small", 8), ("small_q4k", 37)])
def test_fast_mode_is_exact_where_it_does_not_apply(m, name, T):
    """Decode and verify calls (up to 8 tokens), and q4k routed experts with no shared expert planes of their own,
    give the exact mode's bits in fast mode except for the shared expert's single-plane h."""
    from bit_quantized_moe_permute_amd import PRECISION_FAST
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward
    note(f"fast mode not applied {name} T={T}")
    L = _layer(name)
    sp = L.spec
    x = dev_x(synth.activations(name, T, sp.hidden, True, seed=2100 + T))
    DL = DeviceLayer.from_synth(L)
    b_ex, b_fa = LayerBuffers.allocate(DL, T), LayerBuffers.allocate(DL, T)
    forward(DL, x, b_ex)
    forward(DL, x, b_fa, desc=DL.make_desc(precision=PRECISION_FAST))
    torch.cuda.synchronize()
    assert torch.equal(b_fa.slot_out, b_ex.slot_out)
    if T <= 8:
        assert torch.equal(b_fa.y, b_ex.y)
