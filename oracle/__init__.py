"""CPU oracle for the routed 2-bit MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The GPU library never does, and this package never
imports the GPU library: the two share no code.  Every result here is computed
in binary64 by the plain C in ``moe_oracle.c`` (formats, quantizers, router,
permutation, SwiGLU experts, combine, steering); this module only marshals numpy arrays.

Sources: the routed experts are the only quantized tensors, up/gate in
IQ2_XXS, down in Q2_K, shared experts and routing kept at full precision
("antirez가 만든 DeepSeek V4 Flash 전용 로컬 추론 엔진 ds4", summary bullets on
2-bit quantization; "antirez/ds4 — Metal용 … 완벽 가이드", section on the design
philosophy).  The block layouts and arithmetic are this project's readings of
those format names; see the header comment of moe_oracle.c.

Parity status: formats, quantizers, routing, permutation, FFN, combine and
steering are each pinned by tests in tests/test_oracle_*.py (hand-worked
blocks, closed forms, library routines on the special cases, brute force,
invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_IQ2X, FMT_Q2K, FMT_Q4K = 1, 2, 3
BLOCK_BYTES = {FMT_IQ2X: 66, FMT_Q2K: 84, FMT_Q4K: 144}
QK = 256

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, binary64, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_dequant.argtypes = [i32, vp, i64, vp, vp]
        L.oracle_quantize.argtypes = [i32, vp, i64, vp, vp]
        L.oracle_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, i32, vp, vp, vp]
        L.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_expert_ffn.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp]
        L.oracle_shared_ffn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_steer.argtypes = [vp, vp, ctypes.c_double, i32, i32, vp]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (the process-wide OpenMP runtime the library links)."""
    lib()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def get_threads() -> int:
    lib()
    return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a: np.ndarray) -> int:
    """0 = fp32 array, 1 = bf16 bit patterns held as uint16."""
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"activations/weights must be float32 or bf16 bits (uint16), got {a.dtype}")


# ----------------------------------------------------------------------------
# scalar conversions
# ----------------------------------------------------------------------------
def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(int(h))


def f64_to_f16(x: float) -> int:
    return lib().oracle_f64_to_f16(float(x))


def bf16_to_f64(b: int) -> float:
    return lib().oracle_bf16_to_f64(int(b))


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------
def dequantize(fmt: int, blocks: np.ndarray, codebook: np.ndarray | None = None) -> np.ndarray:
    """Canonical blocks (uint8, n*block_bytes) -> float64 weights (n*256)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    bb = BLOCK_BYTES[fmt]
    assert blocks.size % bb == 0
    n = blocks.size // bb
    out = np.empty(n * QK, dtype=np.float64)
    cb = None
    if fmt == FMT_IQ2X:
        cb = np.ascontiguousarray(codebook, dtype=np.uint8).reshape(256 * 8)
    lib().oracle_dequant(fmt, _p(blocks), n, _p(cb), _p(out))
    return out


def quantize(fmt: int, w: np.ndarray, codebook: np.ndarray | None = None) -> np.ndarray:
    """float32 weights (multiple of 256, flattened row-major) -> canonical blocks (uint8)."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert w.size % QK == 0
    n = w.size // QK
    out = np.zeros(n * BLOCK_BYTES[fmt], dtype=np.uint8)
    cb = None
    if fmt == FMT_IQ2X:
        cb = np.ascontiguousarray(codebook, dtype=np.uint8).reshape(256 * 8)
    lib().oracle_quantize(fmt, _p(w), n, _p(cb), _p(out))
    return out


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------
def route(x: np.ndarray, w_router: np.ndarray, k: int, bias: np.ndarray | None = None):
    """x [T][H], w_router [E][H] (fp32 or bf16 bits) -> (logits fp32 [T][E], idx int32 [T][k], w f64 [T][k])."""
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router)
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.shape[1] == H and 1 <= k <= E
    logits = np.empty((T, E), dtype=np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    tw = np.empty((T, k), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_route(_p(x), _dt(x), T, H, _p(w_router), _dt(w_router), E, _p(b), k, _p(logits), _p(idx), _p(tw))
    return logits, idx, tw


def permute(topk_idx: np.ndarray, n_experts: int):
    """-> (offsets int32 [E+1], perm int32 [T*k], active int32 [1+E])."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = topk_idx.shape
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    perm = np.empty(max(T * k, 1), dtype=np.int32)
    active = np.zeros(n_experts + 1, dtype=np.int32)
    lib().oracle_permute(_p(topk_idx), T, k, n_experts, _p(offsets), _p(perm), _p(active))
    return offsets, perm[: T * k], active


def expert_ffn(x, topk_idx, fmt_gu, Wg, Wu, fmt_d, Wd, codebook, n_experts, inter):
    """Routed experts for every slot -> float64 [T*k][H] in slot order."""
    x = np.ascontiguousarray(x)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, H = x.shape
    k = topk_idx.shape[1]
    out = np.zeros((T * k, H), dtype=np.float64)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8).reshape(-1) if codebook is not None else np.zeros(2048, np.uint8)
    Wg = np.ascontiguousarray(Wg, dtype=np.uint8)
    Wu = np.ascontiguousarray(Wu, dtype=np.uint8)
    Wd = np.ascontiguousarray(Wd, dtype=np.uint8)
    lib().oracle_expert_ffn(_p(x), _dt(x), T, H, inter, n_experts, k, _p(topk_idx), fmt_gu, _p(Wg), _p(Wu),
                            fmt_d, _p(Wd), _p(cb), _p(out))
    return out


def shared_ffn(x, Wg, Wu, Wd):
    """bf16 shared expert (weights as uint16 bit patterns) -> float64 [T][H]."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    Is = Wg.shape[0]
    out = np.empty((T, H), dtype=np.float64)
    Wg = np.ascontiguousarray(Wg, dtype=np.uint16)
    Wu = np.ascontiguousarray(Wu, dtype=np.uint16)
    Wd = np.ascontiguousarray(Wd, dtype=np.uint16)
    lib().oracle_shared_ffn(_p(x), _dt(x), T, H, Is, _p(Wg), _p(Wu), _p(Wd), _p(out))
    return out


def combine(slot_out, topk_w, shared_out=None):
    """y[t] = sum_j w[t][j] o[t*k+j] + s[t] in binary64."""
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float64)
    T, k = topk_w.shape
    slot_out = np.ascontiguousarray(slot_out, dtype=np.float64)
    H = slot_out.shape[1]
    y = np.empty((T, H), dtype=np.float64)
    s = None if shared_out is None else np.ascontiguousarray(shared_out, dtype=np.float64)
    lib().oracle_combine(_p(slot_out), _p(topk_w), _p(s), T, k, H, _p(y))
    return y


def steer(y, v, F):
    """y[t] - F * v * dot(v, y[t]) per token in binary64 (directional steering of the FFN output)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    T, H = y.shape
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1)
    if v.shape[0] != H:
        raise ValueError("steering direction must have one entry per hidden unit")
    out = np.empty_like(y)
    lib().oracle_steer(_p(y), _p(v), float(F), T, H, _p(out))
    return out


def layer(x, w_router, k, n_experts, inter, fmt_gu, Wg, Wu, fmt_d, Wd, codebook, bias=None, shared=None,
          steering=None):
    """Whole layer: route -> permute -> routed experts (+ shared) -> combine.

    ``steering`` = (v, F) applies directional steering to the combined output.
    Returns a dict with every intermediate the GPU path exposes.
    """
    logits, idx, tw = route(x, w_router, k, bias)
    offsets, perm, active = permute(idx, n_experts)
    slot_out = expert_ffn(x, idx, fmt_gu, Wg, Wu, fmt_d, Wd, codebook, n_experts, inter)
    s = shared_ffn(x, *shared) if shared is not None else None
    y = combine(slot_out, tw, s)
    if steering is not None:
        y = steer(y, *steering)
    return dict(logits=logits, topk_idx=idx, topk_w=tw, offsets=offsets, perm=perm, active=active,
                slot_out=slot_out, shared_out=s, y=y)
