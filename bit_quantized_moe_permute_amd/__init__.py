"""Routed 2-bit MoE FFN layer for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in include/moe2bit.h (libmoe2bit.so, built
in-tree by build.py).  The functions below have the C names and only marshal
arguments: torch tensors are passed as device pointers, the stream is torch's
current HIP stream, and every step of the layer runs in the library's HIP
kernels.  There is no fallback: if the library is missing or fails to load,
importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe2bit.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE = 0, 1, 2, 3
DT_F32, DT_BF16 = 0, 1
FMT_IQ2X, FMT_Q2K, FMT_Q4K = 1, 2, 3
PATH_AUTO, PATH_GENERIC, PATH_GEMV, PATH_GEMM = 0, 1, 2, 3
PRECISION_EXACT, PRECISION_FAST = 0, 1
ABI_VERSION = 3

EXPORTS = [
    "moe_abi_version", "moe_sync_debug", "moe_last_error", "moe_weight_bytes", "moe_prepare_weights",
    "moe_dequantize", "moe_route_workspace", "moe_route", "moe_expert_ffn_workspace", "moe_expert_ffn",
    "moe_expert_gate_up", "moe_expert_down", "moe_combine", "moe_combine_steer", "moe_probe_stream_read",
    "moe_expert_ffn_noalloc", "moe_layer_workspace", "moe_layer",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class LayerDesc(ctypes.Structure):
    """moe_layer_desc (include/moe2bit.h)."""
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("gate_up_fmt", ctypes.c_int32), ("down_fmt", ctypes.c_int32),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
        ("shared_inter", ctypes.c_int32),
        ("shared_gate", ctypes.c_void_p), ("shared_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p),
        ("path", ctypes.c_int32),
        ("precision", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_moe_permute_amd/build.py` "
                          f"(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_sync_debug.restype = ctypes.c_int
    L.moe_sync_debug.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_weight_bytes.restype = sz
    L.moe_weight_bytes.argtypes = [i32, i64, i64, i64]
    L.moe_prepare_weights.restype = ctypes.c_int
    L.moe_prepare_weights.argtypes = [i32, i64, i64, i64, vp, vp, vp]
    L.moe_dequantize.restype = ctypes.c_int
    L.moe_dequantize.argtypes = [i32, vp, i64, i64, i64, i64, i64, vp, vp, vp]
    L.moe_route_workspace.restype = sz
    L.moe_route_workspace.argtypes = [i32, i32, i32]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn_workspace.restype = sz
    L.moe_expert_ffn_workspace.argtypes = [ctypes.POINTER(LayerDesc), i32]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_gate_up.restype = ctypes.c_int
    L.moe_expert_gate_up.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_down.restype = ctypes.c_int
    L.moe_expert_down.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.restype = ctypes.c_int
    L.moe_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    L.moe_combine_steer.restype = ctypes.c_int
    L.moe_combine_steer.argtypes = [vp, vp, vp, i32, i32, i32, vp, ctypes.c_float, vp, vp]
    L.moe_expert_ffn_noalloc.restype = ctypes.c_int
    L.moe_expert_ffn_noalloc.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_layer_workspace.restype = sz
    L.moe_layer_workspace.argtypes = [ctypes.POINTER(LayerDesc), i32]
    L.moe_layer.restype = ctypes.c_int
    L.moe_layer.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                            ctypes.c_float, vp, vp, sz, vp]
    L.moe_probe_stream_read.restype = ctypes.c_int
    L.moe_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    if L.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"libmoe2bit ABI {L.moe_abi_version()} != binding ABI {ABI_VERSION}")
    return L


lib = _load()


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib.moe_last_error().decode())


def _ptr(t, dtype=None):
    """Device pointer of a contiguous GPU tensor (None passes through); dtype, when given, is checked."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("expected a GPU tensor (the library takes device pointers)")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t):
    import torch
    return _ptr(t, torch.int32)


def _f32(t):
    import torch
    return _ptr(t, torch.float32)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, n: int, what: str):
    """Host-side size check before a device pointer is handed to the library: the kernels index t up to n
    elements (None passes)."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{what}: {t.numel()} elements, the call needs {n}")


def _need_bytes(t, n: int, what: str):
    if t is not None and t.numel() * t.element_size() < n:
        raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, the call needs {n}")


def _rows(x, hidden: int | None = None):
    """(T, H) of a [T][H] activation tensor."""
    if x.dim() != 2:
        raise ValueError(f"activations must be [tokens][hidden], got shape {tuple(x.shape)}")
    if hidden is not None and x.shape[1] != hidden:
        raise ValueError(f"activations have {x.shape[1]} columns, the layer has hidden {hidden}")
    return x.shape[0], x.shape[1]


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------------------
# C-ABI calls (same names)
# ----------------------------------------------------------------------------
def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_sync_debug() -> bool:
    return bool(lib.moe_sync_debug())


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def moe_weight_bytes(fmt: int, n_mats: int, rows: int, cols: int) -> int:
    return lib.moe_weight_bytes(fmt, n_mats, rows, cols)


def moe_prepare_weights(fmt, n_mats, rows, cols, canonical, prepared, stream=None):
    nb = moe_weight_bytes(fmt, n_mats, rows, cols)
    _need_bytes(canonical, nb, "canonical")
    _need_bytes(prepared, nb, "prepared")
    _check(lib.moe_prepare_weights(fmt, n_mats, rows, cols, _ptr(canonical), _ptr(prepared), _stream(stream)))


def moe_dequantize(fmt, prepared, n_mats, rows, cols, mat_begin, mat_count, codebook, out, stream=None):
    _need_bytes(prepared, moe_weight_bytes(fmt, n_mats, rows, cols), "prepared")
    _need(out, max(mat_count, 0) * rows * cols, "out")
    if fmt == FMT_IQ2X:
        _need_bytes(codebook, 256 * 8, "codebook")
    _check(lib.moe_dequantize(fmt, _ptr(prepared), n_mats, rows, cols, mat_begin, mat_count, _ptr(codebook),
                              _f32(out), _stream(stream)))


def moe_route_workspace(n_tokens: int, n_experts: int, top_k: int) -> int:
    return lib.moe_route_workspace(n_tokens, n_experts, top_k)


def moe_route(x, w_router, n_experts, top_k, topk_idx, topk_w, expert_offsets, perm, active, ws, bias=None,
              logits=None, stream=None):
    T, H = _rows(x)
    if w_router.dim() != 2 or tuple(w_router.shape) != (n_experts, H):
        raise ValueError(f"w_router must be [{n_experts}][{H}], got shape {tuple(w_router.shape)}")
    _need(topk_idx, T * top_k, "topk_idx")
    _need(topk_w, T * top_k, "topk_w")
    _need(expert_offsets, n_experts + 1, "expert_offsets")
    _need(perm, T * top_k, "perm")
    _need(active, n_experts + 1, "active")
    _need(bias, n_experts, "bias")
    _need(logits, T * n_experts, "logits")
    _check(lib.moe_route(_ptr(x), _dt(x), T, H, _ptr(w_router), _dt(w_router), n_experts, _f32(bias), top_k,
                         _i32(topk_idx), _f32(topk_w), _f32(logits), _i32(expert_offsets), _i32(perm), _i32(active),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn_workspace(desc: LayerDesc, n_tokens: int) -> int:
    return lib.moe_expert_ffn_workspace(ctypes.byref(desc), n_tokens)


def _routing_sizes(desc: LayerDesc, x, topk_idx, expert_offsets, perm, active):
    T, _ = _rows(x, desc.hidden)
    _need(topk_idx, T * desc.top_k, "topk_idx")
    _need(expert_offsets, desc.n_experts + 1, "expert_offsets")
    _need(perm, T * desc.top_k, "perm")
    _need(active, desc.n_experts + 1, "active")
    return T


def _output_sizes(desc: LayerDesc, T: int, slot_out, shared_out):
    _need(slot_out, T * desc.top_k * desc.hidden, "slot_out")
    _need(shared_out, T * desc.hidden, "shared_out")


def moe_expert_ffn(desc: LayerDesc, x, topk_idx, expert_offsets, perm, active, slot_out, shared_out, ws, stream=None):
    T = _routing_sizes(desc, x, topk_idx, expert_offsets, perm, active)
    _output_sizes(desc, T, slot_out, shared_out)
    _check(lib.moe_expert_ffn(ctypes.byref(desc), _ptr(x), _dt(x), T, _i32(topk_idx), _i32(expert_offsets),
                              _i32(perm), _i32(active), _f32(slot_out), _f32(shared_out), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn_noalloc(desc: LayerDesc, x, topk_idx, expert_offsets, perm, active, slot_out, shared_out,
                           stream=None):
    """moe_expert_ffn with the library's static device scratch instead of a workspace (no allocation)."""
    T = _routing_sizes(desc, x, topk_idx, expert_offsets, perm, active)
    _output_sizes(desc, T, slot_out, shared_out)
    _check(lib.moe_expert_ffn_noalloc(ctypes.byref(desc), _ptr(x), _dt(x), T, _i32(topk_idx), _i32(expert_offsets),
                                      _i32(perm), _i32(active), _f32(slot_out), _f32(shared_out), _stream(stream)))


def moe_expert_gate_up(desc: LayerDesc, x, topk_idx, expert_offsets, perm, active, ws, stream=None):
    _routing_sizes(desc, x, topk_idx, expert_offsets, perm, active)
    _check(lib.moe_expert_gate_up(ctypes.byref(desc), _ptr(x), _dt(x), x.shape[0], _i32(topk_idx),
                                  _i32(expert_offsets), _i32(perm), _i32(active), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_down(desc: LayerDesc, x, topk_idx, expert_offsets, perm, active, slot_out, shared_out, ws, stream=None):
    T = _routing_sizes(desc, x, topk_idx, expert_offsets, perm, active)
    _output_sizes(desc, T, slot_out, shared_out)
    _check(lib.moe_expert_down(ctypes.byref(desc), _ptr(x), _dt(x), x.shape[0], _i32(topk_idx),
                               _i32(expert_offsets), _i32(perm), _i32(active), _f32(slot_out), _f32(shared_out),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _combine_sizes(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, y):
    _need(slot_out, n_tokens * top_k * hidden, "slot_out")
    _need(topk_w, n_tokens * top_k, "topk_w")
    _need(shared_out, n_tokens * hidden, "shared_out")
    _need(y, n_tokens * hidden, "y")


def moe_combine(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, y, stream=None):
    _combine_sizes(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, y)
    _check(lib.moe_combine(_f32(slot_out), _f32(topk_w), _f32(shared_out), n_tokens, top_k, hidden, _f32(y),
                           _stream(stream)))


def moe_combine_steer(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, steer_v, steer_f, y, stream=None):
    _combine_sizes(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, y)
    _need(steer_v, hidden, "steer_v")
    _check(lib.moe_combine_steer(_f32(slot_out), _f32(topk_w), _f32(shared_out), n_tokens, top_k, hidden,
                                 _f32(steer_v), float(steer_f), _f32(y), _stream(stream)))


def moe_layer_workspace(desc: LayerDesc, n_tokens: int) -> int:
    return lib.moe_layer_workspace(ctypes.byref(desc), n_tokens)


def moe_layer(desc: LayerDesc, x, w_router, topk_idx, topk_w, expert_offsets, perm, active, slot_out, shared_out, y,
              ws, bias=None, logits=None, steer_v=None, steer_f=0.0, stream=None):
    """route -> expert FFN -> combine (+ steering when steer_v is given) in one C-ABI call."""
    T = _routing_sizes(desc, x, topk_idx, expert_offsets, perm, active)
    if w_router.dim() != 2 or tuple(w_router.shape) != (desc.n_experts, desc.hidden):
        raise ValueError(f"w_router must be [{desc.n_experts}][{desc.hidden}], got shape {tuple(w_router.shape)}")
    _output_sizes(desc, T, slot_out, shared_out)
    _need(topk_w, T * desc.top_k, "topk_w")
    _need(bias, desc.n_experts, "bias")
    _need(logits, T * desc.n_experts, "logits")
    _need(steer_v, desc.hidden, "steer_v")
    _need(y, T * desc.hidden, "y")
    _check(lib.moe_layer(ctypes.byref(desc), _ptr(x), _dt(x), T, _ptr(w_router), _dt(w_router), _f32(bias),
                         _i32(topk_idx), _f32(topk_w), _f32(logits), _i32(expert_offsets), _i32(perm), _i32(active),
                         _f32(slot_out), _f32(shared_out), _f32(steer_v), float(steer_f), _f32(y), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(stream)))


def moe_probe_stream_read(buf, nbytes, sink, n_blocks, stream=None):
    """Measurement helper: one streaming read of buf's first nbytes bytes (sink: n_blocks uint32 words)."""
    _need_bytes(buf, nbytes, "buf")
    _need_bytes(sink, 4 * n_blocks, "sink")
    _check(lib.moe_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), n_blocks, _stream(stream)))


from .layer import DeviceLayer, LayerBuffers  # noqa: E402  (needs `lib` loaded)
