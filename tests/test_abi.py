"""Host-only checks of the C-ABI library (no GPU needed): it loads, exports
every function include/moe2bit.h declares, reports its ABI version, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_quantized_moe_permute_amd", "libmoe2bit.so")
HDR = os.path.join(ROOT, "include", "moe2bit.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe2bit.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    return L


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe2bit.h but not exported"


def test_binding_lists_the_same_symbols():
    src = open(os.path.join(ROOT, "bit_quantized_moe_permute_amd", "__init__.py")).read()
    exported = re.search(r"EXPORTS = \[(.*?)\]", src, re.S).group(1)
    assert sorted(re.findall(r'"(moe_\w+)"', exported)) == declared_functions()


def test_binding_rejects_host_tensors():
    """The binding takes device tensors only; a host tensor fails before any library call."""
    torch = pytest.importorskip("torch")
    import bit_quantized_moe_permute_amd as m
    t = torch.zeros(8, 64)
    with pytest.raises(TypeError):
        m.moe_combine(t, torch.ones(1, 8), None, 1, 8, 64, torch.empty(1, 64))


def test_abi_version(lib):
    lib.moe_abi_version.restype = ctypes.c_int
    hdr = open(HDR).read()
    assert lib.moe_abi_version() == int(re.search(r"#define MOE_ABI_VERSION (\d+)", hdr).group(1))


def test_weight_bytes(lib):
    f = lib.moe_weight_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    assert f(1, 256, 2048, 4096) == 256 * 2048 * 16 * 66
    assert f(2, 256, 4096, 2048) == 256 * 4096 * 8 * 84
    assert f(3, 2, 256, 256) == 2 * 256 * 144
    assert f(2, 8, 256, 128) == 8 * 128 * 84          # blocks span two rows
    assert f(9, 1, 256, 256) == 0 and f(1, 1, 3, 5) == 0


def _err(lib):
    lib.moe_last_error.restype = ctypes.c_char_p
    return lib.moe_last_error().decode()


def test_route_rejects_bad_arguments(lib):
    f = lib.moe_route
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    p = vp(0x1000)
    ws = 1 << 20
    # null x
    assert f(None, 1, 4, 4096, p, 1, 256, None, 8, p, p, None, p, p, p, p, ws, None) == 1
    assert "null" in _err(lib)
    # top_k > E
    assert f(p, 1, 4, 4096, p, 1, 8, None, 9, p, p, None, p, p, p, p, ws, None) == 1
    # E > 256
    assert f(p, 1, 4, 4096, p, 1, 300, None, 8, p, p, None, p, p, p, p, ws, None) == 1
    # hidden not a multiple of 64
    assert f(p, 1, 4, 100, p, 1, 8, None, 2, p, p, None, p, p, p, p, ws, None) == 1
    # workspace too small
    assert f(p, 1, 4, 4096, p, 1, 256, None, 8, p, p, None, p, p, p, p, 16, None) == 1
    assert "workspace" in _err(lib)
    # unknown dtype
    assert f(p, 7, 4, 4096, p, 1, 256, None, 8, p, p, None, p, p, p, p, ws, None) == 1


def test_expert_ffn_rejects_bad_layers(lib):
    import bit_quantized_moe_permute_amd as m  # noqa: F401  (loads; host only)
    from bit_quantized_moe_permute_amd import LayerDesc
    f = lib.moe_expert_ffn
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    p = vp(0x1000)
    d = LayerDesc(hidden=4096, inter=2048, n_experts=256, top_k=8, gate_up_fmt=1, down_fmt=2, gate=0x1000, up=0x1000,
                  down=0x1000, codebook=0x1000, shared_inter=0, path=0)
    # x dtype unknown
    assert f(ctypes.byref(d), p, 5, 1, p, p, p, p, p, None, p, 1 << 30, None) == 1
    # shared_out given without a shared expert
    assert f(ctypes.byref(d), p, 1, 1, p, p, p, p, p, p, p, 1 << 30, None) == 1
    # bad format
    d.gate_up_fmt = 2
    assert f(ctypes.byref(d), p, 1, 1, p, p, p, p, p, None, p, 1 << 30, None) == 1
    assert "format" in _err(lib)
    d.gate_up_fmt = 1
    # misaligned weights
    d.gate = 0x1004
    assert f(ctypes.byref(d), p, 1, 1, p, p, p, p, p, None, p, 1 << 30, None) == 1
    d.gate = 0x1000
    # top_k > E
    d.top_k = 300
    assert f(ctypes.byref(d), p, 1, 1, p, p, p, p, p, None, p, 1 << 30, None) == 1
    d.top_k = 8
    # workspace too small
    assert f(ctypes.byref(d), p, 1, 1, p, p, p, p, p, None, p, 8, None) == 1
    assert "workspace" in _err(lib)
    # fp32 activations cannot take the decode path when it is forced
    d.path = 2
    assert f(ctypes.byref(d), p, 0, 1, p, p, p, p, p, None, p, 1 << 30, None) == 2


def test_prepare_and_combine_reject_bad_arguments(lib):
    vp = ctypes.c_void_p
    f = lib.moe_prepare_weights
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
    assert f(1, 1, 256, 100, vp(0x1000), vp(0x100000), None) == 1      # cols % 32
    assert f(1, 1, 256, 256, vp(0x1000), vp(0x1008), None) == 1         # overlap / misaligned
    assert f(5, 1, 256, 256, vp(0x1000), vp(0x100000), None) == 1       # format
    g = lib.moe_combine
    g.restype = ctypes.c_int
    g.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    assert g(None, vp(0x1000), None, 1, 8, 4096, vp(0x1000), None) == 1
    assert g(vp(0x1000), vp(0x1000), None, 0, 8, 4096, vp(0x1000), None) == 1
    assert g(vp(0x1000), vp(0x1000), vp(0x1002), 1, 8, 4096, vp(0x1000), None) == 1   # misaligned shared output
    assert "misaligned" in _err(lib)
    h = lib.moe_combine_steer
    h.restype = ctypes.c_int
    h.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_float, vp, vp]
    p = vp(0x1000)
    assert h(p, p, None, 1, 8, 4096, None, 1.0, p, None) == 1                  # no direction
    assert "null" in _err(lib)
    assert h(p, p, None, 1, 0, 4096, p, 1.0, p, None) == 1                     # top_k
    assert h(p, p, None, 1, 8, 4096, vp(0x1002), 1.0, p, None) == 1           # misaligned direction
    assert h(p, p, vp(0x1001), 1, 8, 4096, p, 1.0, p, None) == 1              # misaligned shared output
    assert h(p, p, None, 1, 8, 4096, p, float("nan"), p, None) == 1           # strength not finite
    assert "finite" in _err(lib)
    assert h(p, p, None, 1, 8, 4096, p, float("inf"), p, None) == 1


def test_plain_c_consumer(tmp_path):
    """tests/abi_consumer.c: a C program that includes moe2bit.h and links the library (gcc, no GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "abi_consumer"
    libdir = os.path.dirname(LIB)
    cmd = [gcc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_consumer.c"), "-L", libdir, "-lmoe2bit", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr


def test_binding_rejects_undersized_tensors():
    """The binding checks every tensor's size against T, k, E and H on the host before a pointer reaches the
    library (an undersized output would be written out of bounds); host tensors are enough to see the check."""
    torch = pytest.importorskip("torch")
    import bit_quantized_moe_permute_amd as m
    from bit_quantized_moe_permute_amd import LayerDesc
    i32 = dict(dtype=torch.int32)
    T, H, E, k = 3, 256, 8, 2
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    w = torch.zeros(E, H, dtype=torch.bfloat16)
    ws = torch.zeros(4096, dtype=torch.uint8)
    good = dict(topk_idx=torch.zeros(T * k, **i32), topk_w=torch.zeros(T * k), expert_offsets=torch.zeros(E + 1, **i32),
                perm=torch.zeros(T * k, **i32), active=torch.zeros(E + 1, **i32))
    for name, short in (("topk_idx", torch.zeros(T * k - 1, **i32)), ("topk_w", torch.zeros(1)),
                        ("expert_offsets", torch.zeros(E, **i32)), ("perm", torch.zeros(T, **i32)),
                        ("active", torch.zeros(E, **i32))):
        args = dict(good, **{name: short})
        with pytest.raises(ValueError, match=name):
            m.moe_route(x, w, E, k, args["topk_idx"], args["topk_w"], args["expert_offsets"], args["perm"],
                        args["active"], ws)
    with pytest.raises(ValueError, match="w_router"):
        m.moe_route(x, torch.zeros(E, H + 64, dtype=torch.bfloat16), E, k, *good.values(), ws)
    with pytest.raises(ValueError, match="tokens"):
        m.moe_route(x.reshape(-1), w, E, k, *good.values(), ws)
    with pytest.raises(ValueError, match="logits"):
        m.moe_route(x, w, E, k, *good.values(), ws, logits=torch.zeros(T, E - 1))
    d = LayerDesc(hidden=H, inter=128, n_experts=E, top_k=k, shared_inter=128)
    slot = torch.zeros(T * k, H)
    shared = torch.zeros(T, H)
    routing = (good["topk_idx"], good["expert_offsets"], good["perm"], good["active"])
    with pytest.raises(ValueError, match="slot_out"):
        m.moe_expert_ffn(d, x, *routing, slot[:-1], shared, ws)
    with pytest.raises(ValueError, match="shared_out"):
        m.moe_expert_ffn(d, x, *routing, slot, shared[:-1], ws)
    with pytest.raises(ValueError, match="hidden"):
        m.moe_expert_ffn(d, torch.zeros(T, H + 8, dtype=torch.bfloat16), *routing, slot, shared, ws)
    with pytest.raises(ValueError, match="perm"):
        m.moe_expert_gate_up(d, x, good["topk_idx"], good["expert_offsets"], good["perm"][:-1], good["active"], ws)
    with pytest.raises(ValueError, match="y"):
        m.moe_combine(slot, good["topk_w"], shared, T, k, H, torch.zeros(T, H - 1))
    with pytest.raises(ValueError, match="steer_v"):
        m.moe_combine_steer(slot, good["topk_w"], shared, T, k, H, torch.zeros(H - 1), 1.0, torch.zeros(T, H))
    with pytest.raises(ValueError, match="out"):
        m.moe_dequantize(2, torch.zeros(84 * 4, dtype=torch.uint8), 1, 4, 256, 0, 1, None, torch.zeros(1023))
    with pytest.raises(ValueError, match="prepared"):
        m.moe_prepare_weights(2, 1, 4, 256, torch.zeros(84 * 4, dtype=torch.uint8),
                              torch.zeros(84 * 4 - 1, dtype=torch.uint8))
