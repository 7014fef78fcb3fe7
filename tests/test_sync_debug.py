"""MOE_SYNC_DEBUG: with the switch on, every entry point waits for its stream
before returning (except under graph capture) and the results do not change.

The switch is read once per process, so the switched-on calls run in a child
process (tests/sync_debug_child.py); this process computes the same outputs
with the switch off and compares them bit for bit.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_sync_debug_waits_and_changes_no_result(tmp_path):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import bit_quantized_moe_permute_amd as m
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward, forward_layer
    out = tmp_path / "sync_debug.npz"
    env = dict(os.environ, MOE_SYNC_DEBUG="1")
    print("[sync-debug] starting the child process", flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(HERE, "sync_debug_child.py"), str(out)], env=env,
                       capture_output=True, text=True, timeout=240)
    print(p.stdout[-2000:], flush=True)
    assert p.returncode == 0, p.stderr[-4000:]
    got = np.load(out)
    if os.environ.get("MOE_SYNC_DEBUG", "") in ("", "0"):
        assert not m.moe_sync_debug()
    sp = synth.SPECS["mid"]
    L = synth.make_layer(sp, quantizer=oracle.quantize)
    DL = DeviceLayer.from_synth(L)
    for T in (1, 70):
        x = synth.activations("mid", T, sp.hidden, sp.x_bf16, seed=2100 + T)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        for name, fn in (("layer", forward_layer), ("three", forward)):
            b = LayerBuffers.allocate(DL, T)
            fn(DL, xd, b)
            torch.cuda.synchronize()
            assert np.array_equal(got[f"{name}_T{T}"], b.y.cpu().numpy()), f"{name} T={T}"
    assert np.array_equal(got["graph_T1"], _layer_y(DL, sp, 2101, forward_layer)), "graph replay"


def _layer_y(DL, sp, seed, fn):
    from bit_quantized_moe_permute_amd.layer import LayerBuffers
    x = synth.activations("mid", 1, sp.hidden, sp.x_bf16, seed=seed)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    b = LayerBuffers.allocate(DL, 1)
    fn(DL, xd, b)
    torch.cuda.synchronize()
    return b.y.cpu().numpy()
