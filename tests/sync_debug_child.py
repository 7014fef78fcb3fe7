"""Child process of test_sync_debug.py, started with MOE_SYNC_DEBUG=1.

Runs the 1024-hidden, 32-expert test layer through moe_layer at 1 and 70 tokens
and through the three separate calls, checks after every call that the
stream is already idle (the library waited for it), captures the one-token call
in a HIP graph (the wait is skipped while capturing) and replays it, then
writes every layer output to the .npz file named by argv[1].
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main(out_path: str) -> int:
    import bit_quantized_moe_permute_amd as m
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward, forward_layer
    assert m.moe_sync_debug(), "MOE_SYNC_DEBUG was not seen by the library"
    sp = synth.SPECS["mid"]
    L = synth.make_layer(sp, quantizer=oracle.quantize)
    DL = DeviceLayer.from_synth(L)
    out = {}
    for T in (1, 70):
        x = synth.activations("mid", T, sp.hidden, sp.x_bf16, seed=2100 + T)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        torch.cuda.synchronize()
        for name, fn in (("layer", forward_layer), ("three", forward)):
            b = LayerBuffers.allocate(DL, T)
            torch.cuda.synchronize()
            fn(DL, xd, b)
            assert torch.cuda.current_stream().query(), f"{name} T={T}: stream still busy after the call"
            out[f"{name}_T{T}"] = b.y.cpu().numpy()
            print(f"[sync-debug child] {name} T={T} done", flush=True)
    # one-token call captured into a graph: no wait inside the capture
    x = synth.activations("mid", 1, sp.hidden, sp.x_bf16, seed=2101)
    xin = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    bg = LayerBuffers.allocate(DL, 1)
    forward_layer(DL, xin, bg)
    torch.cuda.synchronize()
    bg.y.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            forward_layer(DL, xin, bg)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out["graph_T1"] = bg.y.cpu().numpy()
    print("[sync-debug child] graph replay done", flush=True)
    np.savez(out_path, **out)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
