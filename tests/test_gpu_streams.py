"""Reentrancy: layer calls enqueued on several streams at once, each with its
own weights, inputs, outputs and workspace, give the same bits as the same
calls run one after another on one stream (GPU)."""
import pytest
import torch

import synth
from gpu_util import DEV, build_layer, layer_inputs, say, to_dev_bf16

pytestmark = pytest.mark.gpu

CFGS = [
    # FP8 on the two-workgroup tile kernel, router logits computed on the GPU
    synth.LayerConfig("streams_fp8", T=300, H=1024, F=384, F_s=384, E=16, E_loc=16, e0=0, K=8, dtype="fp8",
                      T_s=300, logits="router"),
    # BF16 on the weight-streaming kernel
    synth.LayerConfig("streams_bf16", T=64, H=1024, F=384, F_s=384, E=64, E_loc=64, e0=0, K=8, dtype="bf16",
                      T_s=64, logits="router"),
    # FP8 EP share with given logits and a separate shared expert width
    synth.LayerConfig("streams_ep_fp8", T=600, H=512, F=256, F_s=128, E=64, E_loc=8, e0=8, K=8, dtype="fp8",
                      T_s=200, logits="zipf"),
]


def _call(layer, cfg, x, wr, given):
    if given is not None:
        return layer.forward(x, cfg.T_s, logits=given)["y"]
    return layer.forward(x, cfg.T_s, w_router=wr)["y"]


def test_concurrent_streams_match_sequential():
    runs = []
    for cfg in CFGS:
        x_bits, wr, given = layer_inputs(cfg)
        runs.append((build_layer(cfg), cfg, to_dev_bf16(x_bits),
                     torch.from_numpy(wr).to(DEV) if wr is not None else None,
                     torch.from_numpy(given).to(DEV) if given is not None else None))
    ref = [_call(*r).clone() for r in runs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        outs = []
        for r, s in zip(runs, streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs.append(_call(*r))
        torch.cuda.synchronize()
        for (layer, cfg, *_), y, y0 in zip(runs, outs, ref):
            same = torch.equal(y.view(torch.int16), y0.view(torch.int16))
            say(f"[{cfg.name}] replay {rep}: {'identical' if same else 'DIFFERS'}")
            assert same, f"{cfg.name}: concurrent result differs from the sequential one"
