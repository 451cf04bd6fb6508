"""dmoe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay must equal the eager
call bit for bit, also after the inputs change in place and with eager work between replays (GPU). The library
enqueues no allocation, free, memset or host synchronisation, so the whole layer is capturable."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, build_layer, layer_inputs, say, to_dev_bf16

pytestmark = pytest.mark.gpu

import fp8_expert_ffn_amd as dm  # noqa: E402

CASES = {
    # weight-streaming kernels (few rows per expert), router logits computed
    "verify_small_bf16": synth.LayerConfig("verify_small", T=128, H=1024, F=384, F_s=384, E=64, E_loc=64, e0=0,
                                           K=8, dtype="bf16", T_s=128, logits="router"),
    # tile kernels with the device-side schedule, FP8 quantisation of x and h
    "prefill_small_fp8": synth.LayerConfig("prefill_small", T=600, H=512, F=256, F_s=256, E=16, E_loc=16, e0=0,
                                           K=4, dtype="fp8", T_s=600, logits="router"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    cfg = CASES[name]
    say(f"[graph {name}] {cfg}")
    layer = build_layer(cfg)
    x_bits, wr, _ = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    wdev = torch.from_numpy(wr).to(DEV)
    d, p, ws, out = layer.make_call(x, cfg.T_s, w_router=wdev)
    y = out["y"]
    stream = torch.cuda.current_stream()

    def eager():
        dm.dmoe_forward(d, p, ws)
        torch.cuda.synchronize()
        return y.clone()

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dm.dmoe_forward(d, p, ws)
    stream.wait_stream(side)
    scratch = torch.zeros(1 << 20, device=DEV)
    for r in range(3):
        y.zero_()
        g.replay()
        scratch.add_(1.0)            # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs from eager"
    # new input values in the same buffers: the replay follows them
    rng = np.random.default_rng(11)
    x.copy_(to_dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))))
    ref2 = eager()
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref2.view(torch.int16))
