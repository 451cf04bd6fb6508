"""dmoe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed, as decode and speculative verify
batches run (SGLang cookbook "Dots3-Note", Configuration Tips, CUDA graphs paragraph: decode graphs up to batch
32; Deployment, Spec Decode: 4 draft tokens per step). Every replay must equal the eager call bit for bit, also
after the inputs change in place and with eager work between replays, and the replayed output is checked against
the oracle: on the whole layer for the reduced shapes, on sampled tokens for the full verify batches of 128
tokens (32 requests x 4 tokens, hidden 5120, 256 + 1 experts) in BF16 and FP8 (GPU). The library enqueues no
allocation, free, memset or host synchronisation, so the whole layer is capturable."""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DEV, build_layer, compare_y, bf16_values, layer_inputs, near_tie_tokens, say, to_dev_bf16,
                      weights_provider, LOGIT_TOL)

pytestmark = pytest.mark.gpu

import fp8_expert_ffn_amd as dm  # noqa: E402

CASES = {
    # weight-streaming kernels (few rows per expert), router logits computed
    "verify_small_bf16": synth.LayerConfig("verify_small", T=128, H=1024, F=384, F_s=384, E=64, E_loc=64, e0=0,
                                           K=8, dtype="bf16", T_s=128, logits="router"),
    # tile kernels with the device-side schedule, FP8 quantisation of x and h
    "prefill_small_fp8": synth.LayerConfig("prefill_small", T=600, H=512, F=256, F_s=256, E=16, E_loc=16, e0=0,
                                           K=4, dtype="fp8", T_s=600, logits="router"),
    # FP8 gate/up on the wide tile kernel with h quantised in its epilogue (1024 rows per expert by the host bound)
    "wide_gateup_fp8": synth.LayerConfig("wide_gateup_fp8", T=2048, H=256, F=3200, F_s=3200, E=8, E_loc=8, e0=0,
                                         K=4, dtype="fp8", T_s=300, logits="router"),
    # the full verify batches (workloads verify_bf16 and verify_fp8)
    "verify_bf16": synth.config(8),
    "verify_fp8": synth.config(9),
}
SAMPLED = {"verify_bf16": 12, "verify_fp8": 12}


def _tokens(cfg, n):
    rng = np.random.default_rng(99)
    return np.array(sorted({0, cfg.T - 1} | set(rng.choice(cfg.T, size=n, replace=False).tolist())))


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager_and_oracle(name):
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

    # the replayed output against the oracle (the oracle computes its own logits; tokens whose top-K set differs
    # from the GPU's by a near tie are left out)
    tok = _tokens(cfg, SAMPLED[name]) if name in SAMPLED else np.arange(cfg.T)
    res = oracle.moe_forward(cfg, x_bits, weights_provider(cfg), w_r=wr, tokens=tok)
    ids = out["topk_ids"].cpu().numpy()[tok]
    L = out["logits"].cpu().numpy()[tok]
    assert float(np.max(np.abs(L.astype(np.float64) - res.logits))) <= LOGIT_TOL
    diff = near_tie_tokens(ids, res.ids, res.logits, 2 * LOGIT_TOL)
    keep = np.setdiff1d(np.arange(tok.size), diff)
    assert diff.size <= max(1, tok.size // 100)
    compare_y(bf16_values(y)[tok][keep], res.y[keep], res.y_sum[keep], f"replayed y vs oracle ({keep.size} tokens)",
              res.y_allow[keep])

    # new input values in the same buffers: the replay follows them
    rng = np.random.default_rng(11)
    x.copy_(to_dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))))
    ref2 = eager()
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref2.view(torch.int16))
    del g, layer, out, ws
    gc.collect()
    torch.cuda.empty_cache()
