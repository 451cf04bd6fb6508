"""dmoe_forward_noalloc (the library's fixed device workspace) against dmoe_forward (a caller workspace): two
calls in a row on the same GPU, the second with fewer tokens, must give the same routing and bit-identical
outputs; a layer whose workspace exceeds the fixed array is refused before anything is enqueued (GPU)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, build_layer, layer_inputs, say, to_dev_bf16

pytestmark = pytest.mark.gpu

import fp8_expert_ffn_amd as dm  # noqa: E402
from fp8_expert_ffn_amd import _lib as L  # noqa: E402

CFG = {
    "bf16": synth.LayerConfig("noalloc_bf16", T=160, H=1024, F=384, F_s=384, E=32, E_loc=32, e0=0, K=8,
                              dtype="bf16", T_s=160, logits="router"),
    "fp8": synth.LayerConfig("noalloc_fp8", T=600, H=512, F=200, F_s=200, E=16, E_loc=16, e0=0, K=4,
                             dtype="fp8", T_s=600, logits="router"),
}


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_forward_two_calls(dtype):
    cfg = CFG[dtype]
    layer = build_layer(cfg)
    x_bits, wr, _ = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    wdev = torch.from_numpy(wr).to(DEV)
    # first call: all tokens (tile GEMMs); second call: the first 20 tokens (weight-streaming GEMMs)
    for T in (cfg.T, 20):
        say(f"[noalloc {dtype}] T={T}")
        xs = x[:T].contiguous()
        d, p, ws, ref = layer.make_call(xs, min(cfg.T_s, T), w_router=wdev)
        assert L.dmoe_forward_ws_bytes(d) <= L.DMOE_NOALLOC_WS_BYTES
        dm.dmoe_forward(d, p, ws)
        d2, p2, _, got = layer.make_call(xs, min(cfg.T_s, T), w_router=wdev)
        got["y"].fill_(float("nan"))
        L.dmoe_forward_noalloc(d2, p2)
        torch.cuda.synchronize()
        for k in ("logits", "topk_ids", "topk_w", "y"):
            assert _same(got[k], ref[k]), f"T={T}: {k} differs from dmoe_forward"
        assert torch.isfinite(got["y"].float()).all()


def test_noalloc_refuses_a_layer_above_its_array():
    cfg = synth.config(2)  # 8192 tokens: about 1.1 GB of workspace
    d = L.LayerDesc(cfg.T, cfg.H, cfg.F, cfg.F_s, cfg.E, cfg.E_loc, cfg.e0, cfg.K, cfg.T_s, L.DMOE_FP8_E4M3, 0,
                    1, 0, 0, 0.0, 0)
    assert L.dmoe_forward_ws_bytes(d) > L.DMOE_NOALLOC_WS_BYTES
    with pytest.raises(L.DmoeError) as ei:
        L.dmoe_forward_noalloc(d, L.LayerPtrs())
    assert ei.value.status == L.DMOE_ERR_WORKSPACE
    assert "fixed device array" in str(ei.value)
