"""Seeded shape sweep: dmoe_forward against the oracle on 24 drawn layers
(hidden and FFN widths, expert counts, local ranges, shared-token counts,
logit sources and routing options drawn per case; see sweep_cases.py), each
through the exact given-logits check and, for router workloads, the GPU's
own router logits (GPU)."""
import pytest

import oracle
from gpu_util import build_layer, check_forward, layer_inputs, say, score_bias_of, to_dev_bf16, weights_provider
from sweep_cases import sweep_cases

pytestmark = pytest.mark.gpu

CASES = {c.name: c for c in sweep_cases()}


@pytest.mark.parametrize("name", list(CASES))
def test_sweep_forward_matches_oracle(name):
    cfg = CASES[name]
    say(f"[{name}] {cfg}")
    x_bits, wr, given = layer_inputs(cfg)
    ref = oracle.moe_forward(cfg, x_bits, weights_provider(cfg), w_r=wr, logits=given, score_bias=score_bias_of(cfg))
    layer = build_layer(cfg)
    check_forward(cfg, layer, to_dev_bf16(x_bits), wr, given, ref)
