"""Pins for the oracle's expert FFN and whole-layer forward: torch's textbook
SwiGLU, special cases that reduce to dense FFNs, the per-token loop form and
the parameter count the pages print (no GPU)."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dots3_moe_layer.json")


def _weights_provider(cfg):
    cache = {}

    def get(which, e):
        key = (which, e)
        if key not in cache:
            cache[key] = (synth.expert_weight_f32(cfg, which, e) if cfg.dtype == "fp8"
                          else synth.expert_weight_bf16(cfg, which, e))
        return cache[key]
    return get


def _torch_bf16(t):
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _torch_ffn(x, wg, wu, wd):
    """Textbook SwiGLU with the layer's BF16 rounding points, in torch float64."""
    h = _torch_bf16(Fn.silu(Fn.linear(x, wg)) * Fn.linear(x, wu))
    return _torch_bf16(Fn.linear(h, wd))


def test_swiglu_expert_matches_torch_textbook():
    rng = np.random.default_rng(0)
    H, F, n = 256, 96, 9  # non-square so a transposed operand cannot pass
    a = oracle.bf16_round(rng.standard_normal((n, H)))
    wg, wu = (oracle.bf16_round(rng.standard_normal((F, H)) / 16) for _ in range(2))
    wd = oracle.bf16_round(rng.standard_normal((H, F)) / 10)
    got = oracle.swiglu_expert(a, wg, wu, wd, fp8=False)
    ref = _torch_ffn(*(torch.from_numpy(v) for v in (a, wg, wu, wd))).numpy()
    # torch rounds h through float32 first; allow a rare 1-ulp difference in h
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-3
    assert np.mean(got == ref) > 0.97


def test_single_expert_layer_is_dense_ffn_plus_shared():
    """E=1, K=1: every token goes to expert 0 with weight 1; y = bf16(ffn_0(x) + ffn_shared(x))."""
    cfg = synth.LayerConfig("one_expert", T=20, H=256, F=64, F_s=64, E=1, E_loc=1, e0=0, K=1,
                            dtype="bf16", T_s=20, logits="router")
    x = synth.x_bf16(cfg)
    get = _weights_provider(cfg)
    res = oracle.moe_forward(cfg, x, get, w_r=synth.router_weight(cfg))
    np.testing.assert_array_equal(res.w, 1.0)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    W = {(w, e): torch.from_numpy(oracle.bf16_to_f64(get(w, e))) for w in ("gate", "up", "down") for e in (0, -1)}
    o = _torch_ffn(xt, W["gate", 0], W["up", 0], W["down", 0])
    s = _torch_ffn(xt, W["gate", -1], W["up", -1], W["down", -1])
    ref = _torch_bf16(o + s).numpy()
    rel = np.linalg.norm(res.y - ref) / np.linalg.norm(ref)
    assert rel < 2e-3 and np.mean(res.y == ref) > 0.95
    # the shared expert is really added: without it the output changes by ~|s|
    no_shared = oracle.moe_forward(cfg.replace(T_s=0), x, get, w_r=synth.router_weight(cfg))
    np.testing.assert_allclose(res.y - no_shared.y, s.numpy(), rtol=0, atol=0.02 * np.abs(s.numpy()).max())


def test_routed_weights_scale_expert_outputs():
    """K=2 of E=2 with given logits: y = bf16(w0 o_a + w1 o_b) with w from a two-way softmax."""
    cfg = synth.LayerConfig("two", T=6, H=128, F=32, F_s=32, E=2, E_loc=2, e0=0, K=2,
                            dtype="bf16", T_s=0, logits="uniform")
    x = synth.x_bf16(cfg)
    get = _weights_provider(cfg)
    L = np.array([[1.0, 0.0]] * 3 + [[-2.0, 0.5]] * 3, np.float32)
    res = oracle.moe_forward(cfg, x, get, logits=L)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    o = [_torch_ffn(xt, *(torch.from_numpy(oracle.bf16_to_f64(get(w, e))) for w in ("gate", "up", "down")))
         for e in (0, 1)]
    p = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1)
    ref = _torch_bf16(p[:, :1] * o[0] + p[:, 1:] * o[1]).numpy()
    assert np.linalg.norm(res.y - ref) / np.linalg.norm(ref) < 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_vectorised_equals_loop_form(dtype):
    cfg = synth.LayerConfig("tiny_loop", T=24, H=256, F=136, F_s=128, E=8, E_loc=5, e0=2, K=3,
                            dtype=dtype, T_s=10, logits="router")
    x = synth.x_bf16(cfg)
    get = _weights_provider(cfg)
    wr = synth.router_weight(cfg)
    res = oracle.moe_forward(cfg, x, get, w_r=wr)
    loop = oracle.moe_forward_loops(cfg, x, get, w_r=wr)
    np.testing.assert_array_equal(res.y, loop)
    # a sample of tokens is computed exactly as in the full layer
    sub = oracle.moe_forward(cfg, x, get, w_r=wr, tokens=np.array([0, 9, 10, 23]))
    np.testing.assert_array_equal(sub.y, res.y[[0, 9, 10, 23]])


def test_tiny_workload_loop_form():
    cfg = synth.config(0)
    x = synth.x_bf16(cfg)
    get = _weights_provider(cfg)
    wr = synth.router_weight(cfg)
    res = oracle.moe_forward(cfg, x, get, w_r=wr)
    np.testing.assert_array_equal(res.y, oracle.moe_forward_loops(cfg, x, get, w_r=wr))
    assert np.all(np.isfinite(res.y)) and res.y.std() > 0.05


def test_fp8_layer_close_to_unquantised_layer():
    """FP8 quantisation error is a few percent per element, not a structural change."""
    cfg = synth.LayerConfig("q", T=32, H=512, F=256, F_s=256, E=4, E_loc=4, e0=0, K=2,
                            dtype="fp8", T_s=32, logits="router")
    x = synth.x_bf16(cfg)
    get = _weights_provider(cfg)
    wr = synth.router_weight(cfg)
    q = oracle.moe_forward(cfg, x, get, w_r=wr)
    bf = oracle.moe_forward(cfg.replace(dtype="bf16"), x,
                            lambda w, e: synth.f32_to_bf16_bits(get(w, e)), w_r=wr)
    rel = np.linalg.norm(q.y - bf.y) / np.linalg.norm(bf.y)
    assert 0.005 < rel < 0.08


def test_parameter_count_closed_form_from_pages():
    """45 MoE layers x 256 experts x 3 SwiGLU matrices of H x F: ~272B of the 280B total,
    and 45 x (8 routed + 1 shared) x 3 H F of the 16B activated. A two-matrix FFN would
    give only 181B, so the expert has three projections."""
    g = {k: v["value"] for k, v in json.load(open(GOLDEN)).items() if not k.startswith("_")}
    H, F, E, L = g["hidden_size"], g["moe_intermediate_size"], g["n_routed_experts"], g["moe_layers"]
    cfg = synth.LayerConfig("page", T=1, H=H, F=F, F_s=g["shared_experts_intermediate_size"], E=E,
                            E_loc=E, e0=0, K=g["num_experts_per_tok"], dtype="bf16", T_s=1, logits="router")
    names = {"gate_proj": "gate", "up_proj": "up", "down_proj": "down"}
    per_expert = sum(int(np.prod(synth.weight_shape(cfg, names[p], 0))) for p in g["mlp_projections"])
    routed = L * E * per_expert
    active = L * (cfg.K + g["n_shared_experts"]) * per_expert
    assert per_expert == 3 * H * F
    assert g["total_parameters"] > routed > 0.9 * g["total_parameters"]
    assert active < g["activated_parameters"] and active > 0.5 * g["activated_parameters"]
    assert L * E * 2 * H * F < 0.7 * g["total_parameters"]


def test_combine_hand_example():
    """Two tokens, two slots, H = 2: token 0 mixes rows 0 and 2 with weights 1/4 and 3/4 and adds the shared
    row (T_s = 1); token 1's second slot is on another GPU (-1) and it gets no shared row. The float64 sum
    1.75390625 lies halfway between the bfloat16 values 1.75 and 1.7578125 and rounds to the even 1.75."""
    o = np.array([[1.0, 3.0], [0.5, -1.0], [2.0, 2.0]])
    token_row = np.array([[0, 2], [1, -1]], np.int32)
    w = np.array([[0.25, 0.75], [1.0, 0.5]], np.float32)
    s = np.array([[1.0 / 256, 0.0], [7.0, 7.0]])
    y_sum = oracle.combine(o, token_row, w, s, 1, rounded=False)
    np.testing.assert_array_equal(y_sum, [[1.75390625, 2.25], [0.5, -1.0]])
    np.testing.assert_array_equal(oracle.combine(o, token_row, w, s, 1), [[1.75, 2.25], [0.5, -1.0]])
