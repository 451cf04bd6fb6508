"""End-to-end parity of dmoe_forward against the CPU oracle on workloads the
oracle finishes in seconds: the tiny layer at full size, and reduced versions
of the decode, prefill, EP-share and non-divisible layers that still span
several tiles with ragged tails (GPU)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DEV, W_TOL, bf16_values, build_layer, check_forward, check_given_logits_path, compare_y,
                      layer_inputs, say, score_bias_of, to_dev_bf16, weights_provider)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": synth.config(0),
    "decode_small": synth.LayerConfig("decode_small", T=64, H=1024, F=384, F_s=384, E=64, E_loc=64, e0=0, K=8,
                                      dtype="bf16", T_s=64, logits="router"),
    "prefill_small_fp8": synth.LayerConfig("prefill_small", T=300, H=1024, F=384, F_s=384, E=16, E_loc=16, e0=0,
                                           K=4, dtype="fp8", T_s=300, logits="router"),
    "ep_share_small_fp8": synth.LayerConfig("ep_small", T=600, H=512, F=256, F_s=256, E=64, E_loc=8, e0=0, K=8,
                                            dtype="fp8", T_s=75, logits="zipf"),
    "ep_share_mid_fp8": synth.LayerConfig("ep_mid", T=600, H=512, F=256, F_s=256, E=64, E_loc=8, e0=24, K=8,
                                          dtype="fp8", T_s=75, logits="zipf"),
    "nondiv_small_fp8": synth.LayerConfig("nondiv_small", T=128, H=1024, F=1400, F_s=1400, E=16, E_loc=16, e0=0,
                                          K=4, dtype="fp8", T_s=128, logits="uniform"),
    "nondiv_small_bf16": synth.LayerConfig("nondiv_bf16", T=90, H=640, F=200, F_s=136, E=12, E_loc=12, e0=0, K=3,
                                           dtype="bf16", T_s=50, logits="uniform"),
    "single_token_fp8": synth.LayerConfig("one_tok", T=1, H=512, F=128, F_s=128, E=16, E_loc=16, e0=0, K=4,
                                          dtype="fp8", T_s=1, logits="router"),
    # group-limited routing without renormalisation, scaled weights
    "grouped_fp8": synth.LayerConfig("grouped", T=300, H=512, F=256, F_s=256, E=64, E_loc=64, e0=0, K=8,
                                     dtype="fp8", T_s=300, logits="router", n_group=8, topk_group=3,
                                     renormalize=False, scaling=2.5),
    # sigmoid scoring with a per-expert selection bias, grouped by two-best sums, renormalised
    "sigmoid_bias_bf16": synth.LayerConfig("sigmoid", T=200, H=512, F=256, F_s=256, E=64, E_loc=64, e0=0, K=6,
                                           dtype="bf16", T_s=200, logits="router", n_group=8, topk_group=4,
                                           scoring="sigmoid", scaling=1.5),
    # vision-tower MoE shape (hidden 1536, FFN 2112 = 16.5 blocks, 64 experts, no shared expert)
    "vision_small_bf16": synth.LayerConfig("vision_small", T=256, H=1536, F=2112, F_s=0, E=64, E_loc=64, e0=0,
                                           K=8, dtype="bf16", T_s=0, logits="router"),
    "vision_small_fp8": synth.LayerConfig("vision_small_fp8", T=256, H=1536, F=2112, F_s=0, E=64, E_loc=64, e0=0,
                                          K=8, dtype="fp8", T_s=0, logits="router"),
    # dense FFN as one expert with top-1 (routing weight exactly 1)
    "dense_small_fp8": synth.LayerConfig("dense_small", T=192, H=1024, F=13824, F_s=0, E=1, E_loc=1, e0=0, K=1,
                                         dtype="fp8", T_s=0, logits="single"),
    "dense_small_bf16": synth.LayerConfig("dense_small_bf16", T=100, H=512, F=2304, F_s=0, E=1, E_loc=1, e0=0,
                                          K=1, dtype="bf16", T_s=0, logits="single"),
    # shortest reductions on the tile GEMM (about 128 rows per expert): one or two 128-byte K stages,
    # i.e. the pipeline's prologue and drain without a steady state
    "min_k_fp8": synth.LayerConfig("min_k_fp8", T=256, H=128, F=128, F_s=128, E=4, E_loc=4, e0=0, K=2,
                                   dtype="fp8", T_s=256, logits="router"),
    "min_k_bf16": synth.LayerConfig("min_k_bf16", T=256, H=128, F=120, F_s=64, E=4, E_loc=4, e0=0, K=2,
                                    dtype="bf16", T_s=256, logits="router"),
    "short_k_fp8": synth.LayerConfig("short_k_fp8", T=300, H=256, F=200, F_s=200, E=5, E_loc=5, e0=0, K=2,
                                     dtype="fp8", T_s=100, logits="uniform"),
    # 33..64 rows per expert on average (the tile GEMM with one short tile per expert)
    "mid_rows_bf16": synth.LayerConfig("mid_rows_bf16", T=256, H=512, F=256, F_s=256, E=32, E_loc=32, e0=0, K=6,
                                       dtype="bf16", T_s=200, logits="router"),
    "mid_rows_nondiv_fp8": synth.LayerConfig("mid_rows_fp8", T=512, H=1024, F=1400, F_s=1400, E=64, E_loc=64, e0=0,
                                             K=8, dtype="fp8", T_s=512, logits="uniform"),
    # few tokens with H % 1024 == 0: the router leaves four partial planes over K that the route kernel adds;
    # ragged token and expert tiles, grouped selection without renormalisation (sum over all experts' logits),
    # sigmoid scoring with a selection bias (one K-step per wave), and the largest T of that path
    "planes_ragged_bf16": synth.LayerConfig("planes_ragged", T=50, H=1024, F=128, F_s=128, E=40, E_loc=40, e0=0,
                                            K=4, dtype="bf16", T_s=50, logits="router"),
    "planes_grouped_fp8": synth.LayerConfig("planes_grouped", T=200, H=1024, F=256, F_s=256, E=64, E_loc=64, e0=0,
                                            K=8, dtype="fp8", T_s=200, logits="router", n_group=8, topk_group=3,
                                            renormalize=False, scaling=2.5),
    "planes_sigmoid_bf16": synth.LayerConfig("planes_sigmoid", T=96, H=2048, F=256, F_s=256, E=64, E_loc=64, e0=0,
                                             K=6, dtype="bf16", T_s=96, logits="router", n_group=8, topk_group=4,
                                             scoring="sigmoid", scaling=1.5),
    "planes_t256_bf16": synth.LayerConfig("planes_t256", T=256, H=1024, F=128, F_s=0, E=32, E_loc=32, e0=0, K=4,
                                          dtype="bf16", T_s=0, logits="router"),
    # few rows in all (the weight-streaming GEMMs): one token with 8 experts and the shared expert, three tokens
    # on a non-divisible FFN, 17-32 rows per expert (two 16-row subtiles per pass), an EP share of 32 experts
    # (e0 = 32) with untouched experts
    "small_t1_bf16": synth.LayerConfig("small_t1", T=1, H=2048, F=512, F_s=512, E=64, E_loc=64, e0=0, K=8,
                                       dtype="bf16", T_s=1, logits="router"),
    "small_t3_nondiv_fp8": synth.LayerConfig("small_t3", T=3, H=1024, F=1400, F_s=1400, E=32, E_loc=32, e0=0,
                                             K=4, dtype="fp8", T_s=3, logits="router"),
    "stream_r2_fp8": synth.LayerConfig("stream_r2", T=40, H=512, F=256, F_s=256, E=16, E_loc=16, e0=0, K=8,
                                       dtype="fp8", T_s=40, logits="uniform"),
    "small_ep_bf16": synth.LayerConfig("small_ep", T=16, H=1024, F=256, F_s=256, E=256, E_loc=32, e0=32, K=8,
                                       dtype="bf16", T_s=16, logits="zipf"),
    # several 128-row tiles per expert on the two-workgroup tile GEMM (about 500 rows per expert, too few work
    # items for the wide kernel: full tiles and a ragged one), and one expert of 257 or 513 rows (a last tile
    # of one row)
    "many_tiles_fp8": synth.LayerConfig("many_tiles_fp8", T=2000, H=512, F=384, F_s=384, E=8, E_loc=8, e0=0, K=2,
                                        dtype="fp8", T_s=700, logits="router"),
    "many_tiles_bf16": synth.LayerConfig("many_tiles_bf16", T=1500, H=768, F=256, F_s=256, E=6, E_loc=6, e0=0,
                                         K=2, dtype="bf16", T_s=1500, logits="uniform"),
    # the down projection on the wide tile GEMM (at least 128 rows per expert by the host bound and at least
    # 1024 work items: (20 + 40 + 3) 256-row tiles x 20 column blocks): experts of about 128 rows in one partly
    # filled tile each, and the shared rows as an extra group in tiles of 256, 256 and 128 (FP8) or 244 (BF16)
    "wide_down_fp8": synth.LayerConfig("wide_down_fp8", T=640, H=5120, F=256, F_s=256, E=40, E_loc=40, e0=0, K=8,
                                       dtype="fp8", T_s=640, logits="uniform"),
    "wide_down_bf16": synth.LayerConfig("wide_down_bf16", T=640, H=5120, F=384, F_s=384, E=40, E_loc=40, e0=0,
                                        K=8, dtype="bf16", T_s=500, logits="router"),
    # BF16 gate/up on the wide tile GEMM (1024 rows per expert by the host bound, 42 tiles x 25 column blocks),
    # with Zipf-skewed experts of a few to thousands of rows
    "wide_gateup_bf16": synth.LayerConfig("wide_gateup_bf16", T=4096, H=256, F=3200, F_s=3200, E=8, E_loc=8, e0=0,
                                          K=2, dtype="bf16", T_s=300, logits="zipf"),
    # FP8 gate/up on the wide tile GEMM with h quantised in its epilogue (at least 1024 rows per expert by the
    # host bound and 1024 work items): uniform routing with a ragged shared-expert tail, and a Zipf-skewed EP
    # share whose experts range from a few to thousands of rows
    "wide_gateup_fp8": synth.LayerConfig("wide_gateup_fp8", T=4096, H=256, F=3200, F_s=3200, E=8, E_loc=8, e0=0,
                                         K=2, dtype="fp8", T_s=300, logits="uniform"),
    "wide_gateup_ep_fp8": synth.LayerConfig("wide_gateup_ep", T=2048, H=256, F=1920, F_s=1920, E=64, E_loc=8,
                                            e0=0, K=8, dtype="fp8", T_s=200, logits="zipf"),
    # the same path with F = 24 x 128 + 56: a partial last h slice quantised in the epilogue
    "wide_gateup_nondiv_fp8": synth.LayerConfig("wide_gateup_nondiv", T=4096, H=256, F=3128, F_s=3128, E=8,
                                                E_loc=8, e0=0, K=2, dtype="fp8", T_s=300, logits="uniform"),
    # limits of the descriptor: 1024 experts with top-64 (weight streaming, 4 rows per expert), every expert
    # selected (K = E), and the FP8 limits H = 16384 or F = 16384 (128 scale slices along K) on the streaming
    # and the tile kernels
    "max_experts_fp8": synth.LayerConfig("max_experts_fp8", T=64, H=128, F=64, F_s=64, E=1024, E_loc=1024, e0=0,
                                         K=64, dtype="fp8", T_s=64, logits="uniform"),
    "all_experts_bf16": synth.LayerConfig("all_experts_bf16", T=40, H=256, F=136, F_s=136, E=8, E_loc=8, e0=0, K=8,
                                          dtype="bf16", T_s=40, logits="router"),
    "max_hidden_stream_fp8": synth.LayerConfig("max_hidden_stream_fp8", T=24, H=16384, F=128, F_s=128, E=4,
                                               E_loc=4, e0=0, K=2, dtype="fp8", T_s=24, logits="uniform"),
    "max_hidden_tile_fp8": synth.LayerConfig("max_hidden_tile_fp8", T=200, H=16384, F=128, F_s=128, E=4, E_loc=4,
                                             e0=0, K=2, dtype="fp8", T_s=200, logits="uniform"),
    "max_ffn_stream_fp8": synth.LayerConfig("max_ffn_stream_fp8", T=24, H=128, F=16384, F_s=16384, E=4, E_loc=4,
                                            e0=0, K=2, dtype="fp8", T_s=24, logits="uniform"),
    "max_ffn_tile_fp8": synth.LayerConfig("max_ffn_tile_fp8", T=200, H=128, F=16384, F_s=16384, E=4, E_loc=4, e0=0,
                                          K=2, dtype="fp8", T_s=200, logits="uniform"),
    "rows_257_fp8": synth.LayerConfig("rows_257_fp8", T=257, H=512, F=256, F_s=0, E=1, E_loc=1, e0=0, K=1,
                                      dtype="fp8", T_s=0, logits="single"),
    "rows_513_bf16": synth.LayerConfig("rows_513_bf16", T=513, H=384, F=128, F_s=128, E=1, E_loc=1, e0=0, K=1,
                                       dtype="bf16", T_s=513, logits="single"),
}


def _run(name):
    cfg = CASES[name]
    say(f"[{name}] {cfg}")
    layer = build_layer(cfg)
    x_bits, wr, given = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    get = weights_provider(cfg)
    ref = oracle.moe_forward(cfg, x_bits, get, w_r=wr, logits=given, score_bias=score_bias_of(cfg))
    return cfg, layer, x, x_bits, wr, given, ref


@pytest.mark.parametrize("name", list(CASES))
def test_forward_matches_oracle(name):
    cfg, layer, x, x_bits, wr, given, ref = _run(name)
    check_forward(cfg, layer, x, wr, given, ref)


def test_forward_is_deterministic():
    cfg, layer, x, x_bits, wr, given, ref = _run("prefill_small_fp8")
    wdev = torch.from_numpy(wr).to(DEV)
    a = layer.forward(x, cfg.T_s, w_router=wdev)["y"].clone()
    b = layer.forward(x, cfg.T_s, w_router=wdev)["y"].clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,K", [("fp8", 2), ("bf16", 2), ("fp8", 4), ("bf16", 4), ("fp8", 8), ("bf16", 8)])
def test_all_tokens_on_one_expert_and_empty_experts(dtype, K):
    """Every token's top-1 is expert 5 and its next choices are the same 1, 3 or 7 experts (K = 8: experts 9, 12,
    20 and the four lowest-index experts among the equal rest); the other experts get no rows. The host bound on
    rows per expert (T*K/E = 13, 25 or 50) selects the weight-streaming kernel with 16 or 32 rows per pass (the
    200-row experts take 13 or 7 passes) or, at 50, the tile GEMM with two 128-row tiles per busy expert."""
    cfg = synth.LayerConfig("skew", T=200, H=512, F=256, F_s=256, E=32, E_loc=32, e0=0, K=K, dtype=dtype,
                            T_s=0, logits="uniform")
    layer = build_layer(cfg)
    x_bits = synth.x_bf16(cfg)
    L = np.full((cfg.T, cfg.E), -5.0, np.float32)
    L[:, 5] = 3.0
    L[:, 9] = np.linspace(-1, 1, cfg.T).astype(np.float32)
    L[:, 12] = np.linspace(-2, -1.5, cfg.T).astype(np.float32)
    L[:, 20] = -3.0
    ref = oracle.moe_forward(cfg, x_bits, weights_provider(cfg), logits=L)
    check_given_logits_path(cfg, layer, to_dev_bf16(x_bits), ref, L)


def test_zero_tokens_is_a_no_op():
    cfg = CASES["tiny"]
    layer = build_layer(cfg)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device=DEV)
    out = layer.forward(x, 0, logits=torch.empty((0, cfg.E), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert out["y"].shape == (0, cfg.H)


@pytest.mark.parametrize("name", ["nondiv_small_fp8", "prefill_small_fp8", "wide_gateup_fp8"])
def test_separate_entry_points_match_forward(name):
    """route -> permute -> quant -> gateup -> quant -> down -> shared -> combine, one call at a time, bit for bit
    against dmoe_forward on the same logits (weight-streaming and tile GEMMs; the forward runs the shared expert
    as an extra group of the routed launches, the entry point as a GEMM of its own; on the wide case the forward
    quantises h in the gate/up epilogue, the separate calls through dmoe_quant_act)."""
    import fp8_expert_ffn_amd as dm
    cfg, layer, x, x_bits, wr, given, ref = _run(name)
    logits = torch.from_numpy(given if given is not None else ref.logits).to(DEV)
    full = layer.forward(x, cfg.T_s, logits=logits)["y"].clone()
    ids, w = dm.dmoe_route(logits, cfg.K)
    off, rt, rs, tr = dm.dmoe_permute(ids, cfg.e0, cfg.E_loc)
    xq, xs = dm.dmoe_quant_act(x)
    mcap = cfg.T * cfg.K
    h = torch.empty((mcap, layer.fpad), dtype=torch.bfloat16, device=DEV)
    dm.dmoe_grouped_gemm_gateup(dm.DMOE_FP8_E4M3, xq, xs, rt, off, cfg.E_loc, mcap, layer.w_gate, layer.w_up,
                                layer.s_gate, layer.s_up, cfg.H, cfg.F, h)
    M = int(off[-1].item())
    hq, hs = dm.dmoe_quant_act(h[:M], cfg.F)
    o = torch.empty((mcap, cfg.H), dtype=torch.bfloat16, device=DEV)
    dm.dmoe_grouped_gemm_down(dm.DMOE_FP8_E4M3, hq, hs, off, cfg.E_loc, M, layer.w_down, layer.s_down, cfg.F,
                              cfg.H, o)
    s = torch.empty((cfg.T_s, cfg.H), dtype=torch.bfloat16, device=DEV)
    dm.dmoe_shared_expert(dm.DMOE_FP8_E4M3, xq, xs, cfg.T_s, layer.sw_gate, layer.sw_up, layer.sw_down,
                          (layer.ss_gate, layer.ss_up, layer.ss_down), cfg.H, cfg.F_s, s)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    dm.dmoe_combine(o, tr, w, s, cfg.T_s, cfg.H, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), full.view(torch.int16))


def test_timed_forward_matches_forward():
    """dmoe_forward_timed with every stage boundary, with only the gate/up boundaries (NULL entries elsewhere),
    and dmoe_forward produce bit-identical outputs; the recorded events bracket non-negative intervals."""
    import fp8_expert_ffn_amd as dm
    cfg, layer, x, x_bits, wr, given, ref = _run("prefill_small_fp8")
    wdev = torch.from_numpy(wr).to(DEV)
    d, p, ws, out = layer.make_call(x, cfg.T_s, w_router=wdev)
    y = out["y"]
    stream = torch.cuda.current_stream()
    dm.dmoe_forward(d, p, ws)
    torch.cuda.synchronize()
    y0 = y.clone()
    n = dm.DMOE_STAGES + 1
    gu = dm.STAGE_NAMES.index("gateup")
    for which in (set(range(n)), {gu, gu + 1}):
        ev = [torch.cuda.Event(enable_timing=True) if s in which else None for s in range(n)]
        for e in ev:
            if e is not None:
                e.record(stream)
        torch.cuda.synchronize()
        y.zero_()
        dm.dmoe_forward_timed(d, p, ws, ev)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        assert ev[gu].elapsed_time(ev[gu + 1]) >= 0.0
