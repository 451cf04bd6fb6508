"""Full-size workloads through dmoe_forward, in the launch configuration the
benchmark times (GPU).

The oracle computes a sample of tokens exactly as the full layer would (each
token's output depends only on its own row); every token is checked against
properties that hold at any size."""
import gc
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DEV, LOGIT_TOL, W_TOL, bf16_values, build_layer, compare_y, layer_inputs, near_tie_tokens, say,
                      score_bias_of, to_dev_bf16, weights_provider)

pytestmark = pytest.mark.gpu

from fp8_expert_ffn_amd import _lib as L  # noqa: E402

SAMPLES = {1: 16, 2: 5, 3: 6, 4: 5, 5: 8, 6: 8, 7: 4, 8: 10, 9: 6}


def _sample_tokens(cfg, n):
    rng = np.random.default_rng(1234)
    picks = {0, cfg.T - 1}
    if 0 < cfg.T_s < cfg.T:
        picks |= {cfg.T_s - 1, cfg.T_s}
    while len(picks) < min(n, cfg.T):
        picks.add(int(rng.integers(0, cfg.T)))
    return np.array(sorted(picks))


def _expert_o_check(cfg, x_bits, o_rows, tokens, e, what):
    """GPU expert outputs o (rows for the given tokens) against oracle.swiglu_expert on the same tokens."""
    x = oracle.bf16_to_f64(np.asarray(x_bits)[tokens])
    if cfg.dtype == "fp8":
        a = oracle.dequantize_act(*oracle.quantize_act(x))
        w = [oracle.dequantize_weight_blocks(*oracle.quantize_weight_blocks(synth.expert_weight_f32(cfg, n, e)))
             for n in ("gate", "up", "down")]
    else:
        a = x
        w = [oracle.bf16_to_f64(synth.expert_weight_bf16(cfg, n, e)) for n in ("gate", "up", "down")]
    o_ref = oracle.swiglu_expert(a, *w, fp8=cfg.dtype == "fp8")
    o_sum = oracle.swiglu_expert(a, *w, fp8=cfg.dtype == "fp8", rounded=False)
    compare_y(o_rows, o_ref, o_sum, what)


def _check_whole_experts(cfg, layer, d, ws, x_bits, offsets):
    """Expert outputs at full size, where tile positions differ from the reduced tests: the busiest local expert
    (the first and last row of every 64-row block, i.e. of every wave's rows in every 256-row tile), the smallest
    touched expert (all rows) and the last partial tile of the shared expert (all rows)."""
    o = layer.ws_view(d, ws, "o")
    rt = layer.ws_view(d, ws, "row_token").cpu().numpy()
    counts = np.diff(offsets)
    big = int(np.argmax(counts))
    r0, r1 = int(offsets[big]), int(offsets[big + 1])
    rel = np.arange(r1 - r0)
    rows = r0 + rel[(rel % 64 == 0) | (rel % 64 == 63) | (rel == rel[-1])]
    t0 = time.time()
    _expert_o_check(cfg, x_bits, bf16_values(o[rows]), rt[rows], cfg.e0 + big,
                    f"o of the busiest expert {cfg.e0 + big} ({r1 - r0} rows, {rows.size} checked)")
    touched = np.nonzero(counts)[0]
    small = int(touched[np.argmin(counts[touched])])
    s0, s1 = int(offsets[small]), int(offsets[small + 1])
    _expert_o_check(cfg, x_bits, bf16_values(o[s0:s1]), rt[s0:s1], cfg.e0 + small,
                    f"o of the smallest expert {cfg.e0 + small} ({s1 - s0} rows)")
    if cfg.T_s > 0 and cfg.F_s == cfg.F:
        # shared rows follow the T*K routed rows of o; its last tile of the 256-row schedule
        mcap = cfg.T * cfg.K
        first = (cfg.T_s - 1) // 256 * 256
        start = L.dmoe_forward_ws_offset(d, 9)  # o, routed rows then the shared rows
        o_all = ws[start:start + (mcap + cfg.T_s) * cfg.H * 2].view(torch.bfloat16).view(-1, cfg.H)
        _expert_o_check(cfg, x_bits, bf16_values(o_all[mcap + first:mcap + cfg.T_s]),
                        np.arange(first, cfg.T_s), synth.SHARED,
                        f"o of the shared expert's last tile (tokens {first}..{cfg.T_s - 1})")
    say(f"  whole-expert checks in {time.time() - t0:.1f}s")


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_full_size_workload(ci):
    cfg = synth.config(ci)
    say(f"[full size {ci}] {cfg}")
    t0 = time.time()
    layer = build_layer(cfg)
    say(f"  weights ready in {time.time() - t0:.1f}s")
    x_bits, wr, given = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    out = layer.forward(x, cfg.T_s, w_router=None if wr is None else torch.from_numpy(wr).to(DEV),
                        logits=None if given is None else torch.from_numpy(given).to(DEV))
    torch.cuda.synchronize()
    d, p, ws = out["_call"]

    # --- properties of every token
    ids = out["topk_ids"].cpu().numpy()
    w = out["topk_w"].cpu().numpy().astype(np.float64)
    y = bf16_values(out["y"])
    assert np.all((ids >= 0) & (ids < cfg.E))
    assert np.all(np.sort(ids, 1)[:, 1:] != np.sort(ids, 1)[:, :-1]), "duplicate experts in a token"
    assert np.max(np.abs(w.sum(1) - 1)) <= W_TOL and np.all(np.diff(w, axis=1) <= 0)
    local = (ids >= cfg.e0) & (ids < cfg.e0 + cfg.E_loc)
    offsets = layer.ws_view(d, ws, "offsets").cpu().numpy()
    assert offsets[-1] == local.sum()
    np.testing.assert_array_equal(np.diff(offsets), np.bincount(ids[local] - cfg.e0, minlength=cfg.E_loc))
    tr = layer.ws_view(d, ws, "token_row").cpu().numpy()
    assert np.array_equal(tr >= 0, local)
    rt = layer.ws_view(d, ws, "row_token").cpu().numpy()[:offsets[-1]]
    np.testing.assert_array_equal(rt[tr[local]], np.nonzero(local)[0])
    assert np.all(np.isfinite(y))
    say(f"  M = {offsets[-1]}, touched experts = {(np.diff(offsets) > 0).sum()}")

    # --- sampled tokens against the oracle
    tok = _sample_tokens(cfg, SAMPLES[ci])
    t0 = time.time()
    ref = oracle.moe_forward(cfg, x_bits, weights_provider(cfg), w_r=wr, logits=given, tokens=tok,
                             score_bias=score_bias_of(cfg))
    say(f"  oracle on {tok.size} tokens in {time.time() - t0:.1f}s")
    if given is None:
        L = out["logits"].cpu().numpy()[tok]
        err = float(np.max(np.abs(L.astype(np.float64) - ref.logits)))
        say(f"  router logits max |dL| = {err:.3e}")
        assert err <= LOGIT_TOL
    diff = near_tie_tokens(ids[tok], ref.ids, ref.logits, 2 * LOGIT_TOL)
    keep = np.setdiff1d(np.arange(tok.size), diff)
    assert diff.size <= 1
    if given is not None:
        assert diff.size == 0
        assert np.max(np.abs(w[tok] - ref.w)) <= W_TOL
    if cfg.dtype == "fp8":
        xq = layer.ws_view(d, ws, "x_codes").cpu().numpy()[tok]
        xs = layer.ws_view(d, ws, "x_scales").cpu().numpy()[tok]
        np.testing.assert_array_equal(xq, ref.x_codes)
        np.testing.assert_array_equal(xs, ref.x_scales)
    compare_y(y[tok][keep], ref.y[keep], ref.y_sum[keep], f"y sampled ({keep.size} tokens)", ref.y_allow[keep])
    if ci in (2, 3, 4):
        _check_whole_experts(cfg, layer, d, ws, x_bits, offsets)
    del layer, out, ws
    gc.collect()
    torch.cuda.empty_cache()
