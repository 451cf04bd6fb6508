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

SAMPLES = {1: 16, 2: 5, 3: 6, 4: 5, 5: 8, 6: 8, 7: 4, 8: 10, 9: 6}


def _sample_tokens(cfg, n):
    rng = np.random.default_rng(1234)
    picks = {0, cfg.T - 1}
    if 0 < cfg.T_s < cfg.T:
        picks |= {cfg.T_s - 1, cfg.T_s}
    while len(picks) < min(n, cfg.T):
        picks.add(int(rng.integers(0, cfg.T)))
    return np.array(sorted(picks))


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
    compare_y(y[tok][keep], ref.y[keep], ref.y_sum[keep], f"y sampled ({keep.size} tokens)")
    del layer, out, ws
    gc.collect()
    torch.cuda.empty_cache()
