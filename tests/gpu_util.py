"""Helpers for the GPU parity tests: build a device layer from the seeded
workload generator, run the oracle on the same inputs, and compare."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth

DEV = "cuda"

# Output tolerance of the layer (floating point): relative L2 error and
# maximum absolute error relative to the RMS of the reference output.
REL_L2 = 5e-3
MAX_ABS_OVER_RMS = 2e-2
W_TOL = 1e-6        # routing weights
LOGIT_TOL = 1e-4    # router logits (FP32 accumulation order)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def weights_provider(cfg):
    """Host weights as each side takes them: FP32 draws (FP8) or BF16 bits (BF16)."""
    @functools.lru_cache(maxsize=64)
    def get(which, e):
        return (synth.expert_weight_f32(cfg, which, e) if cfg.dtype == "fp8"
                else synth.expert_weight_bf16(cfg, which, e))
    return get


def build_layer(cfg, threads=None):
    """MoELayer with every local expert and the shared expert set from the generator."""
    from fp8_expert_ffn_amd import MoELayer
    layer = MoELayer(cfg.H, cfg.F, cfg.F_s, cfg.E, cfg.E_loc, cfg.e0, cfg.K, cfg.dtype, DEV, n_group=cfg.n_group,
                     topk_group=cfg.topk_group, renormalize=cfg.renormalize, routed_scaling_factor=cfg.scaling,
                     scoring=cfg.scoring)
    if cfg.scoring == "sigmoid":
        layer.set_score_bias(synth.score_bias(cfg))
    as_bf16 = cfg.dtype == "bf16"
    for which in ("gate", "up", "down"):
        synth.fill_expert_weights(cfg, which, cfg.experts,
                                  lambda i, arr, w=which: layer.set_weight(w, i, arr), as_bf16, threads)
        if cfg.F_s:
            arr = synth.expert_weight_bf16(cfg, which, synth.SHARED) if as_bf16 else \
                synth.expert_weight_f32(cfg, which, synth.SHARED)
            layer.set_weight(which, -1, arr)
    torch.cuda.synchronize()
    return layer


def score_bias_of(cfg):
    """The per-expert selection bias for sigmoid-scored workloads (None otherwise)."""
    return synth.score_bias(cfg) if cfg.scoring == "sigmoid" else None


def layer_inputs(cfg):
    x = synth.x_bf16(cfg)
    if cfg.logits == "router":
        return x, synth.router_weight(cfg), None
    return x, None, synth.given_logits(cfg)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v| (8 significant bits); 0 for v == 0."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.frexp(a)[1]  # a = m * 2^e, 0.5 <= m < 1
    return np.where(a > 0, np.ldexp(1.0, np.maximum(e - 8, -133)), 0.0)


def compare_y(y_gpu: np.ndarray, y_ref: np.ndarray, y_sum: np.ndarray, what: str = "y",
              allow: np.ndarray | None = None) -> tuple[float, float]:
    """Layer-output tolerance: relative L2 <= 5e-3 against the oracle's BF16 y, and for EVERY element
    |y_gpu - y_sum| <= 2e-2 * RMS(y_ref) + ulp_bf16 / 2 + allow, where y_sum is the oracle's float64 combine sum
    before its one BF16 rounding.

    The half ulp is the GPU's own final rounding: the GPU output is the BF16 rounding of a value near y_sum,
    and that rounding moves it by at most half a BF16 ulp (taken at the larger of |y_gpu| and |y_sum|, which
    covers a rounding up into the next binade). ``allow`` is the oracle's rounding_allowance: for the expert
    outputs whose exact value sits on a BF16 rounding midpoint within the precision of their sum (float32, or
    on the FP8 path the FP8 matrix cores' block sums), either neighbour is a correct rounding, and the other
    choice moves y by the weight times the BF16 spacing; it is zero for every element whose expert outputs are
    decided. Everything else, i.e. the distance of the GPU's unrounded value
    from the oracle's, must stay within 2e-2 RMS. The literal max |y_gpu - y_ref| / RMS is reported.
    """
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    y_sum = np.asarray(y_sum, np.float64)
    assert y_gpu.shape == y_ref.shape == y_sum.shape, f"{what}: shapes differ"
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    if y_ref.size == 0:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    mx = float(np.abs(y_gpu - y_ref).max() / max(rms, 1e-300))
    err = np.abs(y_gpu - y_sum)
    bound = MAX_ABS_OVER_RMS * rms + 0.5 * bf16_ulp(np.maximum(np.abs(y_gpu), np.abs(y_sum)))
    n_allow = 0
    if allow is not None:
        allow = np.asarray(allow, np.float64)
        assert allow.shape == y_sum.shape, f"{what}: allowance shape differs"
        bound = bound + allow
        n_allow = int(np.count_nonzero(allow))
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  {what}: rel_l2={rel:.3e} max|y-y_ref|/rms={mx:.3e} "
        f"max |y-y_sum|/(2e-2 RMS + ulp/2 + straddle allowance) = {worst:.3f} (n={y_ref.size}, "
        f"{n_allow} elements with an allowance)")
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert worst <= 1.0, f"{what}: an element is further than 2e-2 RMS + ulp/2 from the oracle ({worst:.3f} x)"
    return rel, mx


def near_tie_tokens(ids_gpu: np.ndarray, ids_ref: np.ndarray, logits_ref: np.ndarray, tol: float) -> np.ndarray:
    """Tokens whose top-K sets differ; each difference must be explained by logits within tol."""
    diff = np.nonzero(np.any(np.sort(ids_gpu, 1) != np.sort(ids_ref, 1), axis=1))[0]
    for t in diff:
        only_g = sorted(set(ids_gpu[t]) - set(ids_ref[t]))
        only_r = sorted(set(ids_ref[t]) - set(ids_gpu[t]))
        kth = np.sort(logits_ref[t])[::-1][ids_ref.shape[1] - 1]
        for e in only_g + only_r:
            assert abs(float(logits_ref[t, e]) - float(kth)) <= tol, \
                f"token {t}: expert {e} differs but is not a near tie ({logits_ref[t, e]} vs {kth})"
    return diff


def check_given_logits_path(cfg, layer, x, ref, logits_np):
    """Same logits on both sides: routing, permutation and x codes must be bit-exact."""
    out = layer.forward(x, cfg.T_s, logits=torch.from_numpy(logits_np).to(DEV))
    torch.cuda.synchronize()
    d, p, ws = out["_call"]
    np.testing.assert_array_equal(out["topk_ids"].cpu().numpy(), ref.ids)
    assert np.max(np.abs(out["topk_w"].cpu().numpy().astype(np.float64) - ref.w)) <= W_TOL
    off_r, rt_r, rs_r, tr_r = oracle.permute(ref.ids, cfg.e0, cfg.E_loc)
    M = int(off_r[-1])
    np.testing.assert_array_equal(layer.ws_view(d, ws, "offsets").cpu().numpy(), off_r)
    np.testing.assert_array_equal(layer.ws_view(d, ws, "row_token").cpu().numpy()[:M], rt_r)
    np.testing.assert_array_equal(layer.ws_view(d, ws, "row_slot").cpu().numpy()[:M], rs_r)
    np.testing.assert_array_equal(layer.ws_view(d, ws, "token_row").cpu().numpy(), tr_r)
    if cfg.dtype == "fp8":
        np.testing.assert_array_equal(layer.ws_view(d, ws, "x_codes").cpu().numpy(), ref.x_codes)
        np.testing.assert_array_equal(layer.ws_view(d, ws, "x_scales").cpu().numpy(), ref.x_scales)
    y = bf16_values(out["y"])
    # rows with no local pair and no shared expert are exactly zero on both sides
    idle = ~np.any(tr_r >= 0, axis=1) & (np.arange(cfg.T) >= cfg.T_s)
    assert np.all(y[idle] == 0) and np.all(ref.y[idle] == 0)
    compare_y(y[~idle], ref.y[~idle], ref.y_sum[~idle], "y (given logits)", ref.y_allow[~idle])
    return out


def check_forward(cfg, layer, x, wr, given, ref):
    """Both legs of the layer check: the oracle's (or the given) logits handed to the GPU, then, for router
    workloads, the full path with the GPU's own router logits (near ties may route differently)."""
    if given is not None:
        check_given_logits_path(cfg, layer, x, ref, given)
        return
    # 1) the oracle's logits given to the GPU: exact routing, tolerance on y
    check_given_logits_path(cfg, layer, x, ref, ref.logits)
    # 2) the full path with the GPU's own router logits
    out = layer.forward(x, cfg.T_s, w_router=torch.from_numpy(wr).to(DEV))
    torch.cuda.synchronize()
    L = out["logits"].cpu().numpy()
    err = float(np.max(np.abs(L.astype(np.float64) - ref.logits)))
    say(f"  router logits max |dL| = {err:.3e}")
    assert err <= LOGIT_TOL
    ids = out["topk_ids"].cpu().numpy()
    diff = near_tie_tokens(ids, ref.ids, ref.logits, 2 * LOGIT_TOL)
    keep = np.setdiff1d(np.arange(cfg.T), diff)
    assert diff.size <= max(1, cfg.T // 100), f"{diff.size} tokens routed differently"
    compare_y(bf16_values(out["y"])[keep], ref.y[keep], ref.y_sum[keep], "y (own logits)", ref.y_allow[keep])
