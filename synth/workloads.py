"""Workload shapes and seeded, counter-addressed input draws.

Shapes follow the dots3-note preview MoE layer: hidden 5120, 256 routed experts
plus 1 shared expert, top-8, per-expert FFN 1536 (model card
"dots-studio/dots3-note-prev", Model Overview table; Transformers documentation
"Dots 3 Note Preview", Dots3NoteTextConfig parameters ``hidden_size``,
``n_routed_experts``, ``n_shared_experts``, ``num_experts_per_tok``,
``moe_intermediate_size``, ``shared_experts_intermediate_size``).

Every tensor is drawn from its own PCG64 stream keyed by
``(seed, tensor tag, expert index)``, so any single expert's weights can be
regenerated without drawing the others. Draws:

* ``x``        -- N(0, 1) in float32, rounded to bfloat16 (round to nearest even).
* ``router``   -- N(0, 0.02) in float32, the FP32 router weight ``[E, H]``.
* ``gate``, ``up`` -- N(0, 1/sqrt(H)) in float32, ``[F, H]`` per expert.
* ``down``     -- N(0, 1/sqrt(F)) in float32, ``[H, F]`` per expert.
* skewed logits (EP8 share) -- ``-1.1*ln(e+1) + N(0,1)`` in float64, stored as float32.
* uniform logits (non-divisible stress) -- U[-4, 4) in float64, stored as float32.
* single logits (dense layer as one expert) -- zeros.
* ``bias``     -- N(0, 0.01) in float32, the per-expert selection bias of sigmoid scoring.

BF16 workloads store the weights as bfloat16 (round to nearest even of the
float32 draw); FP8 workloads keep the float32 draw, which each consumer
block-quantises itself.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "SHARED", "config", "rng", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "x_bf16", "router_weight", "given_logits", "score_bias", "expert_weight_f32", "expert_weight_bf16",
    "fill_expert_weights", "weight_shape", "gen_threads",
]

SHARED = -1  # expert index used for the shared expert's streams

_TAGS = {"x": 1, "router": 2, "logits": 3, "bias": 4, "gate": 11, "up": 12, "down": 13}


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One MoE-layer workload.

    T tokens of width H; E routed experts of which this GPU holds E_loc starting
    at e0; top-K routing; routed FFN width F; shared FFN width F_s applied to
    tokens [0, T_s). ``logits`` says where the router logits come from:
    "router" (x @ W_r^T), "zipf" (skewed, given), "uniform" (given) or
    "single" (given zeros, for E = K = 1).
    """
    name: str
    T: int
    H: int
    F: int
    F_s: int
    E: int
    E_loc: int
    e0: int
    K: int
    dtype: str  # "bf16" or "fp8"
    T_s: int
    logits: str
    seed: int = 0
    # routing options (Dots3NoteTextConfig n_group, topk_group, norm_topk_prob, routed_scaling_factor)
    n_group: int = 1
    topk_group: int = 0  # 0: every group
    renormalize: bool = True
    scaling: float = 1.0
    scoring: str = "softmax"  # or "sigmoid" (with a per-expert selection bias, see score_bias)

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def experts(self) -> range:
        return range(self.e0, self.e0 + self.E_loc)


CONFIGS = [
    LayerConfig("tiny_bf16", T=128, H=512, F=128, F_s=128, E=16, E_loc=16, e0=0, K=4,
                dtype="bf16", T_s=128, logits="router"),
    LayerConfig("decode_bf16", T=64, H=5120, F=1536, F_s=1536, E=256, E_loc=256, e0=0, K=8,
                dtype="bf16", T_s=64, logits="router"),
    LayerConfig("prefill_fp8", T=8192, H=5120, F=1536, F_s=1536, E=256, E_loc=256, e0=0, K=8,
                dtype="fp8", T_s=8192, logits="router"),
    LayerConfig("ep8_share_fp8", T=16384, H=5120, F=1536, F_s=1536, E=256, E_loc=32, e0=0, K=8,
                dtype="fp8", T_s=2048, logits="zipf"),
    LayerConfig("nondiv_fp8", T=2048, H=5120, F=1400, F_s=1400, E=256, E_loc=256, e0=0, K=8,
                dtype="fp8", T_s=2048, logits="uniform"),
    # Vision-tower MoE (Transformers documentation "Dots 3 Note Preview", Dots3NoteVisionConfig: hidden_size 1536,
    # moe_intermediate_size 2112, num_local_experts 64, FP32 router; no shared expert). The docs leave
    # num_experts_per_tok unset; the text model's top-8 is used. 2112 = 16.5 x 128: a partial FP8 block.
    LayerConfig("vision_bf16", T=4096, H=1536, F=2112, F_s=0, E=64, E_loc=64, e0=0, K=8,
                dtype="bf16", T_s=0, logits="router"),
    LayerConfig("vision_fp8", T=4096, H=1536, F=2112, F_s=0, E=64, E_loc=64, e0=0, K=8,
                dtype="fp8", T_s=0, logits="router"),
    # Dense first-layer FFN (Dots3NoteTextConfig intermediate_size 13824) as one expert with top-1:
    # every token's single routing weight is exactly 1, so y is the dense SwiGLU FFN output.
    LayerConfig("dense_fp8", T=4096, H=5120, F=13824, F_s=0, E=1, E_loc=1, e0=0, K=1,
                dtype="fp8", T_s=0, logits="single"),
    # Speculative-decoding verify batch: the SGLang cookbook's decode graphs cover batches of up to 32 and NEXTN
    # verifies 4 draft tokens per step, so one verify step carries 32 x 4 = 128 tokens (both checkpoints).
    LayerConfig("verify_bf16", T=128, H=5120, F=1536, F_s=1536, E=256, E_loc=256, e0=0, K=8,
                dtype="bf16", T_s=128, logits="router"),
    LayerConfig("verify_fp8", T=128, H=5120, F=1536, F_s=1536, E=256, E_loc=256, e0=0, K=8,
                dtype="fp8", T_s=128, logits="router"),
]


def config(i: int, **overrides) -> LayerConfig:
    c = CONFIGS[i]
    return c.replace(**overrides) if overrides else c


def gen_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    """Independent stream for (seed, tensor tag, index); index -1 is the shared expert."""
    key = [int(seed), _TAGS[tag], int(idx) + 1]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def x_bf16(cfg: LayerConfig) -> np.ndarray:
    """Token activations [T, H] as bfloat16 bits."""
    g = rng(cfg.seed, "x")
    return f32_to_bf16_bits(g.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def router_weight(cfg: LayerConfig) -> np.ndarray:
    """FP32 router weight [E, H] ~ N(0, 0.02)."""
    g = rng(cfg.seed, "router")
    w = g.standard_normal((cfg.E, cfg.H), dtype=np.float32)
    return (w * np.float32(0.02)).astype(np.float32)


def given_logits(cfg: LayerConfig) -> np.ndarray:
    """Router logits [T, E] for the workloads whose logits are an input."""
    g = rng(cfg.seed, "logits")
    if cfg.logits == "zipf":
        bias = -1.1 * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))
        return (bias[None, :] + g.standard_normal((cfg.T, cfg.E))).astype(np.float32)
    if cfg.logits == "uniform":
        return g.uniform(-4.0, 4.0, size=(cfg.T, cfg.E)).astype(np.float32)
    if cfg.logits == "single":
        return np.zeros((cfg.T, cfg.E), dtype=np.float32)
    raise ValueError(f"workload {cfg.name} computes its logits from x")


def score_bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert FP32 selection bias [E] for sigmoid scoring ~ N(0, 0.01)."""
    g = rng(cfg.seed, "bias")
    return (g.standard_normal(cfg.E, dtype=np.float32) * np.float32(0.01)).astype(np.float32)


def weight_shape(cfg: LayerConfig, which: str, e: int) -> tuple[int, int]:
    f = cfg.F_s if e == SHARED else cfg.F
    return (f, cfg.H) if which in ("gate", "up") else (cfg.H, f)


def expert_weight_f32(cfg: LayerConfig, which: str, e: int) -> np.ndarray:
    """One expert's weight in nn.Linear layout [out, in], float32 draw."""
    rows, cols = weight_shape(cfg, which, e)
    g = rng(cfg.seed, which, e)
    w = g.standard_normal((rows, cols), dtype=np.float32)
    return (w * np.float32(1.0 / np.sqrt(cols))).astype(np.float32)


def expert_weight_bf16(cfg: LayerConfig, which: str, e: int) -> np.ndarray:
    return f32_to_bf16_bits(expert_weight_f32(cfg, which, e))


def fill_expert_weights(cfg: LayerConfig, which: str, experts, sink, as_bf16: bool,
                        threads: int | None = None) -> None:
    """Draw many experts' weights in parallel and hand each to ``sink(i, array)``.

    ``experts`` is a sequence of expert indices; ``sink`` receives the position
    in that sequence and the drawn array (bf16 bits or float32). Calls to sink
    happen in order of position on the calling thread.
    """
    experts = list(experts)
    draw = expert_weight_bf16 if as_bf16 else expert_weight_f32
    n = threads or gen_threads()
    with _cf.ThreadPoolExecutor(max_workers=n) as ex:
        futs = {}
        nxt = 0
        for i in range(len(experts)):
            while nxt < len(experts) and nxt < i + 2 * n:
                futs[nxt] = ex.submit(draw, cfg, which, experts[nxt])
                nxt += 1
            sink(i, futs.pop(i).result())
