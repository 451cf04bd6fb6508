"""Seeded draws of layer shapes for the shape sweep (GPU parity against the
oracle, and the host-side check that every draw is a valid layer).

Only shapes and routing options are drawn here; the tensors come from the
workload generator under each case's own seed. Cases cycle through four
regimes of rows per local expert (the host bound ceil(T*K / E_loc)): at most
32 (weight-streaming kernel), 33-127 and 128-700 (two-workgroup tile kernel,
one or several 128-row tiles per expert) and, for FP8, 512-640 with wide h
(many 128-column slices of h: the wide kernel with h quantised in the gate/up
epilogue). Within a regime the hidden width, FFN widths (any multiple of 8, so
partial 128-wide slices are common), expert counts, local range, shared-token
count, logit source and routing options are drawn at random.
"""
from __future__ import annotations

import math

import numpy as np

import synth

SWEEP_SEED = 20261203
REGIMES = ("stream", "tile", "tile_many", "wide_fused")


def _divisors(n: int) -> list[int]:
    return [d for d in range(2, min(n, 64) + 1) if n % d == 0]


def _rows_target(rng: np.random.Generator, regime: str) -> int:
    lo, hi = {"stream": (1, 32), "tile": (33, 127), "tile_many": (128, 700), "wide_fused": (512, 640)}[regime]
    return int(rng.integers(lo, hi + 1))


def draw_case(rng: np.random.Generator, i: int) -> synth.LayerConfig:
    regime = REGIMES[i % len(REGIMES)]
    dtype = "fp8" if regime == "wide_fused" or (i // len(REGIMES)) % 2 == 0 else "bf16"
    if regime == "wide_fused":
        # 20-25 column blocks of h and 12-16 local experts: (rows / 256 + E_loc) tiles x blocks >= 1024 items
        H = int(rng.choice([128, 256]))
        F = 8 * int(rng.integers(320, 401))  # 2560 .. 3200
        E = int(rng.integers(16, 33))
    elif regime == "tile_many":
        H = int(rng.choice([128, 256, 384, 512]))
        F = 8 * int(rng.integers(1, 129))  # 8 .. 1024
        E = int(rng.integers(1, 17))
    else:
        H = int(rng.choice([128, 256, 384, 512, 768, 1024]))
        F = 8 * int(rng.integers(1, 200))  # 8 .. 1592
        E = int(rng.integers(1, 65))
    K = int(rng.integers(1, min(E, 8) + 1))
    if regime == "wide_fused":
        E_loc = int(rng.integers(12, 17))
        e0 = int(rng.integers(0, E - E_loc + 1))
    elif rng.random() < 0.5:
        E_loc, e0 = E, 0
    else:
        E_loc = int(rng.integers(1, E + 1))
        e0 = int(rng.integers(0, E - E_loc + 1))
    r = _rows_target(rng, regime)
    # T with ceil(T*K / E_loc) == r where possible (at least one token)
    T = max(1, (r * E_loc) // K)
    while T > 1 and math.ceil(T * K / E_loc) > r:
        T -= 1
    u = rng.random()
    T_s = 0 if u < 0.3 else (T if u < 0.65 else int(rng.integers(0, T + 1)))
    v = rng.random()
    F_s = 0 if v < 0.2 else (F if v < 0.6 else 8 * int(rng.integers(1, F // 8 + 33)))
    logits = str(rng.choice(["router", "uniform", "zipf"])) if E > 1 else "single"
    kw = {}
    w = rng.random()
    if E > 1 and w < 0.25:
        divs = [d for d in _divisors(E) if d >= 2]
        if divs:
            g = int(rng.choice(divs))
            gs = E // g
            tg_min = max(1, math.ceil(K / gs))
            tg = int(rng.integers(tg_min, g + 1))
            kw.update(n_group=g, topk_group=tg)
        kw.update(renormalize=bool(rng.random() < 0.5), scaling=float(rng.choice([1.0, 2.5])))
    elif E > 1 and w < 0.4:
        kw.update(scoring="sigmoid", scaling=float(rng.choice([1.0, 1.5])))
    return synth.LayerConfig(f"sweep{i:02d}_{regime}_{dtype}", T=T, H=H, F=F, F_s=F_s, E=E, E_loc=E_loc, e0=e0,
                             K=K, dtype=dtype, T_s=T_s, logits=logits, seed=1000 + i, **kw)


def sweep_cases(n: int = 24, seed: int = SWEEP_SEED) -> list[synth.LayerConfig]:
    rng = np.random.default_rng(seed)
    return [draw_case(rng, i) for i in range(n)]
