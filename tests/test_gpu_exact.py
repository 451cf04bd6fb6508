"""Exactness of the grouped GEMMs on integer-valued operands (GPU).

With integer operands (BF16, or E4M3 codes of small integers with power-of-two
scales) every product and every partial sum is an integer below 2^24, so any
correct float32 evaluation is exact; the expected outputs are plain float64
sums of the drawn integers, rounded once to BF16. Gate/up: activation rows
with 128 ones and zeros elsewhere, gate weights in {0, 1} (so every gate sum
lies in [17, 128], where silu(g) equals g in float32 and is within 1e-7 of it
in float64) and up weights with two non-zero entries of +-1 per row, so
h = g * u is an integer of magnitude at most 256 and exact in BF16. Down: h
and weights in [-15, 15] (every such integer is an E4M3 value) with scales
2^0 .. 2^2; the FP8 down runs on FP8 matrix cores, whose block sums are then
exact too. Each case runs on the weight-streaming, two-workgroup tile and wide
tile kernels (the launcher's choice is checked through the layer's kernel
query for the same row bound)."""
import zlib

import numpy as np
import pytest
import torch

import fp8_expert_ffn_amd as dm
from fp8_expert_ffn_amd import _lib as L
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

# (rows per expert, E_loc, H, F) per kernel regime of each projection
GATEUP = {"stream": (20, 6, 256, 384), "tile": (100, 5, 384, 272), "wide": (1024, 9, 256, 3200)}
DOWN = {"stream": (24, 6, 512, 384), "tile": (100, 5, 512, 264), "wide": (128, 40, 5120, 256)}


def _code(dt):
    return L.DMOE_FP8_E4M3 if dt == "fp8" else L.DMOE_BF16


def _kernel(dt, gateup, M, E_loc, H, F):
    d = L.LayerDesc(M, H, F, 0, E_loc, E_loc, 0, 1, 0, _code(dt), 1)
    return dm.dmoe_forward_gateup_kernel(d) if gateup else dm.dmoe_forward_down_kernel(d)


def _rows(rng, per, E_loc):
    # ragged expert sizes around `per` (one expert left empty when there are several), total E_loc * per
    counts = rng.multinomial(per * E_loc - per, np.ones(E_loc - 1) / (E_loc - 1)) if E_loc > 1 else np.array([])
    counts = np.concatenate([[per], counts]).astype(np.int64)
    if E_loc > 2:
        counts[1] += counts[2]
        counts[2] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return offsets, int(offsets[-1])


def _as_dtype(v, dt):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return (t.to(torch.float8_e4m3fn).view(torch.uint8) if dt == "fp8" else t.to(torch.bfloat16)).to(DEV)


def _bf16_of(v64: np.ndarray) -> np.ndarray:
    # integers below 2^24: the float32 cast is exact, so this is one rounding to nearest even
    return torch.from_numpy(v64).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy()


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("regime", list(GATEUP))
def test_gateup_is_exact_on_integer_operands(dt, regime):
    per, E_loc, H, F = GATEUP[regime]
    rng = np.random.default_rng(zlib.crc32(f"gateup {dt} {regime}".encode()))
    offsets, M = _rows(rng, per, E_loc)
    assert _kernel(dt, True, M, E_loc, H, F) == f"gemm_{'stage' if regime == 'stream' else regime}_kernel"
    fpad = -(-F // 128) * 128
    a = np.zeros((M, H), np.float32)
    for r in range(M):
        a[r, rng.choice(H, 128, replace=False)] = 1.0
    wg = np.zeros((E_loc, fpad, H), np.float32)
    wg[:, :F] = rng.integers(0, 2, (E_loc, F, H))
    wu = np.zeros((E_loc, fpad, H), np.float32)
    for e in range(E_loc):
        for j in range(F):
            wu[e, j, rng.choice(H, 2, replace=False)] = rng.choice([-1.0, 1.0], 2)
    want = np.zeros((M, F), np.float64)
    for e in range(E_loc):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        g = a[r0:r1].astype(np.float64) @ wg[e, :F].T.astype(np.float64)
        u = a[r0:r1].astype(np.float64) @ wu[e, :F].T.astype(np.float64)
        assert r1 == r0 or (g.min() >= 17 and g.max() <= 128), "gate sums outside [17, 128]"
        want[r0:r1] = g * u
    scales = {}
    if dt == "fp8":
        ones = lambda *s: torch.ones(s, dtype=torch.float32, device=DEV)  # noqa: E731
        scales = dict(a_s=ones(M, H // 128), sg=ones(E_loc, -(-F // 128), H // 128),
                      su=ones(E_loc, -(-F // 128), H // 128))
    h = torch.empty((M, fpad), dtype=torch.bfloat16, device=DEV)
    dm.dmoe_grouped_gemm_gateup(_code(dt), _as_dtype(a, dt), scales.get("a_s"),
                                torch.arange(M, dtype=torch.int32, device=DEV),
                                torch.from_numpy(offsets).to(DEV), E_loc, M, _as_dtype(wg, dt), _as_dtype(wu, dt),
                                scales.get("sg"), scales.get("su"), H, F, h)
    torch.cuda.synchronize()
    got = h[:, :F].view(torch.int16).cpu().numpy()
    bad = int(np.count_nonzero(got != _bf16_of(want)))
    say(f"[gate/up {dt} {regime}] M={M} E_loc={E_loc} H={H} F={F}: {bad} BF16 h values differ")
    assert bad == 0


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("regime", list(DOWN))
def test_down_is_exact_on_integer_operands(dt, regime):
    per, E_loc, H, F = DOWN[regime]
    rng = np.random.default_rng(zlib.crc32(f"down {dt} {regime}".encode()))
    offsets, M = _rows(rng, per, E_loc)
    assert _kernel(dt, False, M, E_loc, H, F) == f"gemm_{'stage' if regime == 'stream' else regime}_kernel"
    fpad = -(-F // 128) * 128
    nk = -(-F // 128)
    h = np.zeros((M, fpad), np.float32)
    h[:, :F] = rng.integers(-15, 16, (M, F))
    wd = np.zeros((E_loc, H, fpad), np.float32)
    wd[:, :, :F] = rng.integers(-15, 16, (E_loc, H, F))
    if dt == "fp8":
        # power-of-two scales: per (row, 128-wide slice) of h and per 128 x 128 block of the weights
        hs = np.exp2(rng.integers(0, 3, (M, nk))).astype(np.float32)
        ws = np.exp2(rng.integers(0, 3, (E_loc, H // 128, nk))).astype(np.float32)
        hv = h[:, :F].astype(np.float64) * np.repeat(hs, 128, axis=1)[:, :F]
        wv = wd[:, :, :F].astype(np.float64) * np.repeat(np.repeat(ws, 128, axis=1), 128, axis=2)[:, :, :F]
    else:
        hv, wv = h[:, :F].astype(np.float64), wd[:, :, :F].astype(np.float64)
    want = np.zeros((M, H), np.float64)
    for e in range(E_loc):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        want[r0:r1] = hv[r0:r1] @ wv[e].T
    assert np.abs(want).max() < 2 ** 24
    o = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    hs_t = torch.from_numpy(hs).to(DEV) if dt == "fp8" else None
    ws_t = torch.from_numpy(ws).to(DEV) if dt == "fp8" else None
    dm.dmoe_grouped_gemm_down(_code(dt), _as_dtype(h, dt), hs_t, torch.from_numpy(offsets).to(DEV), E_loc, M,
                              _as_dtype(wd, dt), ws_t, F, H, o)
    torch.cuda.synchronize()
    got = o.view(torch.int16).cpu().numpy()
    bad = int(np.count_nonzero(got != _bf16_of(want)))
    say(f"[down {dt} {regime}] M={M} E_loc={E_loc} H={H} F={F}: {bad} BF16 o values differ")
    assert bad == 0
