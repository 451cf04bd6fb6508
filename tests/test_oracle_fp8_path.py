"""Pins for the oracle's FP8 layer path: the requantisation of h before the down
projection, and the quantised x that feeds both the routed and the shared expert.

Fine-grained FP8 (Transformers PR #47844, implementation list: E4M3 weights in
128x128 blocks, dynamically quantised activations) quantises every activation
that enters an FP8 GEMM; the down projection's input is h, so h is quantised
per 1x128 slice after its BF16 rounding. The expected values here are built
with torch (float64 matmuls, torch's float32 division and its float8_e4m3fn
cast), not with the oracle's own table encoder; the hand-made cases fix the
result of each step to an exact number (no GPU)."""
import numpy as np
import torch
import torch.nn.functional as Fn

import oracle
import synth


def _bf16(t64: torch.Tensor) -> torch.Tensor:
    """Round float64 values to bfloat16 through float32 (exact unless float32 lands on a bfloat16 midpoint)."""
    return t64.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _double_rounding_risk(t64: torch.Tensor) -> torch.Tensor:
    """Elements whose float32 rounding is inexact and lands exactly halfway between two bfloat16 values: there
    the two-step cast above may differ from a direct rounding, so such elements are left out of bitwise
    comparisons."""
    f = t64.to(torch.float32)
    b = f.view(torch.int32)
    return ((b & 0xFFFF) == 0x8000) & (f.to(torch.float64) != t64)


def _torch_quant_dequant(v64: torch.Tensor, width: int = 128) -> torch.Tensor:
    """Per row, per `width`-column slice: s = float32(amax) / 448 (torch float32 division), codes by torch's
    float8_e4m3fn cast of float32(v / s) (all quotients are <= 448 in magnitude up to one float32 ulp, which
    the cast rounds to 448), values code * s; a zero slice stays zero."""
    v32 = v64.to(torch.float32)
    out = torch.zeros_like(v64)
    for j in range(0, v32.shape[1], width):
        sl = v32[:, j:j + width]
        s = sl.abs().amax(dim=1, keepdim=True) / torch.tensor(448.0, dtype=torch.float32)
        safe = torch.where(s == 0, torch.ones_like(s), s)
        q = (sl / safe).to(torch.float8_e4m3fn)
        out[:, j:j + width] = torch.where(s == 0, torch.zeros_like(s, dtype=torch.float64),
                                          q.to(torch.float64) * s.to(torch.float64))
    return out


def _torch_block_quant_dequant(w32: np.ndarray) -> torch.Tensor:
    """128x128 weight blocks with the same rule (amax over the block's valid elements)."""
    w = torch.from_numpy(np.asarray(w32, np.float32))
    out = torch.zeros(w.shape, dtype=torch.float64)
    for i in range(0, w.shape[0], 128):
        for j in range(0, w.shape[1], 128):
            blk = w[i:i + 128, j:j + 128]
            s = blk.abs().amax() / torch.tensor(448.0, dtype=torch.float32)
            q = (blk / s).to(torch.float8_e4m3fn)
            out[i:i + 128, j:j + 128] = q.to(torch.float64) * s.to(torch.float64)
    return out


def _torch_fp8_expert(a, wg, wu, wd):
    """down(q(bf16(silu(a Wg^T) * (a Wu^T)))) rounded to bfloat16, with q = 1x128 quantise-dequantise."""
    h = _bf16(Fn.silu(Fn.linear(a, wg)) * Fn.linear(a, wu))
    return _bf16(Fn.linear(_torch_quant_dequant(h), wd)), h


def test_fp8_expert_requantises_bf16_h_like_torch():
    """swiglu_expert(fp8=True) against an independent torch construction on a random expert whose width has a
    partial last slice (F = 200: slices of 128 and 72 columns). Bitwise, except where the torch side's two-step
    bfloat16 cast could round twice."""
    rng = np.random.default_rng(11)
    n, H, F = 12, 256, 200
    a = oracle.bf16_round(rng.standard_normal((n, H)))
    wg, wu = (oracle.bf16_round(rng.standard_normal((F, H)) / 16) for _ in range(2))
    wd = oracle.bf16_round(rng.standard_normal((H, F)) / 14)
    got = oracle.swiglu_expert(a, wg, wu, wd, fp8=True)
    ta, tg, tu, td = (torch.from_numpy(v) for v in (a, wg, wu, wd))
    ref, h = _torch_fp8_expert(ta, tg, tu, td)
    h64 = Fn.silu(Fn.linear(ta, tg)) * Fn.linear(ta, tu)
    assert not bool(_double_rounding_risk(h64).any()), "pick another seed: h has a double-rounding case"
    o64 = Fn.linear(_torch_quant_dequant(h), td)
    ok = ~_double_rounding_risk(o64).numpy()
    assert ok.mean() > 0.99
    np.testing.assert_array_equal(got[ok], ref.numpy()[ok])
    # the FP8 step is a real change of h: without it most outputs differ
    plain = oracle.swiglu_expert(a, wg, wu, wd, fp8=False)
    assert np.mean(plain != got) > 0.5


def _constructed_expert(h0: float):
    """One token, H = F = 128: a = e_0, every gate row has 64 in column 0 (silu(64) == 64 in float64), so
    h = 64 * u. Up rows give h[0] = h0 and h[1] = 448 (the slice's amax, so its scale is exactly 1);
    down picks o[0] = h[0] and o[1] = h[1] / 448."""
    H = F = 128
    a = np.zeros((1, H))
    a[0, 0] = 1.0
    wg = np.zeros((F, H))
    wg[:, 0] = 64.0
    wu = np.zeros((F, H))
    wu[0, 0] = h0 / 64.0
    wu[1, 0] = 448.0 / 64.0
    wd = np.zeros((H, F))
    wd[0, 0] = 1.0
    wd[1, 1] = 1.0 / 448.0
    return a, wg, wu, wd


def test_fp8_h_step_constructed_values():
    """h[0] = 1.0625 is the midpoint of the E4M3 values 1.0 and 1.125 at scale 1: round-to-nearest-even gives
    1.0 (even code 0x38). With the step the expert outputs 1.0; without it 1.0625 (a margin of 1/16)."""
    a, wg, wu, wd = _constructed_expert(1.0625)
    o = oracle.swiglu_expert(a, wg, wu, wd, fp8=True)
    assert o[0, 0] == 1.0 and o[0, 1] == 1.0
    assert oracle.swiglu_expert(a, wg, wu, wd, fp8=False)[0, 0] == 1.0625


def test_fp8_h_step_quantises_after_bf16_rounding():
    """h[0] = 1.0625 + 2^-12 rounds to the bfloat16 value 1.0625 (a tie in E4M3, to 1.0); quantising the
    unrounded value instead would give 1.125. The oracle must take the BF16 rounding first."""
    a, wg, wu, wd = _constructed_expert(1.0625 + 2.0 ** -12)
    o = oracle.swiglu_expert(a, wg, wu, wd, fp8=True)
    assert o[0, 0] == 1.0
    assert oracle.swiglu_expert(a, wg, wu, wd, fp8=False)[0, 0] == 1.0625


def test_fp8_layer_one_expert_matches_torch():
    """E = 1, K = 1 FP8 layer with the shared expert on every token: y = bf16(o_0 + s), where both experts take
    the 1x128-quantised x and 128x128 block-quantised weights and requantise their BF16 h, all built in torch.
    This pins the FP8 x path into the routed and the shared expert together."""
    cfg = synth.LayerConfig("one_fp8", T=10, H=256, F=200, F_s=136, E=1, E_loc=1, e0=0, K=1,
                            dtype="fp8", T_s=10, logits="single")
    x = synth.x_bf16(cfg)
    get = lambda w, e: synth.expert_weight_f32(cfg, w, e)  # noqa: E731
    res = oracle.moe_forward(cfg, x, get, logits=synth.given_logits(cfg))
    np.testing.assert_array_equal(res.w, 1.0)
    xa = _torch_quant_dequant(torch.from_numpy(oracle.bf16_to_f64(x)))
    W = {(w, e): _torch_block_quant_dequant(get(w, e)) for w in ("gate", "up", "down") for e in (0, -1)}
    o, _ = _torch_fp8_expert(xa, W["gate", 0], W["up", 0], W["down", 0])
    s, _ = _torch_fp8_expert(xa, W["gate", -1], W["up", -1], W["down", -1])
    y64 = o + s
    ref = _bf16(y64)
    ok = ~_double_rounding_risk(y64).numpy()
    assert ok.mean() > 0.99
    np.testing.assert_array_equal(res.y[ok], ref.numpy()[ok])
    # the shared expert's input is the quantised x, not the BF16 x: feeding it BF16 x changes the output
    s_bf, _ = _torch_fp8_expert(torch.from_numpy(oracle.bf16_to_f64(x)), W["gate", -1], W["up", -1],
                                W["down", -1])
    assert np.mean(_bf16(o + s_bf).numpy() != res.y) > 0.3
