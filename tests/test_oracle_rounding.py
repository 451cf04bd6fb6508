"""Pins of the oracle's rounding-straddle allowance (no GPU).

The layer rounds each expert output to bfloat16 before the weighted sum. An exact value that lies on a rounding
midpoint, within float32 precision, may be rounded to either neighbour by a correct float32 evaluation; the
oracle's ``bf16_midpoint_straddle`` flags such values and ``rounding_allowance`` sums, per output element, the
weight times the bfloat16 spacing of the flagged expert outputs. The pins define a straddle independently: v
straddles when torch's round-to-nearest-even bfloat16 cast of v (1 - 2^-18) differs from that of v (1 + 2^-18).
"""
import numpy as np
import torch

import oracle

REL = 2.0 ** -18


def _torch_bf16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _torch_straddle(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, np.float64)
    return _torch_bf16(v * (1 - REL)) != _torch_bf16(v * (1 + REL))


def test_spacing_is_the_gap_between_bracketing_bf16_values():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    lo = _torch_bf16(v)
    # the neighbour on the other side of v, found by stepping the float32 bits of the rounded value
    bits = torch.from_numpy(lo.astype(np.float32)).view(torch.int32).numpy().astype(np.int64)
    step = np.where((np.abs(v) > np.abs(lo)), 1, -1) << 16
    other = torch.from_numpy((bits + step).astype(np.int32)).view(torch.float32).numpy().astype(np.float64)
    gap = np.abs(other - lo)
    np.testing.assert_array_equal(oracle.bf16_spacing(v), gap)


def test_straddle_matches_the_cast_definition():
    rng = np.random.default_rng(2)
    # values on exact midpoints, nudged by up to 2^-19 (straddle) or by 2^-16 .. 2^-10 (decided)
    a = _torch_bf16(rng.standard_normal(5000) * np.exp2(rng.integers(-20, 20, 5000)))
    mid = a + np.sign(a) * oracle.bf16_spacing(a) / 2
    near = mid * (1 + rng.uniform(-2.0 ** -19, 2.0 ** -19, a.size))
    far = mid * (1 + np.sign(rng.standard_normal(a.size)) * np.exp2(rng.uniform(-16, -10, a.size)))
    rand = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    for v in (mid, near, far, rand, a):
        np.testing.assert_array_equal(oracle.bf16_midpoint_straddle(v), _torch_straddle(v))
    assert oracle.bf16_midpoint_straddle(near).all() and not oracle.bf16_midpoint_straddle(far).any()
    assert not oracle.bf16_midpoint_straddle(a).any()  # bfloat16 values themselves are decided
    assert not oracle.bf16_midpoint_straddle(np.zeros(3)).any()


def test_rounding_allowance_by_loops():
    # 4 routed rows, 2 tokens, K = 2, one shared-expert token; some exact outputs on midpoints
    one_mid = 1 + 2.0 ** -8            # midpoint between 1 and 1 + 2^-7
    big_mid = 2.4296875                # midpoint between 2.421875 and 2.4375
    o_exact = np.array([[one_mid, 0.3], [0.7, -big_mid], [0.25, 0.5], [-one_mid * 0.5, 1.0]])
    s_exact = np.array([[big_mid * (1 + 2.0 ** -24), 0.1], [0.0, 0.0]])
    token_row = np.array([[0, 3], [2, -1]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [1.0, 0.0]], dtype=np.float32)
    got = oracle.rounding_allowance(o_exact, token_row, w, s_exact, 1)
    want = np.zeros((2, 2))
    for t in range(2):
        for k in range(2):
            r = token_row[t, k]
            if r < 0:
                continue
            for c in range(2):
                if _torch_straddle(o_exact[r, c]):
                    want[t, c] += abs(float(w[t, k])) * oracle.bf16_spacing(o_exact[r, c])
        if t < 1:
            for c in range(2):
                if _torch_straddle(s_exact[t, c]):
                    want[t, c] += oracle.bf16_spacing(s_exact[t, c])
    np.testing.assert_array_equal(got, want)
    # token 0, column 0: o row 0 (weight 0.75, spacing 2^-7), o row 3 (0.25, spacing 2^-8), shared (2^-6)
    assert got[0, 0] == 0.75 * 2.0 ** -7 + 0.25 * 2.0 ** -8 + 2.0 ** -6
    assert got[0, 1] == 0.0 and got[1, 0] == 0.0 and got[1, 1] == 0.0


def _torch_straddle_band(v: np.ndarray, band: np.ndarray) -> np.ndarray:
    """A midpoint lies within max(2^-18 |v|, band) of v: the bfloat16 casts of the interval's ends differ."""
    v = np.asarray(v, np.float64)
    b = np.maximum(REL * np.abs(v), band)
    return _torch_bf16(v - b) != _torch_bf16(v + b)


def test_straddle_band_matches_the_cast_definition():
    rng = np.random.default_rng(3)
    a = _torch_bf16(rng.standard_normal(8000) * np.exp2(rng.integers(-10, 10, 8000)))
    u = oracle.bf16_spacing(a)
    mid = a + np.sign(a) * u / 2
    # distance to the midpoint as a fraction of the spacing, and bands on either side of it
    frac = rng.uniform(1e-4, 0.4, a.size)
    v = mid + np.sign(rng.standard_normal(a.size)) * frac * u
    inside = frac * u * rng.uniform(1.01, 3.0, a.size)
    outside = frac * u * rng.uniform(0.2, 0.99, a.size)
    for band in (inside, outside, np.zeros(a.size)):
        np.testing.assert_array_equal(oracle.bf16_midpoint_straddle(v, band=band), _torch_straddle_band(v, band))
    assert oracle.bf16_midpoint_straddle(v, band=inside).all()
    far = frac > 1e-3  # further than 2^-18 |v| from the midpoint
    assert not oracle.bf16_midpoint_straddle(v[far], band=outside[far]).any()


def test_abs_terms_by_loops():
    rng = np.random.default_rng(4)
    H, F, n = 128, 136, 3
    a = np.round(rng.standard_normal((n, H)) * 64) / 64  # exact in bfloat16
    wg = rng.standard_normal((F, H)) / 16
    wu = rng.standard_normal((F, H)) / 16
    wd = rng.standard_normal((H, F)) / 16
    for fp8 in (False, True):
        o, ab = oracle.swiglu_expert(a, wg, wu, wd, fp8, rounded=False, abs_terms=True)
        # h as the projection reads it: the same expert with an identity down projection
        h = oracle.swiglu_expert(a, wg, wu, np.eye(F), fp8, rounded=False)
        want = np.zeros((n, H))
        for i in range(n):
            for j in range(H):
                want[i, j] = sum(abs(h[i, k]) * abs(wd[j, k]) for k in range(F))
        np.testing.assert_allclose(ab, want, rtol=1e-12, atol=0)
        np.testing.assert_array_equal(o, oracle.swiglu_expert(a, wg, wu, wd, fp8, rounded=False))
        assert np.all(ab >= np.abs(o) * (1 - 1e-12)) and np.any(ab > np.abs(o) * 1.5)


def test_rounding_allowance_with_bands_by_loops():
    # the loop-form allowance with absolute bands for the routed and the shared outputs
    one_mid = 1 + 2.0 ** -8
    o_exact = np.array([[one_mid + 3e-4, 0.3], [0.7, -2.4296875], [0.25, 0.5], [-one_mid * 0.5, 1.0]])
    o_band = np.array([[5e-4, 0.0], [0.0, 0.0], [0.0, 0.0], [1e-9, 0.0]])
    s_exact = np.array([[2.4296875 + 2e-3, 0.1], [0.0, 0.0]])
    s_band = np.array([[1e-3, 0.0], [0.0, 0.0]])
    token_row = np.array([[0, 3], [2, 1]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]], dtype=np.float32)
    got = oracle.rounding_allowance(o_exact, token_row, w, s_exact, 1, o_band, s_band)
    want = np.zeros((2, 2))
    for t in range(2):
        for k in range(2):
            r = token_row[t, k]
            for c in range(2):
                if _torch_straddle_band(o_exact[r, c], o_band[r, c]):
                    want[t, c] += abs(float(w[t, k])) * oracle.bf16_spacing(o_exact[r, c])
        if t < 1:
            for c in range(2):
                if _torch_straddle_band(s_exact[t, c], s_band[t, c]):
                    want[t, c] += oracle.bf16_spacing(s_exact[t, c])
    np.testing.assert_array_equal(got, want)
    # row 0 is 3e-4 from its midpoint (inside its 5e-4 band); the shared output is 2e-3 from its midpoint,
    # outside its 1e-3 band; row 3 sits on its midpoint; row 1's -2.4296875 is a midpoint (weight 0.5)
    assert got[0, 0] == 0.75 * 2.0 ** -7 + 0.25 * 2.0 ** -8
    assert got[1, 1] == 0.5 * 2.0 ** -6 and got[0, 1] == 0.0 and got[1, 0] == 0.0


def test_fp8_layer_allowance_uses_the_matrix_core_band():
    # a tiny FP8 layer: y_allow equals the allowance built from each expert's exact outputs and the band
    # FP8_MMA_REL x (sum of absolute products), for the routed rows and the shared rows alike
    import synth
    cfg = synth.LayerConfig("allow_fp8", T=40, H=256, F=136, F_s=136, E=6, E_loc=4, e0=1, K=2, dtype="fp8",
                            T_s=25, logits="uniform")
    x_bits = synth.x_bf16(cfg)
    get = lambda which, e: synth.expert_weight_f32(cfg, which, e)  # noqa: E731
    ref = oracle.moe_forward(cfg, x_bits, get, logits=synth.given_logits(cfg))
    offsets, row_token, _, token_row = oracle.permute(ref.ids, cfg.e0, cfg.E_loc)
    xq, xs = oracle.quantize_act(oracle.bf16_to_f64(x_bits))
    a = oracle.dequantize_act(xq, xs)

    def expert(e, rows):
        wg, wu, wd = (oracle.dequantize_weight_blocks(*oracle.quantize_weight_blocks(get(w, e)))
                      for w in ("gate", "up", "down"))
        return oracle.swiglu_expert(a[rows], wg, wu, wd, True, rounded=False, abs_terms=True)
    M = int(offsets[-1])
    o, ob = np.zeros((M, cfg.H)), np.zeros((M, cfg.H))
    for el in range(cfg.E_loc):
        r0, r1 = int(offsets[el]), int(offsets[el + 1])
        if r1 > r0:
            o[r0:r1], ob[r0:r1] = expert(cfg.e0 + el, row_token[r0:r1])
    s, sb = np.zeros((cfg.T, cfg.H)), np.zeros((cfg.T, cfg.H))
    s[:cfg.T_s], sb[:cfg.T_s] = expert(-1, np.arange(cfg.T_s))
    want = oracle.rounding_allowance(o, token_row, ref.w, s, cfg.T, oracle.FP8_MMA_REL * ob,
                                     oracle.FP8_MMA_REL * sb)
    np.testing.assert_array_equal(ref.y_allow, want)
    narrow = oracle.rounding_allowance(o, token_row, ref.w, s, cfg.T)
    assert np.all(ref.y_allow >= narrow) and np.count_nonzero(ref.y_allow) > np.count_nonzero(narrow)
