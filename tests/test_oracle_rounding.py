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
