"""Pins for the oracle's number formats: E4M3FN codes, the activation / weight
quantisers and BF16 rounding, checked against format facts, torch's own casts
and exact constructions (no GPU)."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_table_format_facts():
    v = oracle.e4m3_values()
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) == -1
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0           # largest finite
    assert v[0x01] == 2.0 ** -9                              # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6  # subnormal/normal boundary
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:127]) > 0)                      # positive codes ascend
    np.testing.assert_array_equal(v[128:255], -v[:127])


def test_e4m3_table_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = oracle.e4m3_values()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(v))
    np.testing.assert_array_equal(t[~np.isnan(t)], v[~np.isnan(v)])


def _torch_e4m3(v32):
    return torch.from_numpy(np.ascontiguousarray(v32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(400_000) * np.exp2(rng.integers(-16, 9, 400_000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    np.testing.assert_array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_midpoints_round_to_even():
    pos = oracle.e4m3_values()[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # all exactly representable in float32
    codes = oracle.e4m3_encode(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(codes, expect)
    np.testing.assert_array_equal(codes, _torch_e4m3(mids))
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    np.testing.assert_array_equal(oracle.e4m3_encode(up), lo + 1)
    np.testing.assert_array_equal(oracle.e4m3_encode(dn), lo)
    np.testing.assert_array_equal(oracle.e4m3_encode(-mids), expect | 0x80)


def test_e4m3_encode_saturates_and_keeps_sign():
    big = np.array([448.0, 448.5, 463.9, 464.0, 1e6, 3.0e38], dtype=np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(big), 0x7E)
    np.testing.assert_array_equal(oracle.e4m3_encode(-big), 0xFE)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.array([0.0, -0.0, -1e-30, 1e-30], np.float32)),
                                  [0x00, 0x80, 0x80, 0x00])


def test_e4m3_exhaustive_bf16_times_scales():
    """Every finite BF16 pattern x, divided by several scales in float32, against torch."""
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << np.uint32(16)).view(np.float32)
    x = x[np.isfinite(x)]
    for s in (np.float32(2.0 ** -3), np.float32(1.0), np.float32(2.0 ** 5), np.float32(0.0123456)):
        with np.errstate(over="ignore"):
            q = (x / s).astype(np.float32)
        q = q[np.isfinite(q)]
        ours = oracle.e4m3_encode(q)
        inr = np.abs(q) <= 448
        np.testing.assert_array_equal(ours[inr], _torch_e4m3(q[inr]))
        np.testing.assert_array_equal(ours[~inr] & 0x7F, 0x7E)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(200_000) * np.exp2(rng.integers(-130, 60, 200_000))).astype(np.float32)
    ties = ((np.arange(1, 5000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.array([0.0, -0.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(v.astype(np.float64)), ref)


def test_bf16_to_f64_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        o = oracle.bf16_to_f64(bits)
    fin = np.isfinite(t)
    np.testing.assert_array_equal(o[fin], t[fin])


# --- activation / weight quantisers -------------------------------------------------------

def _e4m3_sample(rng, shape):
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
    return codes


@pytest.mark.parametrize("cols", [128, 512, 1400, 5120, 40])
def test_quantize_act_exact_round_trip(cols):
    """x = 2^j * v with v on the E4M3 grid and one |v| = 448 per slice: s = 2^j exactly, codes recover v."""
    rng = np.random.default_rng(cols)
    rows = 6
    codes = _e4m3_sample(rng, (rows, cols))
    nb = -(-cols // 128)
    for j in range(nb):
        codes[:, j * 128] = 0x7E if j % 2 == 0 else 0xFE  # amax 448 in every slice
    vals = oracle.e4m3_values()[codes]
    exps = rng.integers(-20, 10, size=(rows, nb))
    scale = np.repeat(np.exp2(exps.astype(np.float64)), 128, axis=1)[:, :cols]
    x = (vals * scale).astype(np.float32)
    q, s = oracle.quantize_act(x)
    np.testing.assert_array_equal(s, np.exp2(exps).astype(np.float32))
    nz = vals != 0  # the sign of an exact zero follows x, compare magnitudes there
    np.testing.assert_array_equal(q[nz], codes[nz])
    np.testing.assert_array_equal(q[~nz] & 0x7F, 0)
    assert s.shape == (rows, nb)


def test_quantize_act_zero_and_tiny_slices():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 128:] = np.float32(-1e-30)
    x[1, 130] = np.float32(3.0)
    q, s = oracle.quantize_act(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert q[1, 130] == 0x7E and q[1, 129] == 0x80  # tiny negative keeps its sign


def test_quantize_act_scale_is_float32_division():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    q, s = oracle.quantize_act(x)
    for j in range(3):
        sl = x[:, j * 128:(j + 1) * 128]
        amax = np.abs(sl).max(axis=1)
        ref = torch.from_numpy(amax) / torch.tensor(448.0, dtype=torch.float32)
        np.testing.assert_array_equal(s[:, j], ref.numpy())
        qq = torch.from_numpy(sl) / torch.from_numpy(s[:, j:j + 1])
        inr = qq.abs() <= 448
        np.testing.assert_array_equal(q[:, j * 128:(j + 1) * 128][inr.numpy()],
                                      qq[inr].to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_quantize_weight_blocks_partial_blocks():
    """1400 columns and 300 rows: edge blocks take the amax over their valid elements only."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((300, 1400)) * 0.01).astype(np.float32)
    w[256 + 3, 1280 + 7] = np.float32(0.75)   # the only large value in the corner block (44 x 120)
    q, s = oracle.quantize_weight_blocks(w)
    assert s.shape == (3, 11)
    assert s[2, 10] == np.float32(0.75) / np.float32(448.0)
    assert q[259, 1287] == 0x7E
    for (bi, bj) in [(0, 0), (1, 10), (2, 3)]:
        blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
        assert s[bi, bj] == np.float32(np.abs(blk).max()) / np.float32(448.0)
    deq = oracle.dequantize_weight_blocks(q, s)
    rel = np.abs(deq - w) / np.repeat(np.repeat(s, 128, 0), 128, 1)[:300, :1400]
    assert rel.max() <= 16.0  # at most half an E4M3 step (<= 16 at the top binade) in scale units


def test_quantize_weight_blocks_exact_round_trip():
    rng = np.random.default_rng(9)
    codes = _e4m3_sample(rng, (200, 300))
    for i in range(2):
        for j in range(3):
            codes[i * 128, j * 128] = 0x7E
    exps = rng.integers(-12, 3, size=(2, 3))
    sc = np.repeat(np.repeat(np.exp2(exps.astype(np.float64)), 128, 0), 128, 1)[:200, :300]
    w = (oracle.e4m3_values()[codes] * sc).astype(np.float32)
    q, s = oracle.quantize_weight_blocks(w)
    np.testing.assert_array_equal(s, np.exp2(exps).astype(np.float32))
    nz = oracle.e4m3_values()[codes] != 0
    np.testing.assert_array_equal(q[nz], codes[nz])


def test_fp8_block_gemm_exact_integer_sums():
    """Dequantise-then-float64 matmul equals per-block exact int64 sums scaled once.

    E4M3 values are multiples of 2^-9, so code values times 2^9 are integers
    and each 128-wide block's dot product is an exact int64 sum.
    """
    rng = np.random.default_rng(13)
    T, H, F = 7, 300, 200  # partial blocks on both dims
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((F, H)) / np.sqrt(H)).astype(np.float32)
    qa, sa = oracle.quantize_act(x)
    qw, sw = oracle.quantize_weight_blocks(w)
    got = oracle.dequantize_act(qa, sa) @ oracle.dequantize_weight_blocks(qw, sw).T
    ia = np.rint(oracle.e4m3_values()[qa] * 512).astype(np.int64)
    iw = np.rint(oracle.e4m3_values()[qw] * 512).astype(np.int64)
    ref = np.zeros((T, F))
    for t in range(T):
        for f in range(F):
            acc = 0.0
            for j in range(-(-H // 128)):
                ks = slice(j * 128, (j + 1) * 128)
                blk = int(np.dot(ia[t, ks], iw[f, ks]))
                acc += blk * float(sa[t, j]) * float(sw[f // 128, j]) * 2.0 ** -18
            ref[t, f] = acc
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
