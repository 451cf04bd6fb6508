"""Per-kernel parity of libdmoe against the CPU oracle (GPU).

Integer and byte results (top-K ids, permutation tables, FP8 codes and
scales) must be bit-exact; floating-point results must be within the stated
tolerances."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LOGIT_TOL, W_TOL, bf16_bits, bf16_values, say, to_dev_bf16

pytestmark = pytest.mark.gpu

import fp8_expert_ffn_amd as dm  # noqa: E402


# --------------------------------------------------------------------------- route

def _route_case(L: np.ndarray, K: int):
    say(f"route T={L.shape[0]} E={L.shape[1]} K={K}")
    ids, w = dm.dmoe_route(torch.from_numpy(L).to(DEV), K)
    ids_r, w_r = oracle.route(L, K)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_r)
    w = w.cpu().numpy()
    assert np.max(np.abs(w.astype(np.float64) - w_r)) <= W_TOL
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 1.0)) <= W_TOL


@pytest.mark.parametrize("E,K", [(256, 8), (16, 4), (7, 7), (1024, 64), (100, 1), (65, 3)])
def test_route_random_and_adversarial(E, K):
    rng = np.random.default_rng(E + K)
    L = (rng.standard_normal((333, E)) * 1.43).astype(np.float32)
    L[0] = 0.0                                               # all equal
    L[1] = np.where(np.arange(E) % 2 == 0, 0.0, -0.0)        # signed zeros
    L[2] = np.repeat(rng.standard_normal(E // 4 + 1), 4)[:E]  # ties in groups
    L[3] = np.round(rng.standard_normal(E) * 2)              # many integer ties
    L[4, -1] = L[4, -2] = L[4].max() + 1                     # duplicated maximum at the end
    L[5] = -np.arange(E, dtype=np.float32)                   # strictly decreasing
    L[6] = np.float32(-3e38)
    _route_case(L, K)


@pytest.mark.parametrize("ci", [3, 4])
def test_route_full_size_given_logits(ci):
    cfg = synth.config(ci)
    _route_case(synth.given_logits(cfg), cfg.K)


@pytest.mark.parametrize("E,K,G,TG,renorm,scale", [(256, 8, 8, 4, True, 1.0), (256, 8, 8, 4, False, 2.5),
                                                     (64, 6, 16, 3, True, 1.0), (64, 4, 64, 6, False, 1.0),
                                                     (1024, 16, 32, 5, True, 0.75), (96, 8, 4, 1, True, 1.0),
                                                     (256, 8, 1, 1, False, 1.0)])
def test_route_grouped(E, K, G, TG, renorm, scale):
    say(f"route grouped E={E} K={K} n_group={G} topk_group={TG} renormalize={renorm} scaling={scale}")
    rng = np.random.default_rng(E + 7 * G + TG)
    L = (rng.standard_normal((257, E)) * 1.43).astype(np.float32)
    L[0] = 0.0                                               # all equal: lower groups, lower experts
    L[1] = np.repeat(rng.standard_normal(E // 8), 8)[:E]     # equal values inside groups of 8
    L[2] = np.round(rng.standard_normal(E) * 2)              # integer ties across groups
    ids, w = dm.dmoe_route_grouped(torch.from_numpy(L).to(DEV), K, G, TG, renorm, scale)
    ids_r, w_r = oracle.route(L, K, n_group=G, topk_group=TG, renormalize=renorm, scaling=scale)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_r)
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_r) / scale) <= W_TOL


@pytest.mark.parametrize("E,K,G,TG,renorm,scale,use_bias", [(256, 8, 8, 4, True, 2.5, True),
                                                              (256, 8, 1, 1, True, 1.0, True),
                                                              (64, 6, 16, 3, False, 1.0, True),
                                                              (64, 4, 64, 6, True, 1.0, False),
                                                              (1024, 16, 32, 5, True, 0.75, True)])
def test_route_sigmoid(E, K, G, TG, renorm, scale, use_bias):
    say(f"route sigmoid E={E} K={K} n_group={G} topk_group={TG} renormalize={renorm} scaling={scale} bias={use_bias}")
    rng = np.random.default_rng(E + 3 * G + TG)
    L = (rng.standard_normal((257, E)) * 2).astype(np.float32)
    L[0] = 0.0                                               # equal scores everywhere
    L[1] = np.round(rng.standard_normal(E) * 2)              # integer ties
    L[2, : E // 2] = 40.0                                    # saturated scores (s == 1.0 exactly)
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32) if use_bias else None
    ids, w = dm.dmoe_route_sigmoid(torch.from_numpy(L).to(DEV), K,
                                   torch.from_numpy(bias).to(DEV) if use_bias else None, G, TG, renorm, scale)
    ids_r, w_r = oracle.route_sigmoid(L, K, bias=bias, n_group=G, topk_group=TG, renormalize=renorm, scaling=scale)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_r)
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_r) / scale) <= W_TOL


def test_route_single_token():
    _route_case(np.array([[0.5, 2.0, -1.0, 2.0]], np.float32), 2)


# --------------------------------------------------------------------------- router logits

@pytest.mark.parametrize("T,H,E", [(128, 512, 16), (64, 5120, 256), (300, 1024, 72), (1, 128, 5)])
def test_router_logits(T, H, E):
    say(f"router_logits T={T} H={H} E={E}")
    cfg = synth.LayerConfig("r", T=T, H=H, F=128, F_s=0, E=E, E_loc=E, e0=0, K=1, dtype="bf16", T_s=0,
                            logits="router")
    x = synth.x_bf16(cfg)
    wr = synth.router_weight(cfg)
    L = dm.dmoe_router_logits(to_dev_bf16(x), torch.from_numpy(wr).to(DEV)).cpu().numpy()
    ref = oracle.router_logits(oracle.bf16_to_f64(x), wr)
    err = np.max(np.abs(L.astype(np.float64) - ref))
    say(f"  max |dL| = {err:.3e}")
    assert err <= LOGIT_TOL


def test_vision_router_near_ties_need_fp32():
    """Vision-router shape (hidden 1536, 64 experts, top-8) with experts in near-duplicate triples, so that the
    top-8 boundary (8 = 2 triples + 2) falls inside a triple whose logits are ~1e-3 apart. The FP32 router must
    pick exactly the oracle's experts wherever the decisive gap exceeds 4x the logit tolerance, while a router
    with BF16-rounded weights picks differently on some of those tokens (the precision the FP32 router exists
    for)."""
    T, H, E, K = 512, 1536, 64, 8
    rng = np.random.default_rng(2112)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02)
    for g in range(E // 3):  # experts 3g+1, 3g+2 are small perturbations of expert 3g
        for j in (1, 2):
            w[3 * g + j] = w[3 * g] + rng.standard_normal(H, dtype=np.float32) * np.float32(0.02 * 2.0 ** -10)
    x64 = oracle.bf16_to_f64(x)
    L_ref = oracle.router_logits(x64, w)
    ids_ref, _ = oracle.route(L_ref, K)
    L_gpu = dm.dmoe_router_logits(to_dev_bf16(x), torch.from_numpy(w).to(DEV))
    ids_gpu, _ = dm.dmoe_route(L_gpu, K)
    ids_gpu = ids_gpu.cpu().numpy()
    srt = np.sort(L_ref.astype(np.float64), axis=1)[:, ::-1]
    gap = srt[:, K - 1] - srt[:, K]
    robust = gap > 4 * LOGIT_TOL
    same = np.all(np.sort(ids_gpu, 1) == np.sort(ids_ref, 1), axis=1)
    say(f"  near-tie tokens (gap < 1e-3): {(gap < 1e-3).sum()}, robust {robust.sum()}, "
        f"GPU differs on {(~same).sum()} (all non-robust: {np.all(~robust[~same])})")
    assert np.all(same[robust])
    ids_bf, _ = oracle.route(oracle.router_logits(x64, synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(w))), K)
    bf_diff = ~np.all(np.sort(ids_bf, 1) == np.sort(ids_ref, 1), axis=1)
    say(f"  a BF16-weight router differs on {bf_diff.sum()} tokens, {(bf_diff & robust).sum()} of them robust")
    assert (bf_diff & robust).sum() > 0


# --------------------------------------------------------------------------- permute

def _permute_case(ids: np.ndarray, e0: int, e_loc: int):
    T, K = ids.shape
    say(f"permute T={T} K={K} e0={e0} E_loc={e_loc}")
    off, rt, rs, tr = dm.dmoe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), e0, e_loc)
    off_r, rt_r, rs_r, tr_r = oracle.permute(ids, e0, e_loc)
    off = off.cpu().numpy()
    np.testing.assert_array_equal(off, off_r)
    M = int(off_r[-1])
    np.testing.assert_array_equal(rt.cpu().numpy()[:M], rt_r)
    np.testing.assert_array_equal(rs.cpu().numpy()[:M], rs_r)
    np.testing.assert_array_equal(tr.cpu().numpy(), tr_r)


def test_permute_ep_share_full_size():
    cfg = synth.config(3)
    ids, _ = oracle.route(synth.given_logits(cfg), cfg.K)
    _permute_case(ids, cfg.e0, cfg.E_loc)
    _permute_case(ids, 224, 32)  # the coldest EP rank


@pytest.mark.parametrize("T,E,K,e0,E_loc", [(64, 256, 8, 0, 256), (8192, 256, 8, 0, 256), (1, 256, 8, 0, 256),
                                             (77, 16, 4, 4, 8), (1000, 1024, 3, 0, 1024), (513, 64, 1, 0, 64)])
def test_permute_shapes(T, E, K, e0, E_loc):
    rng = np.random.default_rng(T + E)
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), K)
    _permute_case(ids, e0, E_loc)


def test_permute_one_hot_expert_and_empty_experts():
    T, K = 700, 8
    ids = np.tile(np.arange(K), (T, 1))
    ids[:, 0] = 37  # every token hits expert 37; experts 8..36 and 38.. get nothing
    _permute_case(ids, 0, 64)


# --------------------------------------------------------------------------- quantisation

def _quant_case(x_bits: np.ndarray, cols=None):
    rows = x_bits.shape[0]
    cols = x_bits.shape[1] if cols is None else cols
    q, s = dm.dmoe_quant_act(to_dev_bf16(x_bits), cols)
    q_r, s_r = oracle.quantize_act(oracle.bf16_to_f64(x_bits[:, :cols]))
    q, s = q.cpu().numpy(), s.cpu().numpy()
    np.testing.assert_array_equal(s, s_r)
    np.testing.assert_array_equal(q[:, :cols], q_r)
    assert np.all(q[:, cols:] == 0)


# (2048, 5120) and (1009, 8312) take the launch with four slices per 16-lane group (>= 65536 slices); the latter
# ends in a partly filled workgroup and a 120-wide last slice
@pytest.mark.parametrize("rows,cols", [(2048, 5120), (1009, 8312), (33, 1400), (5, 40), (1, 128), (300, 1536)])
def test_quant_act_workload_values(rows, cols):
    say(f"quant_act {rows}x{cols}")
    cfg = synth.LayerConfig("q", T=rows, H=cols, F=8, F_s=0, E=1, E_loc=1, e0=0, K=1, dtype="fp8", T_s=0,
                            logits="uniform")
    _quant_case(synth.x_bf16(cfg))


def test_quant_act_exhaustive_bf16_patterns():
    """Every finite BF16 pattern, in slices whose amax fixes the scale, for several scales."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << np.uint32(16)).view(np.float32)
    finite = bits[np.isfinite(vals)].astype(np.uint16)
    for amax_bits in (0x7F7F, 0x43E0, 0x3F80, 0x3E00, 0x1B00, 0x0080):  # max finite, 448, 1, 0.125, tiny, min normal
        amax = float((np.uint32(amax_bits) << np.uint32(16)).view(np.float32))
        sel = finite[np.abs((finite.astype(np.uint32) << np.uint32(16)).view(np.float32)) <= amax]
        n = -(-sel.size // 127)
        block = np.zeros((n, 128), dtype=np.uint16)
        flat = np.zeros(n * 127, dtype=np.uint16)
        flat[:sel.size] = sel
        block[:, 1:] = flat.reshape(n, 127)
        block[:, 0] = amax_bits
        say(f"quant_act exhaustive amax=0x{amax_bits:04x}: {sel.size} patterns")
        _quant_case(block)


def test_quant_act_scale_sweep_all_patterns():
    """Scales across the whole exponent range (amax every 0x100 BF16 patterns, denormal to max finite), each with
    every BF16 value inside its slice range: the scaled quotient and its E4M3 code are bit-exact everywhere."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << np.uint32(16)).view(np.float32)
    finite = bits[np.isfinite(vals)].astype(np.uint16)
    fvals = (finite.astype(np.uint32) << np.uint32(16)).view(np.float32)
    blocks = []
    for amax_bits in list(range(0x0001, 0x7F80, 0x100)) + [0x7F7F]:
        amax = float((np.uint32(amax_bits) << np.uint32(16)).view(np.float32))
        sel = finite[np.abs(fvals) <= amax]
        n = -(-sel.size // 127)
        block = np.zeros((n, 128), dtype=np.uint16)
        flat = np.zeros(n * 127, dtype=np.uint16)
        flat[:sel.size] = sel
        block[:, 1:] = flat.reshape(n, 127)
        block[:, 0] = amax_bits
        blocks.append(block)
    x = np.concatenate(blocks)
    say(f"quant_act scale sweep: {len(blocks)} scales, {x.shape[0]} slices")
    _quant_case(x)


def test_quant_act_zero_and_sign_cases():
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, :] = 0x8000          # -0.0 everywhere: scale 0, all codes 0
    x[2, 128:] = 0x8001       # tiny negative denormals
    x[2, 130] = 0x4040        # 3.0
    _quant_case(x)


def test_quant_weight_blocks_partial():
    rng = np.random.default_rng(1)
    for rows, cols in [(300, 1400), (1536, 5120), (5120, 1400), (128, 128), (1, 4)]:
        say(f"quant_weight_blocks {rows}x{cols}")
        w = (rng.standard_normal((rows, cols)) / np.sqrt(cols)).astype(np.float32)
        q, s = dm.dmoe_quant_weight_blocks(torch.from_numpy(w).to(DEV))
        q_r, s_r = oracle.quantize_weight_blocks(w)
        q, s = q.cpu().numpy(), s.cpu().numpy()
        np.testing.assert_array_equal(s, s_r)
        np.testing.assert_array_equal(q[:rows, :cols], q_r)
        assert np.all(q[rows:] == 0) and np.all(q[:, cols:] == 0)


# --------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,K,H,T_s,local_frac", [(64, 8, 5120, 64, 1.0), (500, 8, 512, 100, 0.4), (3, 2, 128, 0, 1.0)])
def test_combine(T, K, H, T_s, local_frac):
    say(f"combine T={T} K={K} H={H} T_s={T_s}")
    rng = np.random.default_rng(T)
    ids, w = oracle.route(rng.standard_normal((T, 64)).astype(np.float32), K)
    e_loc = max(1, int(64 * local_frac))
    _, _, _, tr = oracle.permute(ids, 0, e_loc)
    M = int((tr >= 0).sum())
    o_bits = synth.f32_to_bf16_bits(rng.standard_normal((max(M, 1), H)).astype(np.float32))
    s_bits = synth.f32_to_bf16_bits(rng.standard_normal((max(T_s, 1), H)).astype(np.float32))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    s_dev = to_dev_bf16(s_bits) if T_s else None
    dm.dmoe_combine(to_dev_bf16(o_bits), torch.from_numpy(tr).to(DEV), torch.from_numpy(w).to(DEV), s_dev, T_s, H, y)
    o64, s64 = oracle.bf16_to_f64(o_bits), (oracle.bf16_to_f64(s_bits) if T_s else None)
    ref = oracle.combine(o64, tr, w, s64, T_s)
    y_sum = oracle.combine(o64, tr, w, s64, T_s, rounded=False)
    mag = oracle.combine(np.abs(o64), tr, np.abs(w), None if s64 is None else np.abs(s64), T_s, rounded=False)
    got = bf16_values(y)
    # FP32 accumulation of at most K + 1 terms, then one BF16 rounding of the FP32 sum
    a = np.maximum(np.abs(got), np.abs(y_sum))
    half_ulp = np.where(a > 0, np.ldexp(1.0, np.maximum(np.frexp(a)[1] - 9, -134)), 0.0)
    assert np.all(np.abs(got - y_sum) <= half_ulp + (K + 2) * 2.0 ** -24 * mag)
    assert np.mean(got == ref) > 0.99
