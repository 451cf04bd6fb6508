"""Plain, slow, obviously correct CPU oracle of the MoE layer (NumPy, FP64).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library.

What the layer computes, and where the pages fix it:

* Shape: 256 routed experts plus 1 shared expert, top-8, hidden 5120, expert
  FFN 1536 (model card "dots-studio/dots3-note-prev", Model Overview table;
  Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig: ``n_routed_experts``,
  ``n_shared_experts``, ``num_experts_per_tok``, ``moe_intermediate_size``,
  ``shared_experts_intermediate_size``).
* Router: token-choice top-k, ``norm_topk_prob`` true (renormalise the kept
  weights), ``routed_scaling_factor`` 1.0, ``n_group``/``topk_group`` 1 (no
  group-limited selection) (Dots3NoteTextConfig parameters); the router is
  ungrouped (orcarouter blog "dots-note-3.0 ...", section on the architecture
  the leak got right); routing runs in FP32 (Transformers PR #47844, list of
  what the implementation includes). The scoring function is not stated; the
  docs call the router output "post-softmax" in the conditional-generation
  forward's ``router_logits`` entry, so scores are a softmax over all experts.
* Expert: ``hidden_act`` silu with gate_proj, up_proj and down_proj and no
  bias (Dots3NoteTextConfig ``hidden_act``, ``mlp_bias``), i.e. a SwiGLU FFN
  ``down(silu(gate x) * up x)``. The shared expert has the same form and is
  added with weight 1.
* FP8: E4M3 weights with one scale per 128x128 weight block and dynamically
  quantised activations (PR #47844, implementation list), including weight
  dimensions that are not multiples of 128 ("partial weight blocks": PR #47844,
  Validation list and the authors' reply on the shared FP8 changes).

Readings where the pages are silent (each also listed in the design notes):

* Selection is on the FP32 logits (softmax is monotone); equal logits go to
  the lower expert index; -0.0 counts as +0.0; slots are ordered by rank.
* E4M3 is the OCP E4M3FN format (bias 7, largest finite 448, no infinities,
  0x7F/0xFF are NaN).
* Scale of a 1x128 activation slice or a 128x128 weight block:
  ``s = f32(amax / 448)``; codes ``q = E4M3_RNE(f32(v / s))`` with saturation to
  +-448; a block whose scale is 0 gets all-zero codes; the sign bit of the
  quotient is kept otherwise. Partial slices and blocks take the amax over their
  valid elements only.
* Rounding points: h = silu(g)*u is rounded to BF16 (and, on the FP8 path,
  that BF16 h is quantised like an activation); each expert output o is
  rounded to BF16; the layer output y is rounded to BF16 once, after the
  weighted sum of the routed outputs plus the shared output.
* Where an expert output's exact value lies on a BF16 rounding midpoint within
  float32 precision (2^-18 of its magnitude), both neighbours are correct
  roundings of it; ``rounding_allowance`` gives, per output element, what the
  other choice moves y by (weight x spacing), so that a comparison can accept
  either.
* On the FP8 path each 128-wide block of the down projection is summed on FP8
  matrix cores and then promoted with its two scales (PR #47844, implementation
  list: fine-grained FP8 blocks), so an expert output is known only to the
  accumulation precision of those cores: ``FP8_MMA_REL`` of the sum of the
  absolute products. There the band around a midpoint is the larger of that
  and the float32 one.

Functions marked "parity pinned" are checked in the CPU test suite against
the format definition, library routines, closed forms or brute force.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable

import numpy as np

__all__ = [
    "E4M3_MAX", "e4m3_values", "e4m3_encode", "bf16_to_f64", "bf16_round",
    "quantize_act", "quantize_weight_blocks", "dequantize_act", "dequantize_weight_blocks",
    "router_logits", "route", "sigmoid_scores", "route_sigmoid", "permute", "swiglu_expert", "combine",
    "bf16_spacing", "bf16_midpoint_straddle", "rounding_allowance", "FP8_MMA_REL",
    "OracleResult", "moe_forward", "moe_forward_loops",
]

E4M3_MAX = 448.0
BLOCK = 128


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def e4m3_values() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (float64); NaN for 0x7F and 0xFF.

    Layout: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    Exponent field 0 is subnormal: 2^-6 * m/8. parity pinned (format facts and
    torch.float8_e4m3fn).
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * math.ldexp(man / 8.0, -6)
        else:
            vals[code] = sign * math.ldexp(1.0 + man / 8.0, exp - 7)
    return vals


_E4M3 = e4m3_values()
_E4M3_POS = _E4M3[:127]  # codes 0x00..0x7E, ascending magnitudes 0 .. 448


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest, ties to the even code, saturating at +-448.

    The sign bit of the input is copied into bit 7 (so -0.0 -> 0x80). Inputs
    must be finite. parity pinned.
    """
    v = np.asarray(v)
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first table value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)       # saturation
    code = np.where(a == _E4M3_POS[hi], hi, code)  # exact table hits (incl. 0)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (a bfloat16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits; below 2^-126 the spacing is fixed at
    2^-133. Finite inputs below the bfloat16 overflow threshold. parity pinned
    (torch bfloat16 casts).
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)  # v = m * 2^e, 0.5 <= |m| < 1
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.round(v / step) * step  # np.round: half to even; v/step is exact


# ---------------------------------------------------------------------------
# FP8 quantisation (fine-grained: 1x128 activations, 128x128 weights)
# ---------------------------------------------------------------------------

def _scales(amax32: np.ndarray) -> np.ndarray:
    """s = f32(amax / 448): float32 division, correctly rounded."""
    return (np.asarray(amax32, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)


def _codes(vals32: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E4M3 codes of f32(v / s); a zero scale gives all-zero codes."""
    s = np.asarray(s, dtype=np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    q = e4m3_encode((vals32 / safe).astype(np.float32))
    return np.where(s == 0, np.uint8(0), q).astype(np.uint8)


def quantize_act(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row 1x128 dynamic activation quantisation (PR #47844: dynamic activations).

    x: [R, C] values exactly representable in float32 (BF16 activations).
    Returns codes [R, C] uint8 and scales [R, ceil(C/128)] float32; the last
    slice may be narrower than 128. parity pinned.
    """
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    nb = -(-C // BLOCK)
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((R, nb), dtype=np.float32)
    for j in range(nb):
        sl = x32[:, j * BLOCK:(j + 1) * BLOCK]
        s[:, j] = _scales(np.max(np.abs(sl), axis=1))
        q[:, j * BLOCK:(j + 1) * BLOCK] = _codes(sl, s[:, j:j + 1])
    return q, s


def quantize_weight_blocks(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """128x128 block quantisation of a float32 weight [rows, cols] (PR #47844: 128 x 128 weight blocks).

    Edge blocks cover only the valid rows/columns. Returns codes [rows, cols]
    uint8 and scales [ceil(rows/128), ceil(cols/128)] float32. parity pinned.
    """
    w32 = np.asarray(w, dtype=np.float32)
    R, C = w32.shape
    nr, nc = -(-R // BLOCK), -(-C // BLOCK)
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((nr, nc), dtype=np.float32)
    for i in range(nr):
        for j in range(nc):
            blk = w32[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK]
            s[i, j] = _scales(np.max(np.abs(blk)))
            q[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK] = _codes(blk, s[i, j])
    return q, s


def dequantize_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """value(code) * scale, per 1x128 slice, in float64."""
    v = _E4M3[np.asarray(q)]
    scale = np.repeat(np.asarray(s, dtype=np.float64), BLOCK, axis=1)[:, :v.shape[1]]
    return v * scale


def dequantize_weight_blocks(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """value(code) * scale, per 128x128 block, in float64."""
    v = _E4M3[np.asarray(q)]
    sc = np.asarray(s, dtype=np.float64)
    sc = np.repeat(np.repeat(sc, BLOCK, axis=0), BLOCK, axis=1)[:v.shape[0], :v.shape[1]]
    return v * sc


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """FP32 router logits L[t, e] = sum_h x[t, h] * W_r[e, h], summed in float64, stored as float32.

    Router output shape (batch*seq, num_experts): Transformers documentation "Dots 3 Note Preview",
    ``router_logits`` output entry; FP32 routing: PR #47844 implementation list.
    parity pinned (brute force, special weights).
    """
    return (np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T).astype(np.float32)


def route(logits: np.ndarray, k: int, n_group: int = 1, topk_group: int | None = None,
          renormalize: bool = True, scaling: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Top-k routing with softmax weights.

    Selection: the k largest FP32 logits; equal values go to the lower expert
    index; -0.0 is treated as +0.0; slot j holds the expert of rank j.
    Group-limited selection (Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
    ``n_group``, ``topk_group``; 1 and 1 by default, i.e. ungrouped): the E
    experts form n_group groups of E/n_group consecutive experts, a group's
    score is its largest logit (the docs fix only that the chosen experts lie
    in topk_group groups; the best expert of a group is the plainest score),
    the topk_group groups with the largest scores are kept (equal scores: the
    lower group), and the k experts are the top-k of the kept groups' experts.
    Weights: p = softmax over all E experts (float64); with ``renormalize``
    (``norm_topk_prob``, default true) p_S / sum(p_S) over the selected set S,
    otherwise p_S; times ``scaling`` (``routed_scaling_factor``, default 1.0);
    stored as float32. parity pinned (brute force, closed forms, hand example).
    """
    L = np.asarray(logits, dtype=np.float32)
    L = np.where(L == 0, np.float32(0.0), L)  # canonicalise -0.0
    T, E = L.shape
    topk_group = n_group if topk_group is None else topk_group
    sel = L.astype(np.float64)
    if n_group > 1:
        assert E % n_group == 0 and 1 <= topk_group <= n_group and k <= topk_group * (E // n_group)
        gscore = sel.reshape(T, n_group, E // n_group).max(axis=2)
        gkeep = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]  # ties: lower group first
        allowed = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(allowed, gkeep, True, axis=1)
        sel = np.where(np.repeat(allowed, E // n_group, axis=1), sel, -np.inf)
    order = np.argsort(-sel, axis=1, kind="stable")  # stable: ties keep ascending expert index
    ids = order[:, :k].astype(np.int32)
    L64 = L.astype(np.float64)
    ex = np.exp(L64 - L64.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = (ps / ps.sum(axis=1, keepdims=True) if renormalize else ps) * float(scaling)
    return ids, w.astype(np.float32)


def sigmoid_scores(logits: np.ndarray) -> np.ndarray:
    """Per-expert scores 1 / (1 + exp(-l)), computed in float64 and rounded once to float32."""
    L = np.asarray(logits, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-L))).astype(np.float32)


def route_sigmoid(logits: np.ndarray, k: int, bias: np.ndarray | None = None, n_group: int = 1,
                  topk_group: int | None = None, renormalize: bool = True,
                  scaling: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Sigmoid scoring with a selection-only correction bias, as in the routers the Transformers documentation ("Dots 3 Note Preview",
    model outputs, ``aux_loss`` entry) describe as balancing their experts with a router bias (DeepSeek-V3 and
    its derivatives); written from that published rule.

    s = sigmoid_scores(L) (FP32); b = f32(s + bias) is used for selection only. With n_group > 1 a group's score
    is f32(b1 + b2), its two largest b (the one b for a group of one expert), the topk_group best groups are kept
    (equal scores: the lower group) and the top-k of their experts by b (equal: lower expert) are selected.
    Weights: the unbiased s of the selected experts, divided by their sum when ``renormalize``, times
    ``scaling``, computed in float64 and stored as float32. parity pinned (brute force, hand example).
    """
    s = sigmoid_scores(logits)
    T, E = s.shape
    b = s if bias is None else (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    b = np.where(b == 0, np.float32(0.0), b)
    topk_group = n_group if topk_group is None else topk_group
    sel = b.astype(np.float64)
    if n_group > 1:
        gs = E // n_group
        assert E % n_group == 0 and 1 <= topk_group <= n_group and k <= topk_group * gs
        grouped = np.sort(b.reshape(T, n_group, gs), axis=2)[:, :, ::-1]
        gscore = grouped[:, :, 0] if gs == 1 else (grouped[:, :, 0] + grouped[:, :, 1]).astype(np.float32)
        gkeep = np.argsort(-gscore.astype(np.float64), axis=1, kind="stable")[:, :topk_group]
        allowed = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(allowed, gkeep, True, axis=1)
        sel = np.where(np.repeat(allowed, gs, axis=1), sel, -np.inf)
    ids = np.argsort(-sel, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = np.take_along_axis(s.astype(np.float64), ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, (w * float(scaling)).astype(np.float32)


def permute(ids: np.ndarray, e0: int, e_loc: int):
    """Group the (token, slot) pairs whose expert is local into expert-contiguous rows.

    Local experts are [e0, e0+e_loc). Rows are ordered by (local expert, token),
    i.e. a stable counting sort over the flat pair index t*K + k. Returns
    offsets [e_loc+1], row_token [M], row_slot [M], token_row [T, K] (-1 for a
    pair whose expert is not local). parity pinned (invariants, special cases).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    local = (flat >= e0) & (flat < e0 + e_loc)
    pairs = np.nonzero(local)[0]
    keys = flat[pairs] - e0
    counts = np.bincount(keys, minlength=e_loc)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = pairs[np.argsort(keys, kind="stable")]
    row_token = (rows // K).astype(np.int32)
    row_slot = (rows % K).astype(np.int32)
    token_row = np.full(T * K, -1, dtype=np.int32)
    token_row[rows] = np.arange(rows.size, dtype=np.int32)
    return offsets, row_token, row_slot, token_row.reshape(T, K)


# ---------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------

def _silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu_expert(a: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, fp8: bool,
                  rounded: bool = True, abs_terms: bool = False):
    """One expert on rows a: o = bf16(down(q(bf16(silu(a Wg^T) * (a Wu^T))))).

    a, wg [F, H], wu [F, H], wd [H, F] are float64 (already dequantised on the
    FP8 path). On the FP8 path the BF16 h is quantised per 1x128 slice and
    dequantised before the down projection. Returns float64 values that are
    exactly bfloat16, or with ``rounded=False`` the float64 down projection
    before its BF16 rounding; with ``abs_terms`` also the sum of the absolute
    products of that projection, |h| |Wd|^T. parity pinned (textbook SwiGLU via
    torch; FP8 h step against torch's float8 cast and hand-made values;
    absolute sums by loops).
    """
    g = a @ wg.T
    u = a @ wu.T
    h = bf16_round(_silu(g) * u)
    if fp8:
        qh, sh = quantize_act(h)
        h = dequantize_act(qh, sh)
    o = h @ wd.T
    o = bf16_round(o) if rounded else o
    return (o, np.abs(h) @ np.abs(wd).T) if abs_terms else o


# Accumulation precision of one 128-wide block sum on FP8 matrix cores, as a fraction of the sum of the
# absolute products: 2^-13 (1.2e-4) bounds the largest error measured for one 128-term E4M3 instruction on
# gfx950 matrix cores against the exact sum (1.1e-4, with operands spread over the whole exponent range;
# 1.9e-5 in the normal range). A block's scales multiply its error and its absolute sum alike, so the bound
# holds for the promoted sum over all blocks.
FP8_MMA_REL = 2.0 ** -13


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Distance between the two bfloat16 values that bracket |v| (8 significant bits: 2^(floor(log2|v|) - 7))."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    return 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)


def bf16_midpoint_straddle(v: np.ndarray, rel: float = 2.0 ** -18, band: np.ndarray | None = None) -> np.ndarray:
    """True where the exact value v lies within max(rel * |v|, band) of a midpoint between two adjacent
    bfloat16 values.

    A sum of thousands of products carried out in float32 (or on matrix cores with float32 accumulation) is
    only known to about that relative precision, so such a value can legitimately be rounded to either of
    its two bfloat16 neighbours; ``band`` (same shape as v, or None) widens that to an absolute precision,
    e.g. that of a sum formed on FP8 matrix cores.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    u = bf16_spacing(v)
    q = a / u
    dist = np.abs(q - np.floor(q) - 0.5) * u
    tol = rel * a if band is None else np.maximum(rel * a, np.asarray(band, dtype=np.float64))
    return (a > 0) & (dist <= tol)


def rounding_allowance(o_exact: np.ndarray, token_row: np.ndarray, w: np.ndarray, s_exact: np.ndarray | None,
                       t_s: int, o_band: np.ndarray | None = None, s_band: np.ndarray | None = None) -> np.ndarray:
    """Per output element: sum over the routed pairs (and the shared expert) of |weight| x the bfloat16
    spacing of those expert outputs whose exact value straddles a rounding midpoint (bf16_midpoint_straddle).

    The layer rounds every expert output to bfloat16 before the weighted sum; where the exact value sits on a
    midpoint within float32 precision, either neighbour is a correct rounding, and the two choices move y by
    the weight times the spacing. Elements far from a midpoint get no allowance. ``o_band``/``s_band`` are the
    absolute precision bands of the expert outputs (bf16_midpoint_straddle's ``band``), or None.
    """
    oa = np.where(bf16_midpoint_straddle(o_exact, band=o_band), bf16_spacing(o_exact), 0.0)
    sa = None if s_exact is None else np.where(bf16_midpoint_straddle(s_exact, band=s_band),
                                               bf16_spacing(s_exact), 0.0)
    return combine(oa, token_row, np.abs(np.asarray(w, dtype=np.float64)), sa, t_s, rounded=False)


def combine(o: np.ndarray, token_row: np.ndarray, w: np.ndarray, s: np.ndarray | None, t_s: int,
            rounded: bool = True) -> np.ndarray:
    """y[t] = bf16( sum_k w[t,k] * o[token_row[t,k]] + (t < T_s ? s[t] : 0) ), summed in float64.

    Pairs with token_row < 0 (expert on another GPU) contribute nothing. With
    ``rounded=False`` the float64 sum is returned before its one BF16 rounding.
    """
    T, K = token_row.shape
    H = o.shape[1] if o.size else (s.shape[1] if s is not None else 0)
    acc = np.zeros((T, H), dtype=np.float64)
    for k in range(K):
        r = token_row[:, k]
        m = r >= 0
        acc[m] += np.asarray(w, dtype=np.float64)[m, k][:, None] * o[r[m]]
    if s is not None and t_s > 0:
        acc[:t_s] += s[:t_s]
    return bf16_round(acc) if rounded else acc


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class OracleResult:
    tokens: np.ndarray          # which tokens y holds (all of them unless sampled)
    logits: np.ndarray          # [n, E] float32
    ids: np.ndarray             # [n, K] int32
    w: np.ndarray               # [n, K] float32
    x_codes: np.ndarray | None  # [n, H] uint8 (FP8 path)
    x_scales: np.ndarray | None
    y: np.ndarray               # [n, H] float64 (bfloat16 values)
    y_sum: np.ndarray           # [n, H] float64: the combine's sum before its BF16 rounding
    y_allow: np.ndarray | None = None  # [n, H] float64: rounding_allowance of the expert outputs


def _expert_weights(cfg, weights: Callable, e: int, fp8: bool):
    out = []
    for which in ("gate", "up", "down"):
        wsrc = weights(which, e)
        if fp8:
            q, s = quantize_weight_blocks(wsrc)
            out.append(dequantize_weight_blocks(q, s))
        else:
            out.append(bf16_to_f64(wsrc))
    return out


def moe_forward(cfg, x_bits: np.ndarray, weights: Callable, w_r: np.ndarray | None = None,
                logits: np.ndarray | None = None, tokens: np.ndarray | None = None,
                score_bias: np.ndarray | None = None) -> OracleResult:
    """Forward of one MoE layer for all tokens, or for the listed ``tokens`` only.

    cfg: object with T, H, F, F_s, E, e0, E_loc, K, T_s, dtype, and optionally the
    routing options n_group, topk_group (0: every group), renormalize, scaling and
    scoring ("softmax" or "sigmoid", the latter with the optional per-expert
    selection bias ``score_bias``).
    x_bits: [T, H] bfloat16 bits. weights(which, e) returns expert e's
    "gate"/"up"/"down" weight (float32 for FP8, bfloat16 bits for BF16; e = -1
    is the shared expert). Either w_r (router weight, float32 [E, H]) or given
    logits [T, E] float32.

    Each token's output depends only on its own row, so a sample of tokens is
    computed exactly as the full layer would compute those rows.
    """
    fp8 = cfg.dtype == "fp8"
    tok = np.arange(cfg.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x = bf16_to_f64(np.asarray(x_bits)[tok])
    L = router_logits(x, w_r) if logits is None else np.asarray(logits, dtype=np.float32)[tok]
    ropts = dict(n_group=getattr(cfg, "n_group", 1), topk_group=getattr(cfg, "topk_group", 0) or None,
                 renormalize=getattr(cfg, "renormalize", True), scaling=getattr(cfg, "scaling", 1.0))
    if getattr(cfg, "scoring", "softmax") == "sigmoid":
        ids, w = route_sigmoid(L, cfg.K, bias=score_bias, **ropts)
    else:
        ids, w = route(L, cfg.K, **ropts)
    offsets, row_token, _, token_row = permute(ids, cfg.e0, cfg.E_loc)
    if fp8:
        xq, xs = quantize_act(x)
        a_all = dequantize_act(xq, xs)
    else:
        xq = xs = None
        a_all = x
    o_ex = np.zeros((int(offsets[-1]), cfg.H), dtype=np.float64)  # expert outputs before their BF16 rounding
    # FP8: absolute precision band of each expert output (FP8_MMA_REL x its sum of absolute products)
    o_band = np.zeros_like(o_ex) if fp8 else None
    for el in range(cfg.E_loc):
        r0, r1 = int(offsets[el]), int(offsets[el + 1])
        if r1 == r0:
            continue
        wg, wu, wd = _expert_weights(cfg, weights, cfg.e0 + el, fp8)
        if fp8:
            o_ex[r0:r1], ab = swiglu_expert(a_all[row_token[r0:r1]], wg, wu, wd, fp8, rounded=False,
                                            abs_terms=True)
            o_band[r0:r1] = FP8_MMA_REL * ab
        else:
            o_ex[r0:r1] = swiglu_expert(a_all[row_token[r0:r1]], wg, wu, wd, fp8, rounded=False)
    shared_rows = tok < cfg.T_s
    s_ex = np.zeros((tok.size, cfg.H), dtype=np.float64)
    s_band = np.zeros_like(s_ex) if fp8 else None
    if shared_rows.any():
        wg, wu, wd = _expert_weights(cfg, weights, -1, fp8)
        if fp8:
            s_ex[shared_rows], ab = swiglu_expert(a_all[shared_rows], wg, wu, wd, fp8, rounded=False,
                                                  abs_terms=True)
            s_band[shared_rows] = FP8_MMA_REL * ab
        else:
            s_ex[shared_rows] = swiglu_expert(a_all[shared_rows], wg, wu, wd, fp8, rounded=False)
    # rows of s past T_s are zero
    y_sum = combine(bf16_round(o_ex), token_row, w, bf16_round(s_ex), tok.size, rounded=False)
    y_allow = rounding_allowance(o_ex, token_row, w, s_ex, tok.size, o_band, s_band)
    return OracleResult(tok, L, ids, w, xq, xs, bf16_round(y_sum), y_sum, y_allow)


def moe_forward_loops(cfg, x_bits, weights: Callable, w_r=None, logits=None) -> np.ndarray:
    """Per-token, per-expert loop form of the layer (brute force for tiny workloads).

    For every token: choose its experts by comparing logits pairwise, weight
    them, run each chosen local expert on that token alone, add the shared
    expert, round once. Used to cross-check ``moe_forward`` on tiny shapes.
    """
    fp8 = cfg.dtype == "fp8"
    x = bf16_to_f64(np.asarray(x_bits))
    cache = {}

    def ew(e):
        if e not in cache:
            cache[e] = _expert_weights(cfg, weights, e, fp8)
        return cache[e]

    y = np.zeros((cfg.T, cfg.H), dtype=np.float64)
    for t in range(cfg.T):
        lt = router_logits(x[t:t + 1], w_r)[0] if logits is None else np.asarray(logits, np.float32)[t]
        lt = np.where(lt == 0, np.float32(0.0), lt)
        chosen = []
        for e in range(cfg.E):  # rank of e = number of experts that beat it
            rank = sum(1 for j in range(cfg.E) if lt[j] > lt[e] or (lt[j] == lt[e] and j < e))
            if rank < cfg.K:
                chosen.append((rank, e))
        chosen.sort()
        l64 = lt.astype(np.float64)
        p = np.exp(l64 - l64.max())
        p /= p.sum()
        tot = sum(p[e] for _, e in chosen)
        if fp8:
            xq, xs = quantize_act(x[t:t + 1])
            a = dequantize_act(xq, xs)
        else:
            a = x[t:t + 1]
        acc = np.zeros(cfg.H, dtype=np.float64)
        for _, e in chosen:
            if not (cfg.e0 <= e < cfg.e0 + cfg.E_loc):
                continue
            wgt = float(np.float32(p[e] / tot))
            acc += wgt * swiglu_expert(a, *ew(e), fp8)[0]
        if t < cfg.T_s:
            acc += swiglu_expert(a, *ew(-1), fp8)[0]
        y[t] = bf16_round(acc)
    return y
