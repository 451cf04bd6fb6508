"""The shape sweep's draws are valid layers for the library's host checks and
reach every gate/up kernel, including the wide kernel that quantises h in its
epilogue (no GPU: descriptor checks and kernel choice are host logic)."""
import fp8_expert_ffn_amd as fm
from fp8_expert_ffn_amd import _lib as L
from sweep_cases import REGIMES, sweep_cases


def _desc(c):
    return L.LayerDesc(c.T, c.H, c.F, c.F_s, c.E, c.E_loc, c.e0, c.K, c.T_s,
                       L.DMOE_FP8_E4M3 if c.dtype == "fp8" else L.DMOE_BF16, 0, c.n_group, c.topk_group,
                       0 if c.renormalize else 1, c.scaling,
                       L.DMOE_SCORING_SIGMOID if c.scoring == "sigmoid" else L.DMOE_SCORING_SOFTMAX)


def test_sweep_draws_are_valid_and_reach_every_gateup_kernel():
    cases = sweep_cases()
    assert len({c.name for c in cases}) == len(cases)
    seen = set()
    for c in cases:
        d = _desc(c)
        assert fm.dmoe_forward_ws_bytes(d) > 0, c
        seen.add((fm.dmoe_forward_gateup_kernel(d), c.dtype))
    assert {("gemm_stage_kernel", "fp8"), ("gemm_stage_kernel", "bf16"), ("gemm_tile_kernel", "fp8"),
            ("gemm_tile_kernel", "bf16"), ("gemm_wide_kernel", "fp8")} <= seen
    assert {c.name.split("_", 1)[1].rsplit("_", 1)[0] for c in cases} == set(REGIMES)


def test_sweep_draws_are_reproducible():
    a, b = sweep_cases(), sweep_cases()
    assert a == b
