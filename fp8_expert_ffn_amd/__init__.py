"""libdmoe: the dots3-note preview MoE-layer hot path for AMD Instinct MI355X (gfx950).

The compute lives in libdmoe.so (hand-written HIP kernels behind the C ABI in
include/dmoe.h); this package loads it with ctypes and uses PyTorch only for
device memory and streams. Build the library with
``python -m fp8_expert_ffn_amd.build``.
"""
from ._lib import (  # noqa: F401
    DMOE_BF16, DMOE_FP8_E4M3, DMOE_SCORING_SOFTMAX, DMOE_SCORING_SIGMOID, DmoeError, LayerDesc, LayerPtrs, lib,
    dmoe_router_logits, dmoe_route, dmoe_route_grouped, dmoe_route_sigmoid, dmoe_permute, dmoe_quant_act, dmoe_quant_weight_blocks,
    dmoe_gemm_ws_bytes, dmoe_grouped_gemm_gateup, dmoe_grouped_gemm_down, dmoe_shared_expert,
    dmoe_combine, dmoe_forward, dmoe_forward_timed, dmoe_forward_ws_bytes, dmoe_forward_ws_offset,
    dmoe_forward_gateup_kernel, dmoe_forward_down_kernel,
    DMOE_STAGES, STAGE_NAMES,
)
from .layer import MoELayer  # noqa: F401
