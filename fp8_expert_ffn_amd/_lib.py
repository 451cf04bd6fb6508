"""ctypes binding of libdmoe (include/dmoe.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that live on the GPU (torch supplies device memory and the current
HIP stream), passes their raw pointers and sizes, and raises DmoeError on a
non-zero status. All arithmetic runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DMOE_LIB") or os.path.join(HERE, "libdmoe.so")

DMOE_OK = 0
DMOE_ERR_INVALID_ARG = 1
DMOE_ERR_ALIGNMENT = 2
DMOE_ERR_UNSUPPORTED = 3
DMOE_ERR_WORKSPACE = 4
DMOE_ERR_HIP = 5
DMOE_BF16 = 1
DMOE_FP8_E4M3 = 2
DMOE_SCORING_SOFTMAX = 0
DMOE_SCORING_SIGMOID = 1

EXPORTS = [
    "dmoe_last_error", "dmoe_abi_version", "dmoe_router_logits", "dmoe_route", "dmoe_route_grouped",
    "dmoe_route_sigmoid",
    "dmoe_permute_ws_bytes",
    "dmoe_permute", "dmoe_quant_act", "dmoe_quant_weight_blocks", "dmoe_gemm_ws_bytes",
    "dmoe_grouped_gemm_gateup", "dmoe_grouped_gemm_down", "dmoe_shared_expert_ws_bytes", "dmoe_shared_expert",
    "dmoe_combine", "dmoe_forward_ws_bytes", "dmoe_forward", "dmoe_forward_timed", "dmoe_forward_ws_offset",
    "dmoe_forward_gateup_kernel", "dmoe_forward_down_kernel", "dmoe_forward_noalloc",
]
DMOE_STAGES = 9
STAGE_NAMES = ["router_logits", "route", "permute", "quant_x", "gateup", "quant_h", "down", "shared", "combine"]


class DmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libdmoe status {status}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "F", "F_s", "E", "E_loc", "e0", "K", "T_s", "dtype", "logits_given",
                 "n_group", "topk_group", "no_renormalize")] + [("routed_scaling_factor", ctypes.c_float),
                                                                 ("scoring", ctypes.c_int32)]


class LayerPtrs(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("w_router", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("score_bias", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("ldw_gu", ctypes.c_int64), ("ldw_d", ctypes.c_int64),
        ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
        ("sw_gate", ctypes.c_void_p), ("sw_up", ctypes.c_void_p), ("sw_down", ctypes.c_void_p),
        ("ldsw_gu", ctypes.c_int64), ("ldsw_d", ctypes.c_int64),
        ("sws_gate", ctypes.c_void_p), ("sws_up", ctypes.c_void_p), ("sws_down", ctypes.c_void_p),
        ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
    ]


_lib = None
P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_SIGS = {
    "dmoe_last_error": ([], ctypes.c_char_p),
    "dmoe_abi_version": ([], I32),
    "dmoe_router_logits": ([P, I64, P, I32, I32, I32, P, P], I32),
    "dmoe_route": ([P, I32, I32, I32, P, P, P], I32),
    "dmoe_route_grouped": ([P, I32, I32, I32, I32, I32, I32, ctypes.c_float, P, P, P], I32),
    "dmoe_route_sigmoid": ([P, P, I32, I32, I32, I32, I32, I32, ctypes.c_float, P, P, P], I32),
    "dmoe_permute_ws_bytes": ([I32, I32, I32], SZ),
    "dmoe_permute": ([P, I32, I32, I32, I32, P, P, P, P, P, SZ, P], I32),
    "dmoe_quant_act": ([P, I32, I32, I64, P, I64, P, I64, P], I32),
    "dmoe_quant_weight_blocks": ([P, I32, I32, I64, P, I64, P, P], I32),
    "dmoe_gemm_ws_bytes": ([I32, I32], SZ),
    "dmoe_grouped_gemm_gateup": ([I32, P, I64, P, I64, P, P, I32, I32, P, P, I64, P, P, I32, I32, P, I64, P, SZ, P],
                                 I32),
    "dmoe_grouped_gemm_down": ([I32, P, I64, P, I64, P, I32, I32, P, I64, P, I32, I32, P, I64, P, SZ, P], I32),
    "dmoe_shared_expert_ws_bytes": ([I32, I32, I32, I32], SZ),
    "dmoe_shared_expert": ([I32, P, I64, P, I64, I32, P, P, P, I64, I64, P, P, P, I32, I32, P, I64, P, SZ, P], I32),
    "dmoe_combine": ([P, I64, P, P, P, I64, I32, I32, I32, I32, P, I64, P], I32),
    "dmoe_forward_ws_bytes": ([ctypes.POINTER(LayerDesc)], SZ),
    "dmoe_forward": ([ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerPtrs), P, SZ, P], I32),
    "dmoe_forward_timed": ([ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerPtrs), P, SZ, P, P], I32),
    "dmoe_forward_ws_offset": ([ctypes.POINTER(LayerDesc), I32], I64),
    "dmoe_forward_gateup_kernel": ([ctypes.POINTER(LayerDesc)], ctypes.c_char_p),
    "dmoe_forward_down_kernel": ([ctypes.POINTER(LayerDesc)], ctypes.c_char_p),
    "dmoe_forward_noalloc": ([ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerPtrs), P], I32),
}


def lib() -> ctypes.CDLL:
    """Load libdmoe.so (fails loudly if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp8_expert_ffn_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != DMOE_OK:
        raise DmoeError(status, lib().dmoe_last_error().decode())


def ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdmoe takes device tensors")
    return t.data_ptr()


def stream_handle(stream: torch.cuda.Stream | None = None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


# ---------------------------------------------------------------------------
# One Python function per entry point.
# ---------------------------------------------------------------------------

def dmoe_router_logits(x: torch.Tensor, w_r: torch.Tensor, logits: torch.Tensor | None = None, stream=None):
    T, H = x.shape
    E = w_r.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib().dmoe_router_logits(ptr(x), _ld(x), ptr(w_r), T, H, E, ptr(logits), stream_handle(stream)))
    return logits


def dmoe_route(logits: torch.Tensor, K: int, topk_ids=None, topk_w=None, stream=None):
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check(lib().dmoe_route(ptr(logits), T, E, K, ptr(topk_ids), ptr(topk_w), stream_handle(stream)))
    return topk_ids, topk_w


def dmoe_route_sigmoid(logits: torch.Tensor, K: int, score_bias: torch.Tensor | None = None, n_group: int = 1,
                       topk_group: int = 0, renormalize: bool = True, routed_scaling_factor: float = 1.0,
                       topk_ids=None, topk_w=None, stream=None):
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check(lib().dmoe_route_sigmoid(ptr(logits), ptr(score_bias) if score_bias is not None else None, T, E, K,
                                    n_group, topk_group, 1 if renormalize else 0, routed_scaling_factor,
                                    ptr(topk_ids), ptr(topk_w), stream_handle(stream)))
    return topk_ids, topk_w


def dmoe_route_grouped(logits: torch.Tensor, K: int, n_group: int = 1, topk_group: int = 0,
                       renormalize: bool = True, routed_scaling_factor: float = 1.0, topk_ids=None, topk_w=None,
                       stream=None):
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check(lib().dmoe_route_grouped(ptr(logits), T, E, K, n_group, topk_group, 1 if renormalize else 0,
                                    routed_scaling_factor, ptr(topk_ids), ptr(topk_w), stream_handle(stream)))
    return topk_ids, topk_w


def dmoe_permute(topk_ids: torch.Tensor, e0: int, E_loc: int, stream=None):
    T, K = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
    row_slot = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
    token_row = torch.empty((T, K), dtype=torch.int32, device=dev)
    nbytes = lib().dmoe_permute_ws_bytes(T, K, E_loc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().dmoe_permute(ptr(topk_ids), T, K, e0, E_loc, ptr(offsets), ptr(row_token), ptr(row_slot),
                              ptr(token_row), ptr(ws), nbytes, stream_handle(stream)))
    return offsets, row_token, row_slot, token_row


def dmoe_quant_act(x: torch.Tensor, cols: int | None = None, stream=None):
    """x: [rows, >=cols] BF16 -> (codes [rows, round_up(cols,128)] uint8, scales [rows, ceil(cols/128)] f32)."""
    rows = x.shape[0]
    cols = x.shape[1] if cols is None else cols
    nb = -(-cols // 128)
    q = torch.empty((rows, nb * 128), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, nb), dtype=torch.float32, device=x.device)
    _check(lib().dmoe_quant_act(ptr(x), rows, cols, _ld(x), ptr(q), nb * 128, ptr(s), nb, stream_handle(stream)))
    return q, s


def dmoe_quant_weight_blocks(w: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                             stream=None):
    """w: [rows, cols] FP32 -> codes [round_up(rows,128), ldq >= round_up(cols,128)], scales [ceil, ceil]."""
    rows, cols = w.shape
    if q is None:
        q = torch.empty((-(-rows // 128) * 128, -(-cols // 128) * 128), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((-(-rows // 128), -(-cols // 128)), dtype=torch.float32, device=w.device)
    _check(lib().dmoe_quant_weight_blocks(ptr(w), rows, cols, _ld(w), ptr(q), _ld(q), ptr(scales),
                                          stream_handle(stream)))
    return q, scales


def dmoe_gemm_ws_bytes(max_rows: int, E_loc: int) -> int:
    return lib().dmoe_gemm_ws_bytes(max_rows, E_loc)


def dmoe_grouped_gemm_gateup(dtype, a, a_scales, row_token, offsets, E_loc, max_rows, w_gate, w_up, w_scales_gate,
                             w_scales_up, H, F, h, ws=None, stream=None):
    """w_gate/w_up: [E_loc, F_pad, ldw] in the padded layout; h: [>=max_rows, ldh] BF16."""
    nbytes = dmoe_gemm_ws_bytes(max_rows, E_loc)
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=a.device)
    ldas = _ld(a_scales) if a_scales is not None else 0
    _check(lib().dmoe_grouped_gemm_gateup(dtype, ptr(a), _ld(a), ptr(a_scales), ldas, ptr(row_token), ptr(offsets),
                                          E_loc, max_rows, ptr(w_gate), ptr(w_up), w_gate.stride(1),
                                          ptr(w_scales_gate), ptr(w_scales_up), H, F, ptr(h), _ld(h), ptr(ws),
                                          ws.numel(), stream_handle(stream)))
    return h


def dmoe_grouped_gemm_down(dtype, h, h_scales, offsets, E_loc, max_rows, w_down, w_scales_down, F, H, o, ws=None,
                           stream=None):
    nbytes = dmoe_gemm_ws_bytes(max_rows, E_loc)
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=h.device)
    ldhs = _ld(h_scales) if h_scales is not None else 0
    _check(lib().dmoe_grouped_gemm_down(dtype, ptr(h), _ld(h), ptr(h_scales), ldhs, ptr(offsets), E_loc, max_rows,
                                        ptr(w_down), w_down.stride(1), ptr(w_scales_down), F, H, ptr(o), _ld(o),
                                        ptr(ws), ws.numel(), stream_handle(stream)))
    return o


def dmoe_shared_expert(dtype, a, a_scales, T_s, w_gate, w_up, w_down, w_scales, H, F_s, s_out, stream=None):
    nbytes = lib().dmoe_shared_expert_ws_bytes(dtype, T_s, H, F_s)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=a.device)
    sg, su, sd = w_scales if w_scales is not None else (None, None, None)
    ldas = _ld(a_scales) if a_scales is not None else 0
    _check(lib().dmoe_shared_expert(dtype, ptr(a), _ld(a), ptr(a_scales), ldas, T_s, ptr(w_gate), ptr(w_up),
                                    ptr(w_down), w_gate.stride(-2), w_down.stride(-2), ptr(sg), ptr(su), ptr(sd), H,
                                    F_s, ptr(s_out), _ld(s_out), ptr(ws), nbytes, stream_handle(stream)))
    return s_out


def dmoe_combine(o, token_row, topk_w, s_out, T_s, H, y, stream=None):
    T, K = token_row.shape
    lds = _ld(s_out) if s_out is not None else 0
    _check(lib().dmoe_combine(ptr(o), _ld(o), ptr(token_row), ptr(topk_w), ptr(s_out), lds, T_s, T, K, H, ptr(y),
                              _ld(y), stream_handle(stream)))
    return y


def dmoe_forward_ws_bytes(desc: LayerDesc) -> int:
    return lib().dmoe_forward_ws_bytes(ctypes.byref(desc))


def dmoe_forward_ws_offset(desc: LayerDesc, which: int) -> int:
    return lib().dmoe_forward_ws_offset(ctypes.byref(desc), which)


def dmoe_forward_gateup_kernel(desc: LayerDesc) -> str | None:
    name = lib().dmoe_forward_gateup_kernel(ctypes.byref(desc))
    return name.decode() if name is not None else None


def dmoe_forward_down_kernel(desc: LayerDesc) -> str | None:
    name = lib().dmoe_forward_down_kernel(ctypes.byref(desc))
    return name.decode() if name is not None else None


def dmoe_forward(desc: LayerDesc, ptrs: LayerPtrs, ws: torch.Tensor, stream=None) -> None:
    _check(lib().dmoe_forward(ctypes.byref(desc), ctypes.byref(ptrs), ptr(ws), ws.numel(), stream_handle(stream)))


def dmoe_forward_noalloc(desc: LayerDesc, ptrs: LayerPtrs, stream=None) -> None:
    """dmoe_forward with the library's own fixed device workspace (no caller buffer, nothing allocated)."""
    _check(lib().dmoe_forward_noalloc(ctypes.byref(desc), ctypes.byref(ptrs), stream_handle(stream)))


DMOE_NOALLOC_WS_BYTES = 24 << 20


def dmoe_forward_timed(desc: LayerDesc, ptrs: LayerPtrs, ws: torch.Tensor, events, stream=None) -> None:
    """events: DMOE_STAGES + 1 entries, each a torch.cuda.Event(enable_timing=True) already recorded once
    (so that its HIP event exists) or None (that boundary is not recorded)."""
    if len(events) != DMOE_STAGES + 1:
        raise ValueError(f"need {DMOE_STAGES + 1} events")
    arr = (ctypes.c_void_p * len(events))(*[(e.cuda_event if e is not None else None) for e in events])
    _check(lib().dmoe_forward_timed(ctypes.byref(desc), ctypes.byref(ptrs), ptr(ws), ws.numel(),
                                    stream_handle(stream), arr))
