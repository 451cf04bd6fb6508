"""Device-resident MoE layer: weights in libdmoe's layout plus the whole-layer call.

Weight preparation (BF16 copy into the zero-padded layout, or FP8 128x128
block quantisation by dmoe_quant_weight_blocks) happens once, when weights are
set; dmoe_forward then runs router -> route -> permute -> [quantise x] ->
gate/up+SwiGLU -> [quantise h] -> down -> shared expert -> combine on one
stream with no host synchronisation.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def _round_up(v: int, m: int) -> int:
    return (v + m - 1) // m * m


def _cdiv(v: int, m: int) -> int:
    return -(-v // m)


class MoELayer:
    """One MoE layer's experts on this GPU: routed experts [e0, e0+E_loc) and the shared expert."""

    def __init__(self, H: int, F: int, F_s: int, E: int, E_loc: int, e0: int, K: int, dtype: str,
                 device: str | torch.device = "cuda", n_group: int = 1, topk_group: int = 0,
                 renormalize: bool = True, routed_scaling_factor: float = 1.0, scoring: str = "softmax"):
        if dtype not in ("bf16", "fp8"):
            raise ValueError("dtype must be 'bf16' or 'fp8'")
        self.H, self.F, self.F_s, self.E, self.E_loc, self.e0, self.K = H, F, F_s, E, E_loc, e0, K
        self.n_group, self.topk_group = n_group, topk_group
        self.renormalize, self.routed_scaling_factor = renormalize, routed_scaling_factor
        if scoring not in ("softmax", "sigmoid"):
            raise ValueError("scoring must be 'softmax' or 'sigmoid'")
        self.scoring = scoring
        self.score_bias = None  # [E] FP32 selection bias (sigmoid scoring), see set_score_bias
        self.dtype = dtype
        self.code = L.DMOE_FP8_E4M3 if dtype == "fp8" else L.DMOE_BF16
        self.device = torch.device(device)
        self.fpad = _round_up(F, 128)
        self.fspad = _round_up(F_s, 128) if F_s else 0
        wdt = torch.uint8 if dtype == "fp8" else torch.bfloat16
        z = dict(dtype=wdt, device=self.device)
        self.w_gate = torch.zeros((E_loc, self.fpad, H), **z)
        self.w_up = torch.zeros((E_loc, self.fpad, H), **z)
        self.w_down = torch.zeros((E_loc, H, self.fpad), **z)
        self.sw_gate = torch.zeros((self.fspad, H), **z) if F_s else None
        self.sw_up = torch.zeros((self.fspad, H), **z) if F_s else None
        self.sw_down = torch.zeros((H, self.fspad), **z) if F_s else None
        f = dict(dtype=torch.float32, device=self.device)
        if dtype == "fp8":
            self.s_gate = torch.zeros((E_loc, _cdiv(F, 128), H // 128), **f)
            self.s_up = torch.zeros((E_loc, _cdiv(F, 128), H // 128), **f)
            self.s_down = torch.zeros((E_loc, H // 128, _cdiv(F, 128)), **f)
            if F_s:
                self.ss_gate = torch.zeros((_cdiv(F_s, 128), H // 128), **f)
                self.ss_up = torch.zeros((_cdiv(F_s, 128), H // 128), **f)
                self.ss_down = torch.zeros((H // 128, _cdiv(F_s, 128)), **f)
        else:
            self.s_gate = self.s_up = self.s_down = None
            self.ss_gate = self.ss_up = self.ss_down = None
        self._ws = {}
        self._tmp = None

    # ------------------------------------------------------------------ weights
    def _dst(self, which: str, e: int):
        if e == -1:
            w = {"gate": self.sw_gate, "up": self.sw_up, "down": self.sw_down}[which]
            s = {"gate": self.ss_gate, "up": self.ss_up, "down": self.ss_down}[which] if self.dtype == "fp8" else None
        else:
            w = {"gate": self.w_gate, "up": self.w_up, "down": self.w_down}[which][e]
            s = {"gate": self.s_gate, "up": self.s_up, "down": self.s_down}[which][e] if self.dtype == "fp8" else None
        return w, s

    def set_weight(self, which: str, e: int, host: np.ndarray, stream=None) -> None:
        """Set local expert e's (or the shared expert's, e = -1) "gate"/"up"/"down" weight.

        host: nn.Linear layout [out, in]; BF16 bit patterns (uint16) for a BF16
        layer, FP32 for an FP8 layer (block-quantised here on the GPU).
        """
        w, s = self._dst(which, e)
        rows, cols = host.shape
        if self.dtype == "bf16":
            if host.dtype != np.uint16:
                raise TypeError("BF16 layers take bfloat16 bit patterns (uint16)")
            src = torch.from_numpy(np.ascontiguousarray(host).view(np.int16)).view(torch.bfloat16)
            w[:rows, :cols].copy_(src, non_blocking=False)
        else:
            if host.dtype != np.float32:
                raise TypeError("FP8 layers take float32 weights")
            n = rows * cols
            if self._tmp is None or self._tmp.numel() < n:
                self._tmp = torch.empty(n, dtype=torch.float32, device=self.device)
            tmp = self._tmp[:n].view(rows, cols)
            tmp.copy_(torch.from_numpy(np.ascontiguousarray(host)))
            L.dmoe_quant_weight_blocks(tmp, q=w, scales=s, stream=stream)

    # ------------------------------------------------------------------ forward
    def set_score_bias(self, bias) -> None:
        """Per-expert FP32 selection bias for sigmoid scoring ([E], host array or tensor)."""
        b = torch.as_tensor(bias, dtype=torch.float32)
        if b.shape != (self.E,):
            raise ValueError(f"score bias must have shape ({self.E},)")
        self.score_bias = b.to(self.device).contiguous()

    def desc(self, T: int, T_s: int, logits_given: bool) -> L.LayerDesc:
        return L.LayerDesc(T, self.H, self.F, self.F_s if T_s > 0 else 0, self.E, self.E_loc, self.e0, self.K,
                           T_s if self.F_s else 0, self.code, 1 if logits_given else 0, self.n_group,
                           self.topk_group, 0 if self.renormalize else 1, self.routed_scaling_factor,
                           L.DMOE_SCORING_SIGMOID if self.scoring == "sigmoid" else L.DMOE_SCORING_SOFTMAX)

    def workspace(self, desc: L.LayerDesc) -> torch.Tensor:
        key = tuple(getattr(desc, n) for n, _ in L.LayerDesc._fields_)
        if key not in self._ws:
            nbytes = L.dmoe_forward_ws_bytes(desc)
            if nbytes == 0:
                raise L.DmoeError(L.DMOE_ERR_INVALID_ARG, "invalid layer description")
            self._ws = {key: torch.empty(nbytes, dtype=torch.uint8, device=self.device)}
        return self._ws[key]

    def make_call(self, x: torch.Tensor, T_s: int, w_router: torch.Tensor | None = None,
                  logits: torch.Tensor | None = None):
        """Allocate outputs and build the (desc, ptrs, ws, outputs) of one dmoe_forward call."""
        T = x.shape[0]
        given = logits is not None
        if not given:
            if w_router is None:
                raise ValueError("need w_router or logits")
            logits = torch.empty((T, self.E), dtype=torch.float32, device=self.device)
        out = dict(
            logits=logits,
            topk_ids=torch.empty((T, self.K), dtype=torch.int32, device=self.device),
            topk_w=torch.empty((T, self.K), dtype=torch.float32, device=self.device),
            y=torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device),
        )
        d = self.desc(T, T_s, given)
        p = L.LayerPtrs()
        p.x, p.ldx = L.ptr(x), x.stride(0)
        p.w_router = L.ptr(w_router) if not given else None
        p.logits = L.ptr(logits)
        p.score_bias = L.ptr(self.score_bias) if self.score_bias is not None else None
        p.w_gate, p.w_up, p.w_down = L.ptr(self.w_gate), L.ptr(self.w_up), L.ptr(self.w_down)
        p.ldw_gu, p.ldw_d = self.H, self.fpad
        if self.dtype == "fp8":
            p.ws_gate, p.ws_up, p.ws_down = L.ptr(self.s_gate), L.ptr(self.s_up), L.ptr(self.s_down)
        if self.F_s:
            p.sw_gate, p.sw_up, p.sw_down = L.ptr(self.sw_gate), L.ptr(self.sw_up), L.ptr(self.sw_down)
            p.ldsw_gu, p.ldsw_d = self.H, self.fspad
            if self.dtype == "fp8":
                p.sws_gate, p.sws_up, p.sws_down = L.ptr(self.ss_gate), L.ptr(self.ss_up), L.ptr(self.ss_down)
        p.topk_ids, p.topk_w = L.ptr(out["topk_ids"]), L.ptr(out["topk_w"])
        p.y, p.ldy = L.ptr(out["y"]), self.H
        return d, p, self.workspace(d), out

    def forward(self, x: torch.Tensor, T_s: int, w_router: torch.Tensor | None = None,
                logits: torch.Tensor | None = None, stream=None) -> dict:
        d, p, ws, out = self.make_call(x, T_s, w_router, logits)
        L.dmoe_forward(d, p, ws, stream)
        out["_call"] = (d, p, ws)
        return out

    def ws_view(self, desc: L.LayerDesc, ws: torch.Tensor, which: str) -> torch.Tensor | None:
        """Typed view of an intermediate buffer inside the forward workspace."""
        idx = {"offsets": 0, "row_token": 1, "row_slot": 2, "token_row": 3, "x_codes": 4, "x_scales": 5,
               "h": 6, "h_codes": 7, "h_scales": 8, "o": 9, "shared": 10}[which]
        off = L.dmoe_forward_ws_offset(desc, idx)
        if off < 0:
            return None
        T, K, H = desc.T, desc.K, desc.H
        mcap = T * K
        shapes = {
            "offsets": ((desc.E_loc + 1,), torch.int32), "row_token": ((mcap,), torch.int32),
            "row_slot": ((mcap,), torch.int32), "token_row": ((T, K), torch.int32),
            "x_codes": ((T, H), torch.uint8), "x_scales": ((T, H // 128), torch.float32),
            "h": ((mcap, self.fpad), torch.bfloat16), "h_codes": ((mcap, self.fpad), torch.uint8),
            "h_scales": ((mcap, _cdiv(self.F, 128)), torch.float32), "o": ((mcap, H), torch.bfloat16),
            "shared": ((desc.T_s, H), torch.bfloat16),
        }
        shape, dt = shapes[which]
        n = int(np.prod(shape)) * torch.empty(0, dtype=dt).element_size()
        return ws[off:off + n].view(dt).view(shape)
