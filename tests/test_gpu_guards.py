"""Guard canaries: nothing is written past the rows or the pitches a call owns (GPU).

The workspace, the output y (with a pitch wider than H and two rows past T) and
standalone GEMM outputs are filled with a sentinel byte before the call; after
it, the bytes the call must not touch still hold the sentinel:
- routed rows [M, T*K) of h, of the h codes and scales, and of o (M = the real
  number of local pairs; the buffers are sized to the bound T*K);
- the pitch padding of y and its rows past T;
- for the standalone gate/up and down calls, rows past offsets[E_loc] and the
  pitch padding past the padded width."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, build_layer, layer_inputs, say, to_dev_bf16

pytestmark = pytest.mark.gpu

import fp8_expert_ffn_amd as dm  # noqa: E402
from fp8_expert_ffn_amd import _lib as L  # noqa: E402

SENT = 0xA5

CASES = {
    # tile GEMMs: the two-workgroup kernel for gate/up, separate FP8 h quantisation
    "tile_fp8": synth.LayerConfig("guard_tile_fp8", T=700, H=512, F=200, F_s=200, E=16, E_loc=16, e0=0, K=4,
                                  dtype="fp8", T_s=300, logits="uniform"),
    # FP8 gate/up on the wide kernel with h quantised in its epilogue (1024 rows per expert by the host bound),
    # with all pairs local and as an EP share
    "wide_fp8": synth.LayerConfig("guard_wide_fp8", T=2048, H=256, F=3200, F_s=3200, E=8, E_loc=8, e0=0, K=4,
                                  dtype="fp8", T_s=300, logits="uniform"),
    "wide_ep_fp8": synth.LayerConfig("guard_wide_ep_fp8", T=1024, H=256, F=3200, F_s=3200, E=64, E_loc=8, e0=8,
                                     K=8, dtype="fp8", T_s=100, logits="zipf"),
    # an EP share: most pairs are not local, so M is far below T*K
    "ep_fp8": synth.LayerConfig("guard_ep_fp8", T=900, H=512, F=256, F_s=256, E=64, E_loc=8, e0=8, K=8,
                                dtype="fp8", T_s=100, logits="zipf"),
    "tile_bf16": synth.LayerConfig("guard_tile_bf16", T=600, H=640, F=136, F_s=136, E=8, E_loc=8, e0=0, K=2,
                                   dtype="bf16", T_s=600, logits="router"),
    # weight-streaming GEMMs (few rows per expert), separate FP8 h quantisation
    "stream_fp8": synth.LayerConfig("guard_stream_fp8", T=24, H=1024, F=384, F_s=384, E=64, E_loc=32, e0=16, K=8,
                                    dtype="fp8", T_s=24, logits="uniform"),
}


def _bytes(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_writes_only_its_rows_and_pitches(name):
    cfg = CASES[name]
    say(f"[guard {name}] {cfg}")
    layer = build_layer(cfg)
    x_bits, wr, given = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    kw = dict(w_router=torch.from_numpy(wr).to(DEV)) if wr is not None else \
        dict(logits=torch.from_numpy(given).to(DEV))
    d, p, ws, out = layer.make_call(x, cfg.T_s, **kw)
    # y with 64 columns of pitch padding and two rows past T
    ypad = torch.full((cfg.T + 2, cfg.H + 64), 0, dtype=torch.int16, device=DEV)
    ypad.view(torch.uint8).fill_(SENT)
    p.y, p.ldy = L.ptr(ypad), cfg.H + 64
    ws.fill_(SENT)
    torch.cuda.synchronize()
    dm.dmoe_forward(d, p, ws)
    torch.cuda.synchronize()
    off = layer.ws_view(d, ws, "offsets").cpu().numpy()
    M, mcap = int(off[-1]), cfg.T * cfg.K
    say(f"  M = {M} of T*K = {mcap}")
    assert M < mcap or cfg.E_loc == cfg.E  # every pair is local only when all experts are
    for name_ in ("h", "h_codes", "h_scales", "o"):
        v = layer.ws_view(d, ws, name_)
        if v is None:
            continue
        tail = _bytes(v[M:mcap])
        assert bool((tail == SENT).all()), f"{name_}: rows [M, T*K) were written"
        if name_ in ("h_codes", "h_scales", "o"):
            head = _bytes(v[:M])
            assert not bool((head == SENT).all()), f"{name_}: the real rows were not written"
    yb = ypad.view(torch.uint8).view(cfg.T + 2, 2 * (cfg.H + 64))
    assert bool((yb[:, 2 * cfg.H:] == SENT).all()), "y: pitch padding was written"
    assert bool((yb[cfg.T:] == SENT).all()), "y: rows past T were written"
    assert not bool((yb[:cfg.T, :2 * cfg.H] == SENT).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_standalone_gemms_write_only_real_rows(dtype):
    """dmoe_grouped_gemm_gateup / _down with output pitches wider than the padded width and row buffers sized
    to the bound: rows past offsets[E_loc] and columns past the padded width stay untouched."""
    cfg = synth.LayerConfig(f"guard_gemm_{dtype}", T=500, H=512, F=200, F_s=0, E=16, E_loc=4, e0=2, K=4,
                            dtype=dtype, T_s=0, logits="uniform")
    layer = build_layer(cfg)
    x_bits, _, given = layer_inputs(cfg)
    x = to_dev_bf16(x_bits)
    ids, _ = dm.dmoe_route(torch.from_numpy(given).to(DEV), cfg.K)
    offsets, row_token, _, _ = dm.dmoe_permute(ids, cfg.e0, cfg.E_loc)
    torch.cuda.synchronize()
    M, mcap = int(offsets[-1].item()), cfg.T * cfg.K
    fpad = layer.fpad
    code = L.DMOE_FP8_E4M3 if dtype == "fp8" else L.DMOE_BF16
    if dtype == "fp8":
        a, a_s = dm.dmoe_quant_act(x)
    else:
        a, a_s = x, None
    h = torch.empty((mcap, fpad + 64), dtype=torch.int16, device=DEV)
    h.view(torch.uint8).fill_(SENT)
    hv = h.view(torch.bfloat16)
    dm.dmoe_grouped_gemm_gateup(code, a, a_s, row_token, offsets, cfg.E_loc, mcap, layer.w_gate, layer.w_up,
                                layer.s_gate, layer.s_up, cfg.H, cfg.F, hv)
    torch.cuda.synchronize()
    s16 = int(np.array([SENT * 0x101], np.uint16).view(np.int16)[0])  # the sentinel as one 16-bit element
    assert bool((h[M:] == s16).all()), "gate/up wrote rows past offsets[E_loc]"
    assert bool((h[:, fpad:] == s16).all()), "gate/up wrote past the padded width"
    assert not bool((h[:M, :fpad] == s16).any()), "gate/up left elements of real rows unwritten"
    hin = hv[:, :fpad].contiguous()
    if dtype == "fp8":
        hin, h_s = dm.dmoe_quant_act(hin, cols=cfg.F)
    else:
        h_s = None
    o = torch.empty((mcap, cfg.H + 32), dtype=torch.int16, device=DEV)
    o.view(torch.uint8).fill_(SENT)
    dm.dmoe_grouped_gemm_down(code, hin, h_s, offsets, cfg.E_loc, mcap, layer.w_down, layer.s_down, cfg.F, cfg.H,
                              o.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert bool((o[M:] == s16).all()), "down wrote rows past offsets[E_loc]"
    assert bool((o[:, cfg.H:] == s16).all()), "down wrote past H"
    assert not bool((o[:M, :cfg.H] == s16).any()), "down left elements of real rows unwritten"
