"""libdmoe on the host (no GPU): the library loads, exports every entry point
include/dmoe.h declares, and rejects invalid arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmoe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dmoe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import fp8_expert_ffn_amd as dm
    return dm


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dmoe_route", "dmoe_permute", "dmoe_quant_act", "dmoe_grouped_gemm_gateup", "dmoe_grouped_gemm_down",
              "dmoe_shared_expert", "dmoe_combine", "dmoe_forward", "dmoe_router_logits"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    for n in _declared():
        assert hasattr(lib, n), f"{n} declared in dmoe.h but not exported"
    assert set(_declared()) <= set(L._lib.EXPORTS) | {"dmoe_last_error", "dmoe_abi_version"}
    assert lib.dmoe_abi_version() == 2


def _status(fn, *args):
    return fn(*args)


def test_route_rejects_bad_sizes(L):
    lib = L.lib()
    fake = 0x1000
    assert lib.dmoe_route(fake, 4, 256, 300, fake, fake, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert b"K = 300" in lib.dmoe_last_error()
    assert lib.dmoe_route(fake, 4, 2000, 8, fake, fake, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert lib.dmoe_route(None, 4, 256, 8, fake, fake, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert lib.dmoe_route(None, 0, 256, 8, None, None, None) == 0  # T == 0 is a no-op


def test_quant_act_rejects_misaligned_and_short_pitches(L):
    lib = L.lib()
    assert lib.dmoe_quant_act(0x1008, 4, 128, 128, 0x2000, 128, 0x3000, 1, None) == L._lib.DMOE_ERR_ALIGNMENT
    assert lib.dmoe_quant_act(0x1000, 4, 1400, 1400, 0x2000, 1400, 0x3000, 11, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert lib.dmoe_quant_act(0x1000, 4, 100, 104, 0x2000, 128, 0x3000, 1, None) == L._lib.DMOE_ERR_INVALID_ARG


def test_permute_rejects_small_workspace(L):
    lib = L.lib()
    need = lib.dmoe_permute_ws_bytes(64, 8, 256)
    assert need > 0
    st = lib.dmoe_permute(0x1000, 64, 8, 0, 256, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, need - 1, None)
    assert st == L._lib.DMOE_ERR_WORKSPACE


def test_gemm_rejects_bad_dtype_and_shapes(L):
    lib = L.lib()
    f = 0x1000
    args = [f, 5120, f, 40, f, f, 256, 512, f, f, 5120, f, f, 5120, 1536, f, 1536, f, 1 << 20, None]
    assert lib.dmoe_grouped_gemm_gateup(7, *args) == L._lib.DMOE_ERR_UNSUPPORTED
    bad_h = list(args)
    bad_h[13] = 5000  # H not a multiple of 128
    assert lib.dmoe_grouped_gemm_gateup(1, *bad_h) == L._lib.DMOE_ERR_INVALID_ARG
    small_ws = list(args)
    small_ws[18] = 16
    assert lib.dmoe_grouped_gemm_gateup(2, *small_ws) == L._lib.DMOE_ERR_WORKSPACE


def test_gemm_rejects_operands_spanning_4gib(L):
    """The tile GEMM addresses operands as base + 32-bit offset; larger spans are refused before any launch."""
    lib = L.lib()
    f = 0x1000
    BF16 = 1
    max_rows, ldh = 2_000_000, 4096  # 2e6 rows x 4096 x 2 B = 16 GB of h
    ws = lib.dmoe_gemm_ws_bytes(max_rows, 256)
    st = lib.dmoe_grouped_gemm_down(BF16, f, ldh, None, 0, f, 256, max_rows, f, 1536, None, 1536, 5120, f, 5120, f,
                                    ws, None)
    assert st == L._lib.DMOE_ERR_UNSUPPORTED
    assert b"4 GiB" in lib.dmoe_last_error()
    # the same call with a small row bound passes validation up to the workspace check
    st = lib.dmoe_grouped_gemm_down(BF16, f, ldh, None, 0, f, 256, 512, f, 1536, None, 1536, 5120, f, 5120, f, 16,
                                    None)
    assert st == L._lib.DMOE_ERR_WORKSPACE
    # one expert's gate/up block of 1536 rows x 2^21 BF16 columns = 6.4 GB
    ws = lib.dmoe_gemm_ws_bytes(512, 256)
    st = lib.dmoe_grouped_gemm_gateup(BF16, f, 5120, None, 0, f, f, 256, 512, f, f, 1 << 21, None, None, 5120, 1536,
                                      f, 1536, f, ws, None)
    assert st == L._lib.DMOE_ERR_UNSUPPORTED


def test_forward_desc_validation_and_sizes(L):
    d = L.LayerDesc(8192, 5120, 1536, 1536, 256, 256, 0, 8, 8192, 2, 0)
    n = L.dmoe_forward_ws_bytes(d)
    # o [M, H] BF16 dominates: at least T*K*H*2 bytes
    assert n >= 8192 * 8 * 5120 * 2
    assert L.dmoe_forward_ws_offset(d, 0) == 0
    bad = L.LayerDesc(64, 5120, 1536, 1536, 256, 32, 240, 8, 64, 1, 0)  # local experts past E
    assert L.dmoe_forward_ws_bytes(bad) == 0
    lib = L.lib()
    st = lib.dmoe_forward(ctypes.byref(bad), None, None, 0, None)
    assert st == L._lib.DMOE_ERR_INVALID_ARG
    assert b"local experts" in lib.dmoe_last_error()
    bf = L.LayerDesc(64, 5120, 1536, 1536, 256, 256, 0, 8, 64, 1, 0)
    assert L.dmoe_forward_ws_offset(bf, 4) == -1  # no FP8 codes on the BF16 path
    ptrs = L.LayerPtrs()
    st = lib.dmoe_forward(ctypes.byref(bf), ctypes.byref(ptrs), None, 0, None)
    assert st == L._lib.DMOE_ERR_INVALID_ARG  # x is NULL; rejected before any launch


def test_forward_names_its_gate_up_kernel(L):
    # the launcher's rule, host side only: weight streaming up to 32 rows per expert by the host bound
    # ceil(T*K / E_loc); FP8 gate/up on the two-workgroup tile kernel below 512 rows per expert and on the
    # wide kernel (h quantised in its epilogue) from there with enough work items; BF16 on the wide kernel
    # from 128 rows per expert with enough work items
    def name(T, H, F, Fs, E, E_loc, K, Ts, dtype):
        return L.dmoe_forward_gateup_kernel(L.LayerDesc(T, H, F, Fs, E, E_loc, 0, K, Ts, dtype, 0))
    FP8, BF16 = L._lib.DMOE_FP8_E4M3, L._lib.DMOE_BF16
    assert name(64, 5120, 1536, 1536, 256, 256, 8, 64, BF16) == "gemm_stage_kernel"
    assert name(8192, 5120, 1536, 1536, 256, 256, 8, 8192, FP8) == "gemm_tile_kernel"
    assert name(16384, 5120, 1536, 1536, 256, 32, 8, 2048, FP8) == "gemm_wide_kernel"
    assert name(4096, 1536, 2112, 0, 64, 64, 8, 0, BF16) == "gemm_wide_kernel"
    assert name(4096, 1536, 2112, 0, 64, 64, 8, 0, FP8) == "gemm_wide_kernel"
    assert name(4096, 1536, 2112, 0, 128, 128, 8, 0, FP8) == "gemm_tile_kernel"  # 256 rows per expert
    assert name(2048, 5120, 1400, 1400, 256, 256, 8, 2048, FP8) == "gemm_tile_kernel"
    import test_gpu_layer as gl
    for case in ("wide_gateup_fp8", "wide_gateup_ep_fp8", "wide_gateup_nondiv_fp8", "wide_gateup_bf16"):
        c = gl.CASES[case]
        dt = FP8 if c.dtype == "fp8" else BF16
        assert name(c.T, c.H, c.F, c.F_s, c.E, c.E_loc, c.K, c.T_s, dt) == "gemm_wide_kernel", case
    bad = L.LayerDesc(64, 5120, 1536, 1536, 256, 32, 240, 8, 64, 1, 0)  # local experts past E
    assert L.dmoe_forward_gateup_kernel(bad) is None
    assert L.dmoe_forward_down_kernel(bad) is None


def test_forward_names_its_down_kernel(L):
    # down: weight streaming up to 32 rows per expert by the host bound, the wide kernel from 128 rows per
    # expert with at least 1024 (256-row tile, 256-column block) work items, else the two-workgroup kernel
    def name(T, H, F, Fs, E, E_loc, K, Ts, dtype):
        return L.dmoe_forward_down_kernel(L.LayerDesc(T, H, F, Fs, E, E_loc, 0, K, Ts, dtype, 0))
    FP8, BF16 = L._lib.DMOE_FP8_E4M3, L._lib.DMOE_BF16
    assert name(64, 5120, 1536, 1536, 256, 256, 8, 64, BF16) == "gemm_stage_kernel"  # decode
    assert name(128, 5120, 1536, 1536, 256, 256, 8, 128, FP8) == "gemm_stage_kernel"  # verify
    assert name(8192, 5120, 1536, 1536, 256, 256, 8, 8192, FP8) == "gemm_wide_kernel"  # prefill
    assert name(16384, 5120, 1536, 1536, 256, 32, 8, 2048, FP8) == "gemm_wide_kernel"  # EP share
    assert name(2048, 5120, 1400, 1400, 256, 256, 8, 2048, FP8) == "gemm_tile_kernel"  # 64 rows per expert
    assert name(4096, 5120, 13824, 0, 1, 1, 1, 0, FP8) == "gemm_tile_kernel"  # dense FFN: 340 work items
    assert name(4096, 1536, 2112, 0, 64, 64, 8, 0, BF16) == "gemm_wide_kernel"  # vision
    # the reduced parity cases meant for the wide kernel, and the many-tile ones that stay on the tile kernel
    import test_gpu_layer as gl
    for case, kernel in (("wide_down_fp8", "gemm_wide_kernel"), ("wide_down_bf16", "gemm_wide_kernel"),
                         ("many_tiles_fp8", "gemm_tile_kernel"), ("many_tiles_bf16", "gemm_tile_kernel")):
        c = gl.CASES[case]
        dt = FP8 if c.dtype == "fp8" else BF16
        assert name(c.T, c.H, c.F, c.F_s, c.E, c.E_loc, c.K, c.T_s, dt) == kernel, case


def test_combine_rejects_bad_slot_count_and_width(L):
    lib = L.lib()
    f = 0x1000
    assert lib.dmoe_combine(f, 5120, f, f, None, 0, 0, 64, 65, 5120, f, 5120, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert b"K = 65" in lib.dmoe_last_error()
    assert lib.dmoe_combine(f, 5120, f, f, None, 0, 0, 64, 8, 5124, f, 5124, None) == L._lib.DMOE_ERR_INVALID_ARG
    assert lib.dmoe_combine(None, 5120, None, None, None, 0, 0, 0, 8, 5120, None, 5120, None) == 0  # T == 0


def test_route_grouped_rejects_bad_groups(L):
    lib = L.lib()
    f = 0x1000
    bad = L._lib.DMOE_ERR_INVALID_ARG
    assert lib.dmoe_route_grouped(f, 4, 256, 8, 3, 1, 1, 1.0, f, f, None) == bad    # 256 % 3 != 0
    assert b"n_group = 3" in lib.dmoe_last_error()
    assert lib.dmoe_route_grouped(f, 4, 256, 8, 8, 9, 1, 1.0, f, f, None) == bad    # topk_group > n_group
    assert lib.dmoe_route_grouped(f, 4, 64, 8, 16, 1, 1, 1.0, f, f, None) == bad    # K=8 > 1 group of 4 experts
    assert lib.dmoe_route_grouped(f, 4, 64, 8, 8, 4, 1, -1.0, f, f, None) == bad    # scaling must be positive
    assert lib.dmoe_route_grouped(f, 4, 64, 8, 128, 4, 1, 1.0, f, f, None) == bad   # n_group > 64
    assert lib.dmoe_route_grouped(None, 0, 64, 8, 8, 4, 0, 2.5, None, None, None) == 0  # T == 0
