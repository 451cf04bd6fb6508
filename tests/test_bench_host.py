"""Host-side logic of bench.py (no GPU): the algorithmic byte and FLOP
accounting of the layer and of its gate/up launch on a hand-counted example,
and the lookup of the committed counter records by workload, kernel and kernel
source hash."""
import json
import os

import numpy as np

import bench
import synth


def test_accounting_hand_counted_fp8_layer():
    # 4 tokens, hidden 128, FFN 128 (one 128x128 block per matrix), 2 experts with 3 and 1 rows, top-1, the
    # shared expert (same width) on all 4 tokens, so it runs inside the routed launches
    cfg = synth.LayerConfig("acct", T=4, H=128, F=128, F_s=128, E=2, E_loc=2, e0=0, K=1, dtype="fp8", T_s=4,
                            logits="uniform")
    acc = bench.accounting(cfg, np.array([0, 3, 4]), logits_computed=False)
    gate_up = 2 * (128 * 128 + 4)  # two E4M3 matrices and one FP32 block scale each
    down = 128 * 128 + 4
    assert acc["M"] == 4 and acc["touched"] == 2
    assert acc["flops"] == 2 * 4 * 3 * 128 * 128 + 2 * 4 * 3 * 128 * 128
    # two routed experts + the shared expert, x (BF16) read once, y (BF16) written once, the given FP32 logits
    assert acc["bytes"] == 2 * (gate_up + down) + gate_up + down + 4 * 128 * 2 + 4 * 128 * 2 + 4 * 2 * 4
    # gate/up launch: 4 routed + 4 shared rows, x codes + one scale per row read once, h (BF16) written
    assert acc["gu_rows"] == 8
    assert acc["gu_flops"] == 2 * 8 * 2 * 128 * 128
    assert acc["gu_bytes"] == 2 * gate_up + gate_up + (4 * 128 + 4 * 4) + 8 * 128 * 2
    # with the router: its FP32 weight instead of the logits, and its FLOPs
    acc_r = bench.accounting(cfg, np.array([0, 3, 4]), logits_computed=True)
    assert acc_r["bytes"] - acc["bytes"] == 2 * 128 * 4 - 4 * 2 * 4
    assert acc_r["flops"] - acc["flops"] == 2 * 4 * 128 * 2


def test_accounting_bf16_separate_shared_expert():
    # BF16, shared expert of another width on 2 of 5 tokens: not part of the gate/up launch, one untouched expert
    cfg = synth.LayerConfig("acct_bf16", T=5, H=256, F=64, F_s=96, E=3, E_loc=3, e0=0, K=2, dtype="bf16", T_s=2,
                            logits="uniform")
    acc = bench.accounting(cfg, np.array([0, 6, 6, 10]), logits_computed=False)
    assert acc["M"] == 10 and acc["touched"] == 2
    w_routed = 3 * 64 * 256 * 2
    w_shared = 3 * 96 * 256 * 2
    assert acc["bytes"] == 2 * w_routed + w_shared + 5 * 256 * 2 * 2 + 5 * 3 * 4
    assert acc["flops"] == 2 * 10 * 3 * 256 * 64 + 2 * 2 * 3 * 256 * 96
    assert acc["gu_rows"] == 10
    assert acc["gu_bytes"] == 2 * (2 * 64 * 256 * 2) + 5 * 256 * 2 + 10 * 64 * 2


def test_traffic_records_are_found_by_workload_kernel_and_source():
    pdir = os.path.join(bench.ROOT, "profiles")
    recs = []
    for name in sorted(os.listdir(pdir)):
        for line in open(os.path.join(pdir, name)):
            if line.startswith("traffic-record: "):
                recs.append(json.loads(line[len("traffic-record: "):]))
    assert recs, "no committed counter record"
    for rec in recs:
        for key in ("workload", "kernel", "source_sha256", "hbm_bytes_per_launch", "alg_bytes_per_launch",
                    "copy_fetch_factor", "copy_write_factor", "summary"):
            assert key in rec, key
        assert os.path.exists(os.path.join(bench.ROOT, rec["summary"]))
        assert bench.traffic_record(rec["workload"], rec["kernel"], rec["source_sha256"]) == rec
        assert bench.traffic_record(rec["workload"], rec["kernel"], "0" * 64) is None
        assert bench.traffic_record("no_such_workload", rec["kernel"], rec["source_sha256"]) is None
        # the bytes follow from the counters and the copy calibration (factors stored to 4 decimals)
        hbm = rec["fetch_kib_per_dispatch"] * 1024 * rec["copy_fetch_factor"] + \
            rec["write_kib_per_dispatch"] * 1024 * rec["copy_write_factor"]
        assert abs(hbm - rec["hbm_bytes_per_launch"]) <= 1e-4 * hbm
    # the kernel source hash covers the kernel's own file and the shared headers
    for k in ("gemm_stage_kernel", "gemm_tile_kernel", "gemm_wide_kernel"):
        files = bench.kernel_files(k)
        assert all(os.path.exists(f) for f in files) and len(bench.kernel_source_hash(k)) == 64
