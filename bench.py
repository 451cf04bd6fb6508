#!/usr/bin/env python3
"""MoE-layer throughput of libdmoe on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]
    python bench.py --copy-calibration MIB [--steps REPS]

A step is one dmoe_forward over one batch of synthetic input: router logits
(or given logits) -> route -> permute -> [quantise x] -> gate/up + SwiGLU ->
[quantise h] -> down -> shared expert -> combine. Inputs and weights are
resident in HBM before the timed region. The default workload is the FP8
prefill chunk at full dots3-note shape (T=8192 tokens, hidden 5120, 256 routed
+ 1 shared experts, top-8, expert FFN 1536, E4M3 weights with 128x128 block
scales and dynamic 1x128 activation scales); --workload 1 is the BF16 decode
layer (T=64). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import hashlib
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s / FP8 TFLOP/s vs peak, 1 MI355X"
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def build_layer(cfg, dev):
    import synth
    from fp8_expert_ffn_amd import MoELayer
    layer = MoELayer(cfg.H, cfg.F, cfg.F_s, cfg.E, cfg.E_loc, cfg.e0, cfg.K, cfg.dtype, dev, n_group=cfg.n_group,
                     topk_group=cfg.topk_group, renormalize=cfg.renormalize, routed_scaling_factor=cfg.scaling,
                     scoring=cfg.scoring)
    if cfg.scoring == "sigmoid":
        layer.set_score_bias(synth.score_bias(cfg))
    bf16 = cfg.dtype == "bf16"
    for which in ("gate", "up", "down"):
        synth.fill_expert_weights(cfg, which, cfg.experts, lambda i, a, w=which: layer.set_weight(w, i, a), bf16)
        if cfg.F_s:
            draw = synth.expert_weight_bf16 if bf16 else synth.expert_weight_f32
            layer.set_weight(which, -1, draw(cfg, which, synth.SHARED))
    return layer


def shared_fused(cfg) -> bool:
    """The shared expert runs inside the routed launches when it has the routed width."""
    return cfg.T_s > 0 and cfg.F_s > 0 and cfg.F_s == cfg.F


def kernel_files(kernel: str) -> list[str]:
    csrc = os.path.join(ROOT, "fp8_expert_ffn_amd", "csrc")
    main = {"gemm_stage_kernel": "gemm_stream.hip", "gemm_tile_kernel": "gemm.hip",
            "gemm_wide_kernel": "gemm_wide.hip"}[kernel]
    return [os.path.join(csrc, f) for f in (main, "gemm_common.h", "dmoe_device.h", "dmoe_internal.h")]


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in kernel_files(kernel):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(workload: str, kernel: str, src_hash: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (copy-calibrated), from the
    committed profile summaries; None when no record matches this workload, kernel and kernel source."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(pdir, name)) as fh:
            for line in fh:
                if not line.startswith("traffic-record: "):
                    continue
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("workload") == workload and rec.get("kernel") == kernel and \
                        rec.get("source_sha256") == src_hash:
                    return rec
    return None


def copy_calibration(mib: int, reps: int) -> int:
    """A plain device-to-device copy of `mib` MiB, `reps` times: the reference for scaling the HBM counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)
    return 0


def accounting(cfg, offsets: np.ndarray, logits_computed: bool) -> dict:
    """Algorithmic FLOPs and bytes of the layer and of its gate/up launch, on the real routing."""
    es = 1 if cfg.dtype == "fp8" else 2
    counts = np.diff(offsets)
    M = int(offsets[-1])
    touched = int((counts > 0).sum())
    H, F, Fs, T, Ts, E = cfg.H, cfg.F, cfg.F_s, cfg.T, cfg.T_s, cfg.E
    nb = lambda n: -(-n // 128)  # noqa: E731
    sc = 4 if cfg.dtype == "fp8" else 0  # FP8 block scales (FP32 per 128x128 block)
    w_gu = 2 * (F * H * es + nb(F) * nb(H) * sc)          # one expert's gate + up
    w_d = H * F * es + nb(H) * nb(F) * sc
    ws_gu = 2 * (Fs * H * es + nb(Fs) * nb(H) * sc) if Fs and Ts else 0
    ws_d = (H * Fs * es + nb(H) * nb(Fs) * sc) if Fs and Ts else 0
    flops = 2.0 * M * 3 * H * F + (2.0 * Ts * 3 * H * Fs if Fs else 0.0)
    if logits_computed:
        flops += 2.0 * T * H * E
    bytes_ = touched * (w_gu + w_d) + ws_gu + ws_d + T * H * 2 + T * H * 2  # weights + x read + y written
    bytes_ += E * H * 4 if logits_computed else T * E * 4                  # router weight or given logits
    # gate/up launch: routed experts, plus the shared expert when it runs as an extra group of that launch
    a_bytes = T * H * es + (T * nb(H) * 4 if cfg.dtype == "fp8" else 0)     # x (codes + scales) read once
    gu_rows = M + (Ts if shared_fused(cfg) else 0)
    gu_flops = 2.0 * gu_rows * 2 * H * F
    gu_bytes = touched * w_gu + (ws_gu if shared_fused(cfg) else 0) + a_bytes + gu_rows * F * 2  # + h written
    return dict(M=M, touched=touched, flops=flops, bytes=bytes_, gu_flops=gu_flops, gu_bytes=gu_bytes,
                gu_rows=gu_rows)


def cpu_baseline(cfg, x_bits, wr, given, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload's tokens.

    Returns the baseline record and the oracle's results (one per sampled batch) for the parity check."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    get = (lambda w, e: synth.expert_weight_f32(cfg, w, e)) if cfg.dtype == "fp8" else \
        (lambda w, e: synth.expert_weight_bf16(cfg, w, e))
    rng = np.random.default_rng(7)
    done, n, t0 = 0, 2, time.perf_counter()
    results = []
    while True:
        tok = np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False))
        results.append(oracle.moe_forward(cfg, x_bits, get, w_r=wr, logits=given, tokens=tok,
                                          score_bias=synth.score_bias(cfg) if cfg.scoring == "sigmoid" else None))
        done += tok.size
        el = time.perf_counter() - t0
        if el >= seconds or done >= cfg.T:
            break
        n = min(cfg.T, max(1, int(tok.size * max(1.0, (seconds - el) / max(el, 1e-3)) * 0.5)))
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    rec = {"value": done / el, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
           "host_cpu_count": os.cpu_count(), "host_affinity": affinity,
           "sample": f"{done} tokens of the {cfg.name} workload (random token subsets, each token's full "
                     f"layer output incl. per-expert weight preparation), {el:.1f}s on "
                     f"{platform.processor() or platform.machine()}; BLAS threads {blas}, elementwise NumPy "
                     f"single-threaded"}
    return rec, results


def sample_parity(cfg, results, y_gpu: np.ndarray, ids_gpu: np.ndarray) -> dict:
    """GPU output of the timed layer against the oracle on the cpu_baseline's sampled tokens. Tokens whose top-K
    set differs (router near-ties between the GPU's FP32 logits and the oracle's) are left out and counted.
    Bound: relative L2 <= 5e-3 against the oracle's BF16 y, and every element within 2e-2 RMS plus half a BF16
    ulp (the GPU's own final rounding) of the oracle's unrounded float64 sum, plus the oracle's rounding
    allowance where an expert output sits on a BF16 rounding midpoint."""
    tok = np.concatenate([r.tokens for r in results])
    y_or = np.concatenate([r.y for r in results])
    y_sum = np.concatenate([r.y_sum for r in results])
    y_allow = np.concatenate([r.y_allow for r in results])
    ids_or = np.concatenate([r.ids for r in results])
    same = np.all(np.sort(ids_gpu[tok], 1) == np.sort(ids_or, 1), axis=1)
    yg, yo, ys, ya = y_gpu[tok][same], y_or[same], y_sum[same], y_allow[same]
    if yo.size == 0:
        return {"tokens": 0}
    rms = float(np.sqrt(np.mean(yo ** 2)))
    a = np.maximum(np.abs(yg), np.abs(ys))
    half_ulp = np.where(a > 0, np.ldexp(1.0, np.maximum(np.frexp(a)[1] - 9, -134)), 0.0)
    worst = float(np.max(np.abs(yg - ys) / np.maximum(2e-2 * rms + half_ulp + ya, 1e-300)))
    rel = float(np.linalg.norm(yg - yo) / max(np.linalg.norm(yo), 1e-300))
    return {"tokens": int(same.sum()), "routing_near_ties_skipped": int((~same).sum()),
            "rel_l2": rel, "max_abs_over_rms": float(np.abs(yg - yo).max() / max(rms, 1e-300)),
            "max_err_over_bound": worst, "pass": bool(rel <= 5e-3 and worst <= 1.0),
            "bound": "rel_l2 <= 5e-3; every element |y - y_sum| <= 2e-2 RMS + ulp_bf16/2 + allowance (y_sum: the "
                     "oracle's unrounded combine sum; allowance: weight x BF16 spacing of expert outputs on a "
                     "rounding midpoint)"}


def bit_exact(cfg, layer, d, ws, out, x_bits: np.ndarray) -> dict:
    """Integer and byte results of the timed layer against the oracle at the full workload size: the top-K ids
    from the GPU's own logits (the oracle routes the same FP32 logits), the routing weights (tolerance 1e-6), the
    permutation tables of those ids and, for FP8, the codes and scales of x."""
    import oracle
    import synth
    L = out["logits"].cpu().numpy()
    ids_gpu = out["topk_ids"].cpu().numpy()
    w_gpu = out["topk_w"].cpu().numpy()
    ropts = dict(n_group=cfg.n_group, topk_group=cfg.topk_group or None, renormalize=cfg.renormalize,
                 scaling=cfg.scaling)
    if cfg.scoring == "sigmoid":
        ids_or, w_or = oracle.route_sigmoid(L, cfg.K, bias=synth.score_bias(cfg), **ropts)
    else:
        ids_or, w_or = oracle.route(L, cfg.K, **ropts)
    off, rt, rs, tr = oracle.permute(ids_gpu, cfg.e0, cfg.E_loc)
    m = int(off[-1])
    view = lambda name: layer.ws_view(d, ws, name).cpu().numpy()  # noqa: E731
    rec = {"ids": bool(np.array_equal(ids_gpu, ids_or)),
           "weights_max_abs_diff": float(np.max(np.abs(w_gpu.astype(np.float64) - w_or))),
           "perm": bool(np.array_equal(view("offsets"), off) and np.array_equal(view("row_token")[:m], rt)
                        and np.array_equal(view("row_slot")[:m], rs) and np.array_equal(view("token_row"), tr))}
    if cfg.dtype == "fp8":
        q, sc = oracle.quantize_act((x_bits.astype(np.uint32) << 16).view(np.float32))
        rec["x_codes"] = bool(np.array_equal(view("x_codes"), q))
        rec["x_scales"] = bool(np.array_equal(view("x_scales").view(np.uint32), sc.view(np.uint32)))
    rec["pass"] = bool(rec["ids"] and rec["perm"] and rec["weights_max_abs_diff"] <= 1e-6
                       and rec.get("x_codes", True) and rec.get("x_scales", True))
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="workload index (0 tiny, 1 decode, 2 prefill, "
                                                                "3 EP share, 4 non-divisible, 5 vision BF16, "
                                                                "6 vision FP8, 7 dense FFN FP8, "
                                                                "8/9 speculative verify batch BF16/FP8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer captured once in a HIP graph and replayed (decode-style serving)")
    ap.add_argument("--tokens", type=int, default=0, metavar="T",
                    help="run the workload's layer with T tokens instead of its own (the shared expert then takes "
                         "min(T, its T_s) tokens, all of them when it took all before)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the multi-GPU exchange "
              f"is not part of this library)", file=sys.stderr)
        return 2

    import torch
    import synth
    import fp8_expert_ffn_amd as dm
    from fp8_expert_ffn_amd import _lib as dml

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, max(1, args.steps))
    cfg = synth.config(args.workload)
    if args.tokens > 0:
        t_s = args.tokens if cfg.T_s == cfg.T else min(cfg.T_s, args.tokens)
        cfg = cfg.replace(name=f"{cfg.name}_T{args.tokens}", T=args.tokens, T_s=t_s)
    t0 = time.time()
    layer = build_layer(cfg, dev)
    x_bits = synth.x_bf16(cfg)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if cfg.logits == "router":
        wr, given = synth.router_weight(cfg), None
        kw = dict(w_router=torch.from_numpy(wr).to(dev))
    else:
        wr, given = None, synth.given_logits(cfg)
        kw = dict(logits=torch.from_numpy(given).to(dev))
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: weights and inputs resident after {time.time() - t0:.1f}s")

    d, p, ws, out = layer.make_call(x, cfg.T_s, **kw)
    stream = torch.cuda.current_stream()
    nstage = dm.DMOE_STAGES + 1
    gu = dm.STAGE_NAMES.index("gateup")
    for _ in range(args.warmup):
        dm.dmoe_forward(d, p, ws)
    torch.cuda.synchronize()

    def make_events(n, which):
        evs = [[torch.cuda.Event(enable_timing=True) if s in which else None for s in range(nstage)]
               for _ in range(n)]
        for row in evs:
            for e in row:
                if e is not None:
                    e.record(stream)  # creates the underlying HIP event
        return evs

    # Timed region: K layer calls; only the gate/up launch is bracketed by events (each recorded event is a
    # stream marker of a few microseconds, so the other stage boundaries are left out of this region).
    ev = make_events(args.steps, {gu, gu + 1})
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        dm.dmoe_forward_timed(d, p, ws, ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    ms_step = start.elapsed_time(end) / args.steps
    gu_ms = float(np.mean([ev[i][gu].elapsed_time(ev[i][gu + 1]) for i in range(args.steps)]))
    # per-step layer times: from one step's gate/up start to the next one's (no extra markers)
    step_ms = np.array([ev[i][gu].elapsed_time(ev[i + 1][gu]) for i in range(args.steps - 1)])
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (host {1e3 * (h1 - h0) / args.steps:.4f} ms/step), "
        f"gate/up launch {gu_ms:.4f} ms")

    # Per-stage breakdown (separate pass, events at every stage boundary; not part of the timed region).
    nb = min(args.steps, 20)
    evb = make_events(nb, set(range(nstage)))
    torch.cuda.synchronize()
    for i in range(nb):
        dm.dmoe_forward_timed(d, p, ws, evb[i])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([evb[i][s].elapsed_time(evb[i][s + 1]) for i in range(nb)]))
                for s, name in enumerate(dm.STAGE_NAMES)}
    log("[bench] stages (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))

    graph_rec = None
    if args.graph:
        # One dmoe_forward captured on a side stream, then replayed K times on the current stream.
        y_eager = out["y"].clone()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                dm.dmoe_forward(d, p, ws)
        stream.wait_stream(side)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        same = bool(torch.equal(out["y"].view(torch.int16), y_eager.view(torch.int16)))
        graph_rec = {"ms_per_step": round(gms, 5), "value": round(cfg.T / (gms / 1e3), 1), "unit": "tokens/s",
                     "replays": args.steps, "output_identical_to_eager": same}
        log(f"[bench] graph replay: {gms:.4f} ms/step (eager {ms_step:.4f}); output identical: {same}")

    offsets = layer.ws_view(d, ws, "offsets").cpu().numpy()
    acc = accounting(cfg, offsets, cfg.logits == "router")
    sec = ms_step / 1e3
    gu_sec = gu_ms / 1e3
    # Every gate/up launch multiplies on BF16 matrix cores: FP8 operands are converted exactly to BF16 first
    # (exact E4M3 products), so the contraction's own peak is the BF16 one; the FP8 fraction is reported too.
    gu_peak = PEAK_TFLOPS["bf16"]
    gu_time_hbm = acc["gu_bytes"] / (PEAK_HBM_GBPS * 1e9)
    gu_time_mfma = acc["gu_flops"] / (gu_peak * 1e12)
    ach_hbm = acc["gu_bytes"] / gu_sec / 1e9
    ach_mfma = acc["gu_flops"] / gu_sec / 1e12
    hbm_side = {"achieved": round(ach_hbm, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach_hbm / PEAK_HBM_GBPS, 4)}
    mfma_side = {"achieved": round(ach_mfma, 1), "peak": gu_peak, "unit": "TFLOP/s",
                 "frac": round(ach_mfma / gu_peak, 4), "mfma": "bf16 (exact products of the E4M3 codes)"
                 if cfg.dtype == "fp8" else "bf16"}
    if cfg.dtype == "fp8":
        mfma_side["frac_of_fp8_peak"] = round(ach_mfma / PEAK_TFLOPS["fp8"], 4)
    # the binding resource at peak rates decides `bound`; the other side is reported next to it
    if gu_time_hbm >= gu_time_mfma:
        roof = {"bound": "hbm", **hbm_side, "traffic": None, "other_roof": {"bound": "mfma", **mfma_side}}
    else:
        roof = {"bound": "mfma", **mfma_side, "traffic": None, "other_roof": {"bound": "hbm", **hbm_side}}
    kbase = dml.dmoe_forward_gateup_kernel(d)  # the launcher's own choice for this layer
    kname = f"{kbase}<{cfg.dtype}, gate/up>"
    roof["kernel"] = kname + (" (routed experts + shared expert as an extra group)" if shared_fused(cfg)
                              else " (routed experts)")
    rec = traffic_record(cfg.name, kname, kernel_source_hash(kbase))
    if rec is not None:
        roof["traffic"] = rec["hbm_bytes_per_launch"]
        roof["traffic_source"] = rec["summary"]
    roof["alg_bytes_per_launch"] = acc["gu_bytes"]
    roof["alg_flops_per_launch"] = acc["gu_flops"]
    roof["avg_launch_ms"] = round(gu_ms, 5)

    result = {
        "metric": METRIC,
        "value": round(cfg.T / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)]
        if step_ms.size else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "F": cfg.F, "F_s": cfg.F_s, "E": cfg.E,
                   "E_loc": cfg.E_loc, "e0": cfg.e0, "K": cfg.K, "T_s": cfg.T_s, "logits": cfg.logits,
                   "M": acc["M"], "touched_experts": acc["touched"], "parallelism": "single GPU"},
        "layer": {"alg_bytes": acc["bytes"], "alg_flops": acc["flops"],
                  "GBps": round(acc["bytes"] / sec / 1e9, 1),
                  "TFLOPs": round(acc["flops"] / sec / 1e12, 2),
                  "frac_hbm": round(acc["bytes"] / sec / 1e9 / PEAK_HBM_GBPS, 4),
                  "frac_mfma": round(acc["flops"] / sec / 1e12 / PEAK_TFLOPS[cfg.dtype], 4)},
        "kernels": {"gateup": kbase, "down": dml.dmoe_forward_down_kernel(d)},
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stages_note": "separate pass with an event at every stage boundary (markers add a few us each)",
        "roofline": roof,
    }
    if graph_rec is not None:
        result["graph"] = graph_rec
    if not args.no_cpu_baseline:
        result["cpu_baseline"], results = cpu_baseline(cfg, x_bits, wr, given, args.cpu_seconds)
        y_gpu = out["y"].view(torch.int16).cpu().numpy().view(np.uint16)
        y_gpu = (y_gpu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        result["parity_sample"] = sample_parity(cfg, results, y_gpu, out["topk_ids"].cpu().numpy())
        result["bit_exact"] = bit_exact(cfg, layer, d, ws, out, x_bits)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
