"""Benchmark of the MoE layer's hot path on one MI355X.

One step = the whole layer on one batch: route (router GEMM, top-k softmax,
plan) [+ token rounding], permute, grouped SwiGLU expert GEMMs, combine, and
the full backward.  Inputs are synthetic (seeded), already resident in HBM when
the timed region starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config fine_e128]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd+bwd at 1 GPU; grouped-GEMM % MFMA peak; permute GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 (MXFP8) MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 256 << 20


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_layer_fine_e128_forward_gemm_hbm_traffic.md")


def recorded_traffic(workload):
    """Calibrated HBM bytes per forward expert-GEMM call from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None when that summary is for another
    workload or the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith((" ", "|", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("workload") != workload:
            return None
        h = hashlib.sha256()
        for src in kv["kernel_sources"].split():
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != kv["kernel_sources_sha256"]:
            return None
        return float(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="fine_e128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-gather", choices=("auto", "on", "off"), default="auto",
                    help="on: the forward reads x through the plan inside the expert GEMMs (bf16) or the MXFP8 "
                         "quantiser (no x_perm); off: x is permuted once and x_perm handed to the backward; "
                         "auto (default): on for MXFP8 expert GEMMs, off for bf16")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = automatic)")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (reference for the HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(cfg, g, tokens):
    """The CPU oracle (float64 numpy, contract precision) on the first `tokens`
    tokens of the same workload: forward + backward, timed on the host cores."""
    import numpy as np
    import threadpoolctl
    from oracle import moe_oracle as mo

    f = lambda t: None if t is None else t.double().numpy()
    x = f(g["x"][:tokens])
    dout = f(g["dout"][:tokens]) if "dout" in g else None
    wg, b, w1, w2 = f(g["w_gate"]), f(g.get("bias")), f(g["w1"]), f(g["w2"])
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    mo.layer(x, wg, b, w1, w2, cfg.k, dout=dout, round_tile=cfg.round_tile,
             prec=mo.MX_CONTRACT if cfg.gemm == "mxfp8" else (mo.CONTRACT if cfg.act == "bf16" else mo.TRUTH))
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {tokens} of {cfg.T} tokens of {cfg.name} (same weights), fwd+bwd, "
                      f"float64 numpy{', MXFP8 operands' if cfg.gemm == 'mxfp8' else ''}, {dt:.1f} s"}


def activation_bytes(cfg, rows, plan_bytes, fwd_ws_bytes):
    """Bytes one layer keeps alive from the forward to the backward (weights and
    their gradients excluded).  The conventional layer keeps X_perm, H, A and the
    expert outputs Y, because it takes the router-score gradient as <dO, Y>; this
    one takes it as <dA', A> with A recomputed from H (SonicMoE article, section
    1), so it needs only the layer input x, the routing plan and H.  Handing the
    backward the forward's x_perm (and, with MXFP8, the forward workspace with
    the backward-orientation codes) keeps those alive too, to save work."""
    e = 2 if cfg.act == "bf16" else 4
    x, x_perm = cfg.T * cfg.d * e, rows * cfg.d * e
    H, A, Y = rows * 2 * cfg.f * e, rows * cfg.f * e, rows * cfg.d * e
    minimal = x + plan_bytes + H
    store_y = x + plan_bytes + x_perm + H + A + Y
    return {"minimal": minimal, "with_x_perm": minimal + x_perm, "store_y_layer": store_y,
            "saving_minimal_vs_store_y": 1.0 - minimal / store_y,
            # MXFP8: the forward workspace handed to the backward (codes of x_perm, A and of
            # both weights in both orientations)
            "forward_workspace": fwd_ws_bytes if cfg.gemm == "mxfp8" else 0}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_27_amd import binding, configs, synth

    if a.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)
        return

    cfg = configs.get(a.config)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    g = synth.generate(cfg)
    # bf16 default: permute x once and hand x_perm to the backward (the backward reads dout through
    # the plan inside its GEMMs either way).  MXFP8 default: the forward quantiser reads x through
    # the plan (it writes both code orientations the backward reuses, so x_perm is never needed)
    want = a.fused_gather == "on" or (a.fused_gather == "auto" and cfg.gemm == "mxfp8")
    fused = want and cfg.act == "bf16" and cfg.T * cfg.d * 2 < 2 ** 31
    run = binding.LayerRun(cfg, g, fused_gather=fused)
    s = run.s
    stream = torch.cuda.current_stream()

    phases = ["route", "permute", "experts", "combine", "backward"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        run.route()
        mark(1)
        if not fused:
            binding.permute(s, run.inp["x"], run.plan, run.x_perm)
        mark(2)
        if fused:
            binding.grouped_gemm_swiglu_gather(s, run.inp["x"], run.inp["w1"], run.inp["w2"], run.plan, run.h, run.y,
                                               run.ws_fwd)
        else:
            binding.grouped_gemm_swiglu(s, run.x_perm, run.inp["w1"], run.inp["w2"], run.plan, run.h, run.y,
                                        run.ws_fwd)
        mark(3)
        binding.unpermute_combine(s, run.y, run.plan, run.out)
        mark(4)
        if run.has_bwd:
            run.backward(with_optional=False)
        mark(5)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(a.steps)]
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {p: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(a.steps)) / a.steps
          for j, p in enumerate(phases)}
    step_ms = sum(evs[i][0].elapsed_time(evs[i][5]) for i in range(a.steps)) / a.steps
    ms_per_step = wall * 1000.0 / a.steps
    step_q = sorted(evs[i][0].elapsed_time(evs[i][5]) for i in range(a.steps))
    pct = lambda q: step_q[min(len(step_q) - 1, int(round(q * (len(step_q) - 1))))]

    # data-movement rates with cold caches: a 1 GiB scratch write before each
    # timed launch evicts L2 and the 256 MB last-level cache
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def cold_ms(fn, n=5):
        t = []
        for _ in range(n):
            flush_buf.fill_(1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    # moe_permute on its own (outside the step when it is fused into the GEMMs)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        binding.permute(s, run.inp["x"], run.plan, run.x_perm)
    pev[0].record(stream)
    for _ in range(10):
        binding.permute(s, run.inp["x"], run.plan, run.x_perm)
    pev[1].record(stream)
    torch.cuda.synchronize()
    permute_ms = pev[0].elapsed_time(pev[1]) / 10
    permute_cold_ms = cold_ms(lambda: binding.permute(s, run.inp["x"], run.plan, run.x_perm))

    N = cfg.N  # rows without rounding (algorithmic work)
    counts = run.plan.arrays()["counts"].cpu()
    rows = int(counts.sum())
    esz = 2 if cfg.act == "bf16" else 4
    # practical HBM rate of a plain device-to-device copy of the permutation's size
    # (reference for the data-movement kernels, not part of the layer)
    cbytes = (cfg.T + rows) * cfg.d * esz // 2 // 16 * 16
    csrc = torch.empty(cbytes, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        cdst.copy_(csrc)
    pev[0].record(stream)
    for _ in range(10):
        cdst.copy_(csrc)
    pev[1].record(stream)
    torch.cuda.synchronize()
    copy_GBps = 2 * cbytes / (pev[0].elapsed_time(pev[1]) / 10 * 1e-3) / 1e9
    copy_cold_ms = cold_ms(lambda: cdst.copy_(csrc))
    del csrc, cdst, flush_buf
    fwd_gemm_flops = 2.0 * rows * cfg.d * 2 * cfg.f + 2.0 * rows * cfg.f * cfg.d
    peak = {"mxfp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS}.get(cfg.gemm, PEAK_F32_TFLOPS)
    achieved = fwd_gemm_flops / (ms["experts"] * 1e-3) / 1e12
    permute_bytes = cfg.T * cfg.d * esz + rows * cfg.d * esz + 4 * (cfg.T + 1) + 4 * rows
    combine_bytes = rows * cfg.d * esz + cfg.T * cfg.d * esz + 8 * rows
    bwd_flops = 2 * fwd_gemm_flops
    out = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp8": "mxfp8", "bf16": "bf16"}.get(cfg.gemm, "f32"),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d_model={cfg.d} E={cfg.E} top-k={cfg.k} "
                               f"d_ff={cfg.f} SwiGLU, {'fwd+bwd' if run.has_bwd else 'fwd'}"
                               f"{', token rounding ' + str(cfg.round_tile) if cfg.round_tile else ''}",
                   "global_batch": cfg.T, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "forward expert GEMMs (up+SwiGLU, down) in one call",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": recorded_traffic(cfg.name), "traffic_unit": "HBM bytes per call"},
        "phases_ms": ms,
        "events_ms_per_step": step_ms,
        "grouped_gemm_mfma_frac": {"forward": achieved / peak,
                                   "backward_call": bwd_flops / (ms["backward"] * 1e-3) / 1e12 / peak
                                   if run.has_bwd else None},
        "permute_GBps": permute_bytes / (permute_ms * 1e-3) / 1e9,
        "permute_fused_into_gemms": fused,
        "combine_GBps": combine_bytes / (ms["combine"] * 1e-3) / 1e9,
        "hbm_peak_GBps": PEAK_HBM_GBS,
        "device_copy_GBps": copy_GBps,
        "cold_cache_GBps": {"permute": permute_bytes / (permute_cold_ms * 1e-3) / 1e9,
                            "device_copy": 2 * cbytes / (copy_cold_ms * 1e-3) / 1e9,
                            "note": "median of 5 launches, each after a 1 GiB scratch write"},
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "rows": rows,
        "max_expert_rows": int(counts.max()),
        "activation_memory_bytes": activation_bytes(cfg, rows, binding.plan_bytes(s), run.ws_fwd.numel())
        if run.has_bwd else None,
    }
    if not a.no_cpu_baseline:
        del run
        torch.cuda.empty_cache()
        tokens = a.cpu_tokens or max(1, min(cfg.T, 16384))
        print(f"[bench] cpu oracle on {tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, g, tokens)
    line = json.dumps(out)
    print(line, flush=True)
    if a.out:
        with open(a.out, "a") as fh:
            fh.write(line + "\n")


if __name__ == "__main__":
    main()
