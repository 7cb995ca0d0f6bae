"""Benchmark of the MoE layer's hot path on one MI355X.

One step = the whole layer on one batch: route (router GEMM, top-k softmax,
plan) [+ token rounding], permute, grouped SwiGLU expert GEMMs, combine, and
the full backward.  Inputs are synthetic (seeded), already resident in HBM when
the timed region starts.  Prints ONE JSON line.

The headline workload is the largest forward+backward one that fits one GPU
(sparse_e256: T=32768, d_model=4096, E=256, top-8, d_ff=512).  The other
workloads (coarse_e8 forward, fine_e128, its Zipf-imbalanced variant, the
token-rounded sparse_e256 and fine_e128 with MXFP8 expert GEMMs) are timed the
same way and reported under "sub_results".

Timing: W warm-up steps, then K timed steps bracketed by synchronisations;
each step's device time comes from HIP events on the compute stream and the
reported step time is the median (p10/p90 beside it).  The expert-GEMM call and
the backward run through their *_traced entry points, which record events
between their kernels, so every kernel's mean device time over the timed
steps is known; the roofline entry is for the kernel with the largest mean.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config sparse_e256] [--no-sub]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd+bwd at 1 GPU; grouped-GEMM % MFMA peak; permute GB/s"
HEADLINE = "sparse_e256"
SUB_CONFIGS = ("coarse_e8", "fine_e128", "fine_e128_zipf", "sparse_e256_round", "fine_e128_mxfp8", "sparse_e256_mxfp8",
               "fine_e128_router_losses", "fine_e128_zipf_capacity")
# workloads timed as one optimizer step over 4 micro-batches (bf16, MXFP8, MXFP8 with reused weight codes)
ACCUM_CONFIGS = ("fine_e128", "sparse_e256")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 (MXFP8) MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_layer_sparse_e256_dw1_hbm_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--no-sub", action="store_true", help="skip the other workloads")
    ap.add_argument("--sub-steps", type=int, default=30)
    ap.add_argument("--sub-warmup", type=int, default=5)
    ap.add_argument("--accum-steps", type=int, default=6, help="optimizer steps timed per gradient-accumulation run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-gather", choices=("auto", "on", "off"), default="auto",
                    help="on: the forward reads x through the plan inside the expert GEMMs (bf16) or the MXFP8 "
                         "quantiser, and the backward's dW1 reads x the same way (no x_perm); off: x is permuted "
                         "once and x_perm handed to the backward; auto (default): on wherever the row offsets "
                         "fit 32 bits")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = automatic)")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (reference for the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------- host facts


def gpu_clocks():
    """Shader/memory clocks and power from the SMI tools (whatever answers); not
    under a profiler, whose preloaded library would make the tools' interpreter
    start-up an exec after GPU initialisation."""
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], ["amd-smi", "metric", "-c", "-p", "--json"],
                ["rocm-smi", "--showclocks", "--showpower", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if r.returncode == 0 and r.stdout.strip():
            try:
                return {"tool": " ".join(cmd), **compact_clocks(json.loads(r.stdout))}
            except ValueError:
                return {"tool": " ".join(cmd), "reading": r.stdout.strip()[:500]}
    return None


def compact_clocks(reading):
    """Shader clock per XCD, memory clock and socket power out of an amd-smi
    metric reading; anything else is kept as (shortened) text."""
    try:
        gpu = (reading["gpu_data"] if isinstance(reading, dict) else reading)[0]
        clk = gpu["clock"]
        gfx = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_") and isinstance(clk[k], dict)
               and isinstance(clk[k].get("clk"), dict)]
        mem = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("mem_") and isinstance(clk[k], dict)
               and isinstance(clk[k].get("clk"), dict)]
        return {"gfx_clk_mhz_per_xcd": gfx, "mem_clk_mhz": mem[0] if mem else None,
                "socket_power_w": gpu["power"]["socket_power"]["value"]}
    except (KeyError, IndexError, TypeError):
        return {"reading": json.dumps(reading)[:500]}


def cpu_facts():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        import threadpoolctl
        for i in threadpoolctl.threadpool_info():
            blas.append({k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")})
    except Exception:
        pass
    return {"os_cpu_count": os.cpu_count(), "cpu_model": model, "blas": blas}


def cpu_baseline(cfg, g, tokens):
    """The CPU oracle (float64 numpy, contract precision) on the first `tokens`
    tokens of the same workload: forward + backward, timed on the host cores."""
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
            "sample": f"first {tokens} of {cfg.T} tokens of {cfg.name} (same weights, routed among themselves), "
                      f"fwd+bwd, float64 numpy{', MXFP8 operands' if cfg.gemm == 'mxfp8' else ''}, {dt:.1f} s",
            "seconds": dt, **cpu_facts()}


def recorded_traffic(workload, kernel):
    """Calibrated HBM bytes per launch of `kernel` on `workload` from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None when there is none or the kernel
    sources changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith((" ", "|", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("workload") != workload or kv.get("kernel") != kernel:
            return None
        h = hashlib.sha256()
        for src in kv["kernel_sources"].split():
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != kv["kernel_sources_sha256"]:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------- work per kernel


def kernel_work(cfg, rows):
    """Algorithmic work of one launch of each traced GEMM kernel: (flops, peak).
    rows = routed rows of the plan (each GEMM's M or K over all experts)."""
    d, f = cfg.d, cfg.f
    mx = cfg.gemm == "mxfp8"
    peak = PEAK_FP8_TFLOPS if mx else (PEAK_BF16_TFLOPS if cfg.gemm == "bf16" else PEAK_F32_TFLOPS)
    w = {"up_swiglu": 2.0 * rows * d * 2 * f, "down": 2.0 * rows * f * d, "dact": 2.0 * rows * d * f,
         "dx_perm": 2.0 * rows * 2 * f * d, "dw1": 2.0 * rows * 2 * f * d, "dw2": 2.0 * rows * d * f}
    out = {k: (v, peak) for k, v in w.items()}
    out.update({"mx_" + k: (v, peak) for k, v in w.items()})
    out["router_dwg"] = (2.0 * cfg.T * cfg.E * d, PEAK_BF16_TFLOPS if cfg.act == "bf16" else PEAK_F32_TFLOPS)
    return out


GEMM_KERNELS = ("up_swiglu", "down", "dact", "dx_perm", "dw1", "dw2")


# ----------------------------------------------------------------- one workload


def gather_possible(cfg):
    """The expert GEMMs can read x through the plan (bf16 activations, 32-bit row offsets)."""
    return cfg.act == "bf16" and cfg.T * cfg.d * 2 < 2 ** 31


def measure(cfg, steps, warmup, fused_gather="auto", extras=False):
    """Time `steps` training steps of one workload; returns (metrics dict, inputs)."""
    import torch
    from mixture_experts_layer_27_amd import binding, synth

    log(f"{cfg.name}: generating inputs")
    g = synth.generate(cfg)
    fused = fused_gather != "off" and gather_possible(cfg)
    torch.cuda.reset_peak_memory_stats()
    run = binding.LayerRun(cfg, g, fused_gather=fused)
    s = run.s
    stream = torch.cuda.current_stream()
    phases = ["route", "permute", "experts", "combine", "backward"]

    def step(ev=None, ftr=None, btr=None):
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
                                               run.ws_fwd, trace=ftr)
        else:
            binding.grouped_gemm_swiglu(s, run.x_perm, run.inp["w1"], run.inp["w2"], run.plan, run.h, run.y,
                                        run.ws_fwd, trace=ftr)
        mark(3)
        binding.unpermute_combine(s, run.y, run.plan, run.out)
        mark(4)
        if run.has_bwd:
            run.backward(with_optional=False, trace=btr)
        mark(5)

    log(f"{cfg.name}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    # one trace per call and step, read after the timed region (no sync inside it)
    ftrs = [binding.Trace(8) for _ in range(steps)]
    btrs = [binding.Trace(binding.TRACE_MAX_KERNELS + 1) if run.has_bwd else None for _ in range(steps)]
    log(f"{cfg.name}: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i], ftrs[i], btrs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = {}
    for i in range(steps):
        for name, ms in ftrs[i].durations_ms() + (btrs[i].durations_ms() if btrs[i] else []):
            kern.setdefault(name, []).append(ms)
    step_ms = [evs[i][0].elapsed_time(evs[i][5]) for i in range(steps)]
    ph = {p: statistics.median(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps))
          for j, p in enumerate(phases)}
    q = sorted(step_ms)
    pct = lambda x: q[min(len(q) - 1, int(round(x * (len(q) - 1))))]
    med = statistics.median(step_ms)
    # the same steps without the trace events (their cost on the step time)
    for _ in range(3):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n_plain = max(5, steps // 5)
    for _ in range(n_plain):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    plain_ms = e0.elapsed_time(e1) / n_plain

    counts = run.plan.arrays()["counts"].cpu()
    rows = int(counts.sum())
    work = kernel_work(cfg, rows)
    kernels_us = {k: 1e3 * statistics.mean(v) for k, v in kern.items()}
    dominant = max(kernels_us, key=kernels_us.get) if kernels_us else None
    per_gemm = {}
    gflops = gtime = 0.0
    for k, us in kernels_us.items():
        if k in work and k != "router_dwg":
            fl, peak = work[k]
            per_gemm[k] = {"us": us, "tflops": fl / (us * 1e-6) / 1e12, "frac": fl / (us * 1e-6) / 1e12 / peak}
            gflops += fl
            gtime += us * 1e-6
    peak = work["up_swiglu"][1]
    esz = 2 if cfg.act == "bf16" else 4
    permute_bytes = cfg.T * cfg.d * esz + rows * cfg.d * esz + 4 * (cfg.T + 1) + 4 * rows
    combine_bytes = rows * cfg.d * esz + cfg.T * cfg.d * esz + 8 * rows
    fwd_flops = work["up_swiglu"][0] + work["down"][0]
    out = {
        "workload": f"{cfg.name}: T={cfg.T} d_model={cfg.d} E={cfg.E} top-k={cfg.k} d_ff={cfg.f} SwiGLU, "
                    f"{'fwd+bwd' if run.has_bwd else 'fwd'}"
                    f"{', token rounding ' + str(cfg.round_tile) if cfg.round_tile else ''}"
                    f"{', MXFP8 expert GEMMs' if cfg.gemm == 'mxfp8' else ''}"
                    f"{', full-softmax gates' if cfg.gate == 'all' else ''}"
                    f"{', routing noise N(0, %g)' % cfg.noise_std if cfg.noise_std else ''}"
                    f"{', load-balance loss %g' % cfg.lb_coef if cfg.lb_coef else ''}"
                    f"{', z-loss %g' % cfg.z_coef if cfg.z_coef else ''}"
                    f"{', capacity factor %g' % cfg.capacity_factor if cfg.capacity_factor else ''}"
                    f"{', Zipf routing' if cfg.bias == 'zipf' else ''}",
        "tokens_per_s": cfg.T / (med * 1e-3),
        "ms_per_step_median": med,
        "ms_per_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "ms_per_step_wall_mean": wall * 1e3 / steps,
        "ms_per_step_untraced": plain_ms,
        "phases_ms_median": ph,
        "kernels_us_mean": kernels_us,
        "grouped_gemm": {"per_kernel": per_gemm,
                         "aggregate_tflops": gflops / gtime / 1e12 if gtime else None,
                         "aggregate_frac": gflops / gtime / 1e12 / peak if gtime else None,
                         "forward_call_frac": fwd_flops / (ph["experts"] * 1e-3) / 1e12 / peak},
        "permute_GBps": None,
        "combine_GBps": combine_bytes / (ph["combine"] * 1e-3) / 1e9,
        "rows": rows,
        "max_expert_rows": int(counts.max()),
        "fused_gather": fused,
    }
    if dominant is not None:
        fl, pk = work.get(dominant, (None, None))
        out["dominant_kernel"] = {"name": dominant, "us": kernels_us[dominant],
                                  "achieved_tflops": fl / (kernels_us[dominant] * 1e-6) / 1e12 if fl else None,
                                  "peak_tflops": pk}
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
    out["permute_GBps"] = permute_bytes / (permute_ms * 1e-3) / 1e9
    if extras:
        out.update(data_movement_extras(cfg, run, rows, permute_bytes, stream))
        out["activation_memory"] = activation_memory(cfg, run, binding) if run.has_bwd else None
    out["peak_allocated_bytes"] = torch.cuda.max_memory_allocated()
    del run
    torch.cuda.empty_cache()
    return out, g


def data_movement_extras(cfg, run, rows, permute_bytes, stream):
    """Cold-cache permute and plain device-copy rates (references for the
    data-movement kernels; not part of the layer)."""
    import torch
    from mixture_experts_layer_27_amd import binding
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def cold_ms(fn, n=5):
        t = []
        for _ in range(n):
            flush_buf.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    s = run.s
    permute_cold = cold_ms(lambda: binding.permute(s, run.inp["x"], run.plan, run.x_perm))
    esz = 2 if cfg.act == "bf16" else 4
    cbytes = (cfg.T + rows) * cfg.d * esz // 2 // 16 * 16
    csrc = torch.empty(cbytes, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        cdst.copy_(csrc)
    pev[0].record(stream)
    for _ in range(10):
        cdst.copy_(csrc)
    pev[1].record(stream)
    torch.cuda.synchronize()
    copy_GBps = 2 * cbytes / (pev[0].elapsed_time(pev[1]) / 10 * 1e-3) / 1e9
    copy_cold = cold_ms(lambda: cdst.copy_(csrc))
    # hand-written streaming kernels over the same byte count (moe_ref_stream): the
    # practical read, write and copy rates the data-movement kernels are held to
    ref = {}
    for name, mode, moved in (("read_nontemporal", binding.REF_READ, cbytes),
                              ("write", binding.REF_WRITE, cbytes),
                              ("copy_nontemporal_loads", binding.REF_COPY_NT_LOAD, 2 * cbytes),
                              ("copy_nontemporal_loads_stores", binding.REF_COPY_NT_BOTH, 2 * cbytes)):
        fn = lambda: binding.ref_stream(csrc, cdst, cbytes, mode)
        for _ in range(3):
            fn()
        pev[0].record(stream)
        for _ in range(10):
            fn()
        pev[1].record(stream)
        torch.cuda.synchronize()
        ref[name] = {"warm": moved / (pev[0].elapsed_time(pev[1]) / 10 * 1e-3) / 1e9,
                     "cold": moved / (cold_ms(fn) * 1e-3) / 1e9}
    del csrc, cdst, flush_buf
    return {"device_copy_GBps": copy_GBps,
            "reference_stream_GBps": ref,
            "cold_cache_GBps": {"permute": permute_bytes / (permute_cold * 1e-3) / 1e9,
                                "device_copy": 2 * cbytes / (copy_cold * 1e-3) / 1e9,
                                "note": "median of 5 launches, each after a 1 GiB scratch write"}}


def measure_accumulation(cfg, micro, steps, warmup):
    """One optimizer step of gradient accumulation over `micro` micro-batches
    (different x and dout, same weights), three ways in one process on the same
    inputs: bf16 expert GEMMs; MXFP8 quantising the weights in every micro-batch
    (the plain step); MXFP8 with the weight codes written once per optimizer step
    (moe_quantize_weights_mx) and read by every micro-batch
    (moe_grouped_gemm_swiglu_wcodes, moe_backward with the forward workspace).
    Each micro-batch is a whole layer step: route, expert FFN, combine, backward.
    Summing the weight gradients over the micro-batches is the caller's and costs
    the same for every variant, so it is not part of the timed work."""
    import dataclasses
    import torch
    from mixture_experts_layer_27_amd import binding, synth

    g = synth.generate(cfg)
    mbs = [{k: v.cuda() for k, v in synth.micro_batch(cfg, j).items()} for j in range(micro)]
    stream = torch.cuda.current_stream()
    res = {}
    for variant in ("bf16", "mxfp8", "mxfp8_weight_codes_reused"):
        c = dataclasses.replace(cfg, gemm="bf16" if variant == "bf16" else "mxfp8")
        log(f"{cfg.name}: gradient accumulation x{micro}, {variant}")
        run = binding.LayerRun(c, g, fused_gather=True)
        s = run.s

        def opt_step():
            if variant == "mxfp8_weight_codes_reused":
                binding.quantize_weights_mx(s, run.inp["w1"], run.inp["w2"], run.ws_fwd)
            for mb in mbs:
                run.inp["x"], run.inp["dout"] = mb["x"], mb["dout"]
                run.route()
                if variant == "mxfp8_weight_codes_reused":
                    binding.grouped_gemm_swiglu_wcodes(s, run.inp["x"], run.plan, run.h, run.y, run.ws_fwd)
                else:
                    run.experts()
                binding.unpermute_combine(s, run.y, run.plan, run.out)
                run.backward(with_optional=False)

        for _ in range(warmup):
            opt_step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(stream)
            opt_step()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        med = statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)
        res[variant] = {"ms_per_optimizer_step": med, "ms_per_micro_batch": med / micro,
                        "tokens_per_s": micro * cfg.T / (med * 1e-3)}
        del run
        torch.cuda.empty_cache()
    base = res["bf16"]["ms_per_micro_batch"]
    for v in res.values():
        v["speedup_vs_bf16"] = base / v["ms_per_micro_batch"]
    return {"workload": f"{cfg.name} shapes: T={cfg.T} per micro-batch, d_model={cfg.d} E={cfg.E} top-k={cfg.k} "
                        f"d_ff={cfg.f} SwiGLU, fwd+bwd, gradient accumulation over {micro} micro-batches",
            "micro_batches": micro, "optimizer_steps_timed": steps, "variants": res,
            "timing": "median over the timed optimizer steps of HIP events around each; per micro-batch = / micro"}


def measure_combine_in_gemm2(cfg, steps, warmup):
    """The forward's expert FFN + combine two ways in one process on the same
    routed batch: the separate calls (GEMM2 stores Y, the combine gathers each
    token's rows and applies the gates) and moe_grouped_gemm_swiglu_combine (GEMM2's
    epilogue applies the gate and stores each row at its token-order position, a
    segmented sum adds each token's contiguous rows)."""
    import torch
    from mixture_experts_layer_27_amd import binding, synth

    run = binding.LayerRun(cfg, synth.generate(cfg), fused_gather=True)
    s = run.s
    run.route()
    ws = binding._aligned_ws(binding.workspace_bytes(s, binding.MOE_WS_EXPERTS_COMBINE))
    h2, out2 = torch.empty_like(run.h), torch.empty_like(run.out)
    ms = {"separate": [], "combine_in_gemm2": []}
    kern = {}
    for i in range(warmup + steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        tr = binding.Trace(8)
        ev[0].record()
        binding.grouped_gemm_swiglu_gather(s, run.inp["x"], run.inp["w1"], run.inp["w2"], run.plan, run.h, run.y,
                                           run.ws_fwd)
        binding.unpermute_combine(s, run.y, run.plan, run.out)
        ev[1].record()
        ev[2].record()
        binding.grouped_gemm_swiglu_combine(s, run.inp["x"], run.inp["w1"], run.inp["w2"], run.plan, h2, out2, ws,
                                            trace=tr)
        ev[3].record()
        torch.cuda.synchronize()
        if i >= warmup:
            ms["separate"].append(ev[0].elapsed_time(ev[1]))
            ms["combine_in_gemm2"].append(ev[2].elapsed_time(ev[3]))
            for name, t in tr.durations_ms():
                kern.setdefault(name, []).append(t * 1e3)
    diff = (out2.float() - run.out.float()).abs()
    res = {"workload": f"{cfg.name}: T={cfg.T} d_model={cfg.d} E={cfg.E} top-k={cfg.k} d_ff={cfg.f}, forward expert "
                       f"FFN + combine",
           "ms_separate": statistics.median(ms["separate"]),
           "ms_combine_in_gemm2": statistics.median(ms["combine_in_gemm2"]),
           "kernels_us_combine_in_gemm2": {k: statistics.median(v) for k, v in kern.items()},
           "out_max_abs_diff": diff.max().item(), "out_mean_abs_diff": diff.mean().item()}
    del run, ws, h2, out2
    torch.cuda.empty_cache()
    return res


def activation_memory(cfg, run, binding):
    """Bytes the allocator holds from the end of the forward to the backward, for
    this layer (dS = <dA', A>, A recomputed from H: keeps x, the plan and H; x_perm
    too when handed to the backward) and for a layer that keeps what the
    conventional backward (dS = <dO, Y>) reads: x_perm, H, A and Y (SonicMoE
    article, section 1).  Each set is allocated as the forward leaves it, the
    forward run into it, and the allocator's count read; the layer input x is
    included, weights and the layer output are not."""
    import torch
    s = run.s
    dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    N = binding.max_rows(s)

    def held(keep_x_perm, keep_a_y):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        x = run.inp["x"].clone()
        plan = binding.Plan(s)
        x_perm = torch.empty((N, s.d), dtype=dt, device="cuda")
        h = torch.empty((N, 2 * s.d_ff), dtype=dt, device="cuda")
        y = torch.empty((N, s.d), dtype=dt, device="cuda")
        ws = torch.empty(binding.workspace_bytes(s, binding.MOE_WS_EXPERTS), dtype=torch.uint8, device="cuda")
        binding.route(s, x, run.inp["w_gate"], run.inp.get("bias"), plan, noise=run.inp.get("noise"))
        if s.round_tile:
            binding.round_tokens(s, plan)
        binding.permute(s, x, plan, x_perm)
        binding.grouped_gemm_swiglu(s, x_perm, run.inp["w1"], run.inp["w2"], plan, h, y, ws)
        torch.cuda.synchronize()
        if keep_a_y and cfg.gemm == "mxfp8":
            # the bf16 A this layer never stores (its workspace holds the MXFP8 operand codes instead)
            a_keep = torch.empty((N, s.d_ff), dtype=dt, device="cuda")
        else:
            a_keep = ws
        keep = [x, plan, h] + ([x_perm] if keep_x_perm else []) + ([a_keep, y] if keep_a_y else [])
        del y, ws, x_perm, a_keep
        torch.cuda.synchronize()
        n = torch.cuda.memory_allocated() - base
        del keep, x, plan, h
        torch.cuda.synchronize()
        return n

    minimal = held(False, False)
    with_xp = held(True, False)
    store_y = held(True, True)
    return {"minimal": minimal, "with_x_perm": with_xp, "store_y_layer": store_y,
            "timed_step_keeps": "with_x_perm" if run.x_perm is not None and not run.fused_gather else "minimal",
            "saving_minimal_vs_store_y": 1.0 - minimal / store_y,
            "saving_with_x_perm_vs_store_y": 1.0 - with_xp / store_y,
            "how": "torch.cuda.memory_allocated() after the forward, with only the tensors that set keeps alive "
                   "(A lives in the expert-GEMM workspace; with MXFP8 that workspace holds the operand codes)"}


# ----------------------------------------------------------------- main


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_27_amd import configs

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
    clocks_before = gpu_clocks()
    head, g = measure(cfg, a.steps, a.warmup, a.fused_gather, extras=True)
    clocks_after = gpu_clocks()
    dom = head.get("dominant_kernel") or {}
    fl_peak = kernel_work(cfg, head["rows"]).get(dom.get("name"), (None, None))
    achieved = dom.get("achieved_tflops")
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp8": "mxfp8", "bf16": "bf16"}.get(cfg.gemm, "f32"),
        "data": "synthetic",
        "config": {"workload": head["workload"], "global_batch": cfg.T, "seq_len": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": dom.get("name"), "achieved": achieved, "peak": fl_peak[1],
                     "unit": "TFLOP/s", "frac": achieved / fl_peak[1] if achieved else None,
                     "traffic": recorded_traffic(cfg.name, dom.get("name")), "traffic_unit": "HBM bytes per launch",
                     "algorithmic_flops_per_launch": fl_peak[0], "mean_launch_us": dom.get("us")},
        "timing": "value = T / median step device time (HIP events on the compute stream) over the timed steps",
        **{k: v for k, v in head.items() if k not in ("workload", "tokens_per_s")},
        "hbm_peak_GBps": PEAK_HBM_GBS,
        "gpu_clocks": {"before": clocks_before, "after": clocks_after},
    }
    if not a.no_sub:
        subs = {}
        for name in SUB_CONFIGS:
            if name == cfg.name:
                continue
            try:
                r, _ = measure(configs.get(name), a.sub_steps, a.sub_warmup, a.fused_gather)
            except Exception as exc:        # report, keep the headline
                r = {"error": f"{type(exc).__name__}: {exc}"}
            subs[name] = r
        out["sub_results"] = subs
        accum = {}
        for name in ACCUM_CONFIGS:
            try:
                accum[name] = measure_accumulation(configs.get(name), 4, a.accum_steps, 2)
            except Exception as exc:
                accum[name] = {"error": f"{type(exc).__name__}: {exc}"}
        out["gradient_accumulation"] = accum
        comb = {}
        for name in ACCUM_CONFIGS:
            try:
                comb[name] = measure_combine_in_gemm2(configs.get(name), 20, 3)
            except Exception as exc:
                comb[name] = {"error": f"{type(exc).__name__}: {exc}"}
        out["combine_in_gemm2"] = comb
    if not a.no_cpu_baseline:
        torch.cuda.empty_cache()
        tokens = a.cpu_tokens or min(cfg.T, 8192 if cfg.d * cfg.f * cfg.k > 2 ** 23 else 16384)
        log(f"cpu oracle on {tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, g, tokens)
    line = json.dumps(out)
    print(line, flush=True)
    if a.out:
        with open(a.out, "a") as fh:
            fh.write(line + "\n")


if __name__ == "__main__":
    main()
