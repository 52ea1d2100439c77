"""Benchmark of the MI355X MoE block: one step = one full pass of the block (route -> permute ->
grouped gate_up+SwiGLU -> grouped down -> [shared expert] -> combine) over one batch of seeded
synthetic tokens already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill] [--no-cpu-baseline]

Prints ONE JSON line. `value` is whole-layer tokens/s on the headline workload (the 16,384-token
Qwen3-VL-30B-A3B prefill layer). `roofline` reports the grouped gate_up GEMM (the dominant kernel),
timed with events on its launch stream inside the timed steps. `decode` adds the 64-token decode
layer (weight-read bound). `configs` reports every workload (tiny, keras, decode, prefill, fanout):
per-step GPU time (median, p10, p90), tokens/s, TFLOP/s, GB/s, the binding roofline and its
fraction, and the CPU oracle's tokens/s on all host threads and on one. `ceilings` holds the
measured read rate and register-only matrix-core rate of this machine beside the published peaks.
`quantized_experts` repeats prefill and decode with int8, int4 and fp8 expert weights (one scale per
weight row). `backward` times moe_backward on both workloads. `cpu_baseline` times the CPU oracle
on a bounded token sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "MoE-layer tokens/s; % bf16 MFMA peak (prefill), % HBM GB/s (decode)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector (the fp32 layer's FMA kernels)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(shape, touched, wbits=None):
    """FLOPs and bytes the method itself must do (not the dense all-expert work it avoids).
    wbits: bits per expert weight when the experts are quantised (one fp32 scale per weight row;
    int4 also one multiplier byte per 32 weights)."""
    N, D, E, k, I, Is = shape.n_tokens, shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter
    b = 2 if shape.dtype == "bf16" else 4
    wb = b if wbits is None else wbits / 8 + (1 / 32 if wbits == 4 else 0)   # bytes per expert weight
    rows = lambda n_out_rows: 0 if wbits is None else n_out_rows * 4      # scale bytes
    flops = 2 * N * D * E + 6 * D * I * N * k + (6 * D * Is * N + 2 * N * D if Is else 0)
    bytes_ = (touched * (3 * D * I * wb + rows(2 * I + D)) + E * D * b
              + (3 * D * Is * wb + rows(2 * Is + D) + D * b if Is else 0) + 2 * N * D * b + N * k * 8)
    gate_up_flops = 4 * D * I * N * k
    gate_up_bytes = touched * (2 * I * D * wb + rows(2 * I)) + N * k * D * b + N * k * I * b
    return dict(flops=flops, bytes=bytes_, gate_up_flops=gate_up_flops, gate_up_bytes=gate_up_bytes)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE runs scaled by a copy of known size), or None when there is none or the kernel
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gate_up_prefill_traffic.md")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "mixture_experts_layer_10_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec["kernel"] == kernel and rec["sources_sha256"] == h.hexdigest():
                    return rec["bytes_per_launch"]
    return None


def time_router_stats(B, chain, cfg, dev, steps):
    """Router load statistics and balance loss (moe_router_stats) on this workload's logits: the
    logits come from one moe_route call outside the timing; `steps` timed calls follow."""
    import torch
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    lg = torch.empty((N, E), dtype=torch.float32, device="cuda")
    w = torch.empty((N, k), dtype=torch.float32, device="cuda")
    e = torch.empty((N, k), dtype=torch.int32, device="cuda")
    ss = torch.empty((N,), dtype=torch.float32, device="cuda") if chain.gated else None
    B.moe_route(cfg, dev["x"], dev["w_router"], dev.get("w_shared_gate") if chain.gated else None, lg, w, e, ss, chain.ws)
    f = torch.empty(E, dtype=torch.float32, device="cuda")
    P = torch.empty(E, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    us = gpu_time_us(lambda: B.moe_router_stats(cfg, lg, chain.counts, f, P, loss, chain.ws), steps)
    return dict(us=round(us, 2), logits_gbs=round(N * E * 4 / (us * 1e-6) / 1e9, 1), loss=round(float(loss.item()), 6))


def gpu_time_us(run, steps):
    """GPU time per call of `run` (short kernels): a bounded GPU sleep first lets the host queue
    every call, so the events time the GPU work back to back."""
    import torch
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def time_variants(B, chain, cfg, dev, steps):
    """Routing variants on this workload: the sigmoid-score router with a selection bias, and the
    capacity-limited permute at 1.25 x the mean load per expert (with the share it drops)."""
    import torch
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    bias = torch.from_numpy(np.random.default_rng(7).normal(0.0, 0.05, E).astype(np.float32)).cuda()
    w = torch.empty((N, k), dtype=torch.float32, device="cuda")
    e = torch.empty((N, k), dtype=torch.int32, device="cuda")
    sig_us = gpu_time_us(lambda: B.moe_route_sigmoid(cfg, dev["x"], dev["w_router"], bias, None, w, e, chain.ws), steps)
    cap = max(1, int(1.25 * N * k / E))
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    token_of = torch.empty(N * k, dtype=torch.int32, device="cuda")
    slot_pos = torch.empty(N * k, dtype=torch.int32, device="cuda")
    run = lambda: B.moe_permute_capped(cfg, cap, chain.experts, None, counts, offsets, token_of, slot_pos, None, chain.ws)
    cap_us = gpu_time_us(run, steps)
    kept = int(offsets[E].item())
    return dict(sigmoid_route_us=round(sig_us, 2), capped_permute_us=round(cap_us, 2), capacity=cap,
                dropped_share=round(1.0 - kept / (N * k), 4))


LAYOUT_NAMES = {0: "rows", 1: "packed", 2: "int8", 3: "int4", 4: "fp8"}


EXPERT_OUT = {"f32": 0, "f16s": 1}


def run_workload(name, steps, warmup, out_dtype, inner_events=True, layout=1, data=None, extras=True, expert_out="f16s"):
    """Times `steps` whole-path steps. With inner_events every timed step is the decomposed chain of
    ABI calls with its gate_up launch bracketed by events on its stream (its duration comes from the
    timed region itself; at this size moe_forward launches exactly these kernels); without, the timed
    steps are moe_forward calls carrying no events (a recorded event idles the GPU for a few
    microseconds, which matters at decode sizes) and the gate_up duration comes from a second run of
    `steps` decomposed steps.
    layout: 1 packed bf16 experts (rows if the shape cannot be packed), 2 / 3 / 4 int8 / int4 / fp8
    experts. expert_out: "f16s" keeps the per-assignment expert outputs as fp16 values with a
    power-of-two exponent per 16 columns where the layer allows it (bf16 rows or packed weights,
    D % 16 == 0), else fp32; "f32" always fp32."""
    import torch
    from mixture_experts_layer_10_amd import binding as B
    from mixture_experts_layer_10_amd import inputs as I
    from mixture_experts_layer_10_amd.chain import Chain

    shape = I.WORKLOADS[name]
    t0 = time.perf_counter()
    if data is None:
        data = I.make_inputs(shape)
    dev = B.to_device(data.store)
    cfg = B.config_for(shape, out_dtype, layout=layout)
    if layout >= 2:                     # experts quantised once, as at model load
        dev = B.quantize_device_weights(cfg, dev)
        torch.cuda.synchronize()
    elif B.packable(cfg):               # expert weights packed once, as at model load
        dev = B.pack_device_weights(cfg, dev)
        torch.cuda.synchronize()
    else:
        cfg = B.config_for(shape, out_dtype)
    if EXPERT_OUT[expert_out] and B.f16s_supported(cfg):
        cfg = cfg.copy(expert_out=B.MOE_EXPERT_OUT_F16S)
    log(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s (weight layout "
        f"{LAYOUT_NAMES[cfg.weight_layout]}, expert outputs {'f16s' if cfg.expert_out else 'f32'})")
    chain = Chain(cfg, dev)
    y_ref = B.forward(cfg, dev)
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
    chain.decomposed()
    torch.cuda.synchronize()
    assert torch.equal(bits(chain.y), bits(y_ref)), "the decomposed chain and moe_forward disagree"
    counts = chain.counts.cpu().numpy()
    for _ in range(warmup):
        chain.step()
    torch.cuda.synchronize()
    assert torch.equal(bits(chain.y), bits(y_ref)), "moe_forward is not deterministic"
    touched = int((counts > 0).sum())
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    all0, all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all0.record()
    for i in range(steps):
        chain.step(ev[i] if inner_events else None)
    all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = all0.elapsed_time(all1)
    if not inner_events:
        for i in range(steps):
            chain.step(ev[i])
        torch.cuda.synchronize()
    gate_up_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_per_step = wall * 1e3 / steps
    stats = time_router_stats(B, chain, cfg, dev, steps) if extras else None
    variants = time_variants(B, chain, cfg, dev, steps) if extras else None
    alg = algorithmic(shape, touched, {2: 8, 3: 4, 4: 8}.get(cfg.weight_layout))
    log(f"[bench] {name}: {ms_per_step:.3f} ms/step (gpu {gpu_ms / steps:.3f}), gate_up {gate_up_ms:.3f} ms, "
        f"touched {touched}/{shape.n_experts}")
    return dict(shape=shape, data=data, cfg=cfg, chain=chain, stats=stats, variants=variants, ms_per_step=ms_per_step,
                gpu_ms_per_step=gpu_ms / steps,
                y=y_ref.float().cpu().numpy(),
                gate_up_ms=gate_up_ms, touched=touched, counts=counts, alg=alg,
                tokens_per_s=shape.n_tokens / (ms_per_step / 1e3))


def quantized_runs(args, runs):
    """Weight-only quantised experts (int8, int4 and fp8 e4m3, one fp32 scale per weight row; router and
    activations bf16) on the same inputs as the bf16 runs: step time, HBM fraction of the quantised
    algorithmic bytes, stored expert bytes, and the layer output's deviation from the bf16 layer."""
    out = {}
    for bits, layout in ((8, 2), (4, 3), ("f8", 4)):
        res = {}
        for wl, base in runs.items():
            decode = wl == "decode"
            q = run_workload(wl, max(args.steps, 50) if decode else args.steps, args.warmup, args.out_dtype,
                             inner_events=not decode, layout=layout, data=base["data"], extras=False)
            st = q["ms_per_step"] / 1e3
            sh = q["shape"]
            d = q["y"].astype(np.float64) - base["y"]
            ref_rms = float(np.sqrt(np.mean(base["y"].astype(np.float64) ** 2)))
            r = {"ms_per_step": round(q["ms_per_step"], 4), "tokens_per_s": round(q["tokens_per_s"], 1),
                 "alg_gbs": round(q["alg"]["bytes"] / st / 1e9, 1),
                 "hbm_frac": round(q["alg"]["bytes"] / st / 1e9 / PEAK_HBM_GBS, 4),
                 "gate_up_ms": round(q["gate_up_ms"], 4),
                 "expert_weight_bytes": int(sh.n_experts * (3 * sh.hidden * sh.inter * (4 if bits == 4 else 8) // 8
                                                            + (2 * sh.inter + sh.hidden) * 4)),
                 "y_rms_rel_vs_bf16": round(float(np.sqrt(np.mean(d * d))) / ref_rms, 5),
                 "y_maxabs_rel_vs_bf16": round(float(np.abs(d).max()) / ref_rms, 5)}
            if decode:
                r["gate_up_hbm_frac"] = round(q["alg"]["gate_up_bytes"] / (q["gate_up_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
            else:
                r["gate_up_tflops"] = round(q["alg"]["gate_up_flops"] / (q["gate_up_ms"] / 1e3) / 1e12, 1)
            res[wl] = r
        out["fp8" if bits == "f8" else f"int{bits}"] = res
    return out


def time_backward(base, steps, warmup):
    """moe_backward (gradients of x, W_r, gate_up and down for a seeded dy) on the same inputs as the
    forward run, row-layout weights: ms per call and TFLOP/s of the gradient contractions
    (12 D I per assignment + 4 N D E for the router; the recomputed pre-activations, 4 D I per
    assignment, are counted apart)."""
    import torch
    from mixture_experts_layer_10_amd import binding as B
    sh, data = base["shape"], base["data"]
    cfg = B.config_for(sh)
    dev = B.to_device(data.store)
    dy = torch.randn((sh.n_tokens, sh.hidden), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).cuda()
    ws = torch.empty(B.moe_backward_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    outs = None
    for _ in range(max(warmup, 1)):
        outs = B.backward(cfg, dev, dy, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        B.moe_backward(cfg, dev["x"], dev["w_router"], dev["gate_up"], dev["down"], dev.get("shared_gate_up"),
                       dev.get("shared_down"), dev.get("w_shared_gate"), dy, outs["dx"], outs["dw_router"],
                       outs["dgate_up"], outs["ddown"], outs.get("dshared_gate_up"), outs.get("dshared_down"),
                       outs.get("dw_shared_gate"), ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    A = sh.n_tokens * sh.top_k
    flops = 12 * sh.hidden * sh.inter * A + 4 * sh.n_tokens * sh.hidden * sh.n_experts
    return {"ms": round(ms, 4), "grad_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "recompute_tflops_extra": round(4 * sh.hidden * sh.inter * A / (ms * 1e-3) / 1e12, 1),
            "workspace_bytes": int(ws.numel()), "weight_layout": "rows"}


def step_stats(chain, samples, per):
    """GPU time per step over `samples` event-bracketed blocks of `per` back-to-back steps (blocks,
    so that at decode sizes the events' own idle time is spread over several steps): median, p10
    and p90 in ms."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    chain.step()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        for _ in range(per):
            chain.step()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / per for a, b in ev])
    return {"median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
            "p90": round(float(np.percentile(t, 90)), 4), "samples": samples, "steps_per_sample": per}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_oracle_rates(data, runs, one_thread_s=4.0):
    """The CPU oracle (grouped form, fp64) on this workload: all host BLAS threads over every token
    (median of `runs` runs), and one thread over a seeded token sample sized to about one_thread_s
    seconds. Returns tokens/s for both and what each timed."""
    import oracle as O
    s = data.shape
    w_router, gate_up, down = data.values("w_router"), data.values("gate_up"), data.values("down")   # converted outside the timing
    kw = {}
    if s.shared_inter:
        kw = dict(shared_gate_up=data.values("shared_gate_up"), shared_down=data.values("shared_down"),
                  w_shared_gate=data.values("w_shared_gate") if s.shared_gated else None)

    def run(toks):
        x = data.token_rows(toks)
        t0 = time.perf_counter()
        O.forward_grouped(x, w_router, gate_up, down, s.top_k, s.norm_topk_prob, **kw)
        return time.perf_counter() - t0

    all_toks = np.arange(s.n_tokens)
    t_all = float(np.median([run(all_toks) for _ in range(runs)]))
    rng = np.random.default_rng(0)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:
        limiter = None
    try:
        n = min(16, s.n_tokens)
        dt = run(np.sort(rng.choice(s.n_tokens, n, replace=False)))
        n1 = int(min(s.n_tokens, max(n, n * one_thread_s / max(dt, 1e-4))))
        t1 = run(np.sort(rng.choice(s.n_tokens, n1, replace=False)))
    finally:
        if limiter is not None:
            limiter.unregister()
    return {"tokens_per_s": round(s.n_tokens / t_all, 1), "threads": blas_threads(), "runs": runs,
            "tokens_per_s_1thread": round(n1 / t1, 1), "sample_1thread": f"{n1} of {s.n_tokens} tokens"}


def summarize_config(run, stats, cpu):
    """One workload's line of the configs block: rates at the median step time and the binding
    roofline (the larger of FLOPs / peak and bytes / HBM bandwidth, over the measured time)."""
    alg, sh = run["alg"], run["shape"]
    t = stats["median"] / 1e3
    peak = PEAK_FP32_TFLOPS if sh.dtype == "f32" else PEAK_BF16_TFLOPS
    t_flop, t_byte = alg["flops"] / (peak * 1e12), alg["bytes"] / (PEAK_HBM_GBS * 1e9)
    return {"shape": {"n_tokens": sh.n_tokens, "hidden": sh.hidden, "n_experts": sh.n_experts, "top_k": sh.top_k,
                      "inter": sh.inter, "shared_inter": sh.shared_inter, "dtype": sh.dtype},
            "weight_layout": LAYOUT_NAMES[run["cfg"].weight_layout],
            "expert_out": "f16s" if run["cfg"].expert_out else "f32",
            "ms_per_step": stats, "ms_per_step_wall_mean": round(run["ms_per_step"], 4),
            "tokens_per_s": round(sh.n_tokens / t, 1),
            "tflops": round(alg["flops"] / t / 1e12, 3), "alg_gbs": round(alg["bytes"] / t / 1e9, 1),
            "alg_flops": alg["flops"], "alg_bytes": alg["bytes"],
            "compute_peak_tflops": peak, "compute_frac": round(t_flop / t, 4), "hbm_frac": round(t_byte / t, 4),
            "bound": ("mfma" if sh.dtype == "bf16" else "fp32 alu") if t_flop >= t_byte else "hbm",
            "roofline_frac": round(max(t_flop, t_byte) / t, 4),
            "experts_touched": run["touched"], "max_rows_per_expert": int(run["counts"].max()),
            "cpu_oracle": cpu}


def measured_ceilings():
    """Read rate of a streaming kernel over 4 GiB and the register-only bf16 matrix-core rate."""
    import ctypes
    import torch
    from mixture_experts_layer_10_amd import build as BUILD
    lib = ctypes.CDLL(BUILD.PROBE_PATH)
    lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    nbytes, grid = 4 << 30, 1024
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4 * 4096, dtype=torch.float32, device="cuda")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / 1e3)
        return float(np.median(out))

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    # the best of a small sweep: 1,024 to 4,096 workgroups, 4 or 8 loads in flight, cached or nontemporal
    reads = {}
    for g in (1024, 2048, 4096):
        for mode in range(4):
            reads[(g, mode)] = timed(lambda: check(lib.probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), g, mode, st)), 3)
    (best_g, best_mode), t_read = min(reads.items(), key=lambda kv: kv[1])
    iters = 20000
    t_mfma = timed(lambda: check(lib.probe_mfma(sink.data_ptr(), iters, grid, st)))
    flops = grid * 4 * 4 * iters * 32 * 32 * 16 * 2
    del buf
    return {"read_gbs": round(nbytes / t_read / 1e9, 1), "read_frac_of_peak": round(nbytes / t_read / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
            "mfma_frac_of_peak": round(flops / t_mfma / 1e12 / PEAK_BF16_TFLOPS, 4),
            "read_config": {"workgroups": best_g, "loads_in_flight": 8 if best_mode & 1 else 4,
                            "nontemporal": bool(best_mode & 2)},
            "what": "probe/ceilings.hip: 16-byte reads of 4 GiB (best of 1,024-4,096 workgroups, 4 or 8 loads in "
                    "flight per lane, cached or nontemporal); 32x32x16 bf16 matrix-core steps on register operands, "
                    "four chains per wave, 16 waves per CU"}


def cpu_baseline(data, target_s=15.0):
    """The CPU oracle (grouped form, fp64) on a seeded token sample of the same workload."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    s = data.shape
    w_router = data.values("w_router")
    gate_up, down = data.values("gate_up"), data.values("down")     # converted outside the timed region
    rng = np.random.default_rng(0)

    def run(n):
        toks = np.sort(rng.choice(s.n_tokens, size=n, replace=False))
        x = data.token_rows(toks)
        t0 = time.perf_counter()
        O.forward_grouped(x, w_router, gate_up, down, s.top_k, s.norm_topk_prob)
        return time.perf_counter() - t0

    n = min(64, s.n_tokens)
    dt = run(n)
    n2 = int(min(s.n_tokens, max(n, n * target_s / max(dt, 1e-3))))
    dt2 = run(n2)
    log(f"[bench] cpu oracle: {n2} tokens in {dt2:.1f}s with {threads} threads")
    return dict(value=n2 / dt2, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{n2} of {s.n_tokens} tokens of the {s.name} workload (seeded sample), grouped fp64 oracle")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--out-dtype", default="f32")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quant", action="store_true", help="skip the int8 / int4 expert runs")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--expert-out", default="f16s", choices=sorted(EXPERT_OUT),
                    help="form of the per-assignment expert outputs (f16s where the layer allows it)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload configs block")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured read / matrix-core ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy a 256 MiB buffer once (a kernel of known traffic for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    # gate_up events inside the timed steps where the decomposed chain launches what moe_forward
    # launches (batches above 64 tokens); smaller batches time moe_forward itself
    from mixture_experts_layer_10_amd import inputs as I
    main_run = run_workload(args.workload, args.steps, args.warmup, args.out_dtype, expert_out=args.expert_out,
                            inner_events=I.WORKLOADS[args.workload].n_tokens > 64)
    shape, alg = main_run["shape"], main_run["alg"]
    gemm_s = main_run["gate_up_ms"] / 1e3
    # the roofline that binds: arithmetic intensity of the gate_up launch against the ridge point
    # (peak matrix-core rate / peak HBM bandwidth)
    mfma_bound = alg["gate_up_flops"] / alg["gate_up_bytes"] > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = alg["gate_up_flops"] / gemm_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=None)
    else:
        achieved = alg["gate_up_bytes"] / gemm_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=None)
    # the kernel the library launches: weight streaming when an expert averages at most 64 rows
    # (the assignment count N k is the row bound of the grouped launch), else 256 x 256 tiles
    cfg = main_run["cfg"]
    packed = "true" if cfg.weight_layout else "false"
    streaming = shape.n_tokens * shape.top_k <= 64 * shape.n_experts
    mean_rows = shape.n_tokens * shape.top_k // shape.n_experts          # 16-row slabs per pass: 1, 2 or 4
    slabs = 1 if mean_rows <= 8 else 2 if mean_rows <= 20 else 4
    kname = (f"gemm_wstream_kernel<{slabs},true,{packed},0>" if streaming
             else f"gemm_stream_kernel<2,4,4,2,true,{packed},0,false,false,true>")
    roof["kernel"] = kname + (" (grouped gate_up + SwiGLU, weight streaming)" if streaming else " (grouped gate_up + SwiGLU)")
    if args.workload == "prefill":
        roof["traffic"] = measured_traffic(kname)
    roof["per_launch"] = dict(flops=alg["gate_up_flops"], bytes=alg["gate_up_bytes"], avg_ms=round(main_run["gate_up_ms"], 4))
    layer_s = main_run["ms_per_step"] / 1e3
    out = {
        "metric": METRIC,
        "value": round(main_run["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; random-init weights N(0, 0.02^2))",
        "config": {"workload": shape.name, "n_tokens": shape.n_tokens, "hidden": shape.hidden,
                   "n_experts": shape.n_experts, "top_k": shape.top_k, "inter": shape.inter,
                   "shared_inter": shape.shared_inter, "norm_topk_prob": shape.norm_topk_prob,
                   "zipf_s": shape.zipf_s, "out_dtype": args.out_dtype, "seed": shape.seed,
                   "weight_layout": "packed" if main_run["cfg"].weight_layout else "rows",
                   "expert_out": "f16s" if main_run["cfg"].expert_out else "f32",
                   "parallelism": "none (1 GPU)"},
        "layer": {"tflops": round(alg["flops"] / layer_s / 1e12, 2),
                  "mfma_frac": round(alg["flops"] / layer_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "alg_gbs": round(alg["bytes"] / layer_s / 1e9, 1),
                  "hbm_frac": round(alg["bytes"] / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                  "experts_touched": main_run["touched"], "max_rows_per_expert": int(main_run["counts"].max()),
                  "min_rows_per_expert": int(main_run["counts"].min())},
        "roofline": roof,
        "router_stats": main_run["stats"],
        "routing_variants": main_run["variants"],
    }
    out["ms_per_step_gpu"] = step_stats(main_run["chain"], args.steps, 1)
    dec = None
    if not args.no_decode and args.workload != "decode":
        dec = run_workload("decode", max(args.steps, 50), args.warmup, args.out_dtype, inner_events=False,
                           expert_out=args.expert_out)
        ds = dec["ms_per_step"] / 1e3
        out["decode"] = {"workload": "decode", "tokens_per_s": round(dec["tokens_per_s"], 1),
                         "ms_per_step": round(dec["ms_per_step"], 4),
                         "alg_gbs": round(dec["alg"]["bytes"] / ds / 1e9, 1),
                         "hbm_frac": round(dec["alg"]["bytes"] / ds / 1e9 / PEAK_HBM_GBS, 4),
                         "experts_touched": dec["touched"],
                         "gate_up_ms": round(dec["gate_up_ms"], 4),
                         "gate_up_hbm_frac": round(dec["alg"]["gate_up_bytes"] / (dec["gate_up_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
        if not args.no_quant and args.workload == "prefill":
            out["quantized_experts"] = quantized_runs(args, {"decode": dec, "prefill": main_run})
        if not args.no_backward and args.workload == "prefill":
            out["backward"] = {"prefill": time_backward(main_run, args.steps, args.warmup),
                               "decode": time_backward(dec, max(args.steps, 50), args.warmup)}
            log(f"[bench] backward: {out['backward']}")
    if not args.no_configs:
        configs = {}
        for wl in ("tiny", "keras", "decode", "prefill", "fanout"):
            if wl == args.workload:
                r = main_run
            elif wl == "decode" and dec is not None:
                r = dec
            else:
                r = run_workload(wl, args.steps, args.warmup, args.out_dtype, inner_events=False, extras=False,
                                 expert_out=args.expert_out)
            small = r["shape"].n_tokens * r["shape"].top_k <= 8192
            st = step_stats(r["chain"], 20, 10 if small else 1)
            cpu = None if args.no_cpu_baseline else cpu_oracle_rates(r["data"], 1 if wl == "prefill" else 3)
            configs[wl] = summarize_config(r, st, cpu)
            log(f"[bench] config {wl}: {configs[wl]['ms_per_step']} ms, {configs[wl]['bound']} "
                f"{configs[wl]['roofline_frac']}, cpu {cpu}")
            if r is not main_run and r is not dec:
                del r
        out["configs"] = configs
        if not args.no_cpu_baseline:
            out["cpu_model"] = cpu_model()
    if not args.no_ceilings:
        out["ceilings"] = measured_ceilings()
        log(f"[bench] ceilings: {out['ceilings']}")
    if args.copy_calibration:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "written": dst.numel() * 4}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(main_run["data"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
