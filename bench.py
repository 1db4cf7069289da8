#!/usr/bin/env python3
"""Benchmark of the denoise step: canvas positions/s and ms per step on one MI355X.

Default workload "batch8_ragged_32k": the 12-layer MoE model (d 2048, 16 q / 8 kv heads,
head_dim 128, 64 experts top-4, d_ff 768, shared SwiGLU FFN 4096, vocab 65536) serving eight
requests whose prefixes are round(32768 (1 + U(-1/4, 1/4))) random tokens (prefilled causally,
untimed), their eight 256-token canvases denoised together: 2048 canvas rows per step.  A step
is one dg_denoise_step (embedding, 12 layers, final norm, fused vocab head) plus one
dg_sample_commit on all eight canvases, cycling through the 48-step schedule (temperature
0.8 -> 0.4, commit 16, re-noise below 0.1).  Weights and tokens are seeded synthetic data (no
checkpoint exists), drawn on the device.  The same run also measures the one-canvas loop (prefix
2048) on the same model and reports it under "full_canvas_loop".

Output: one JSON line with the metric, a roofline entry for the dominant kernel (canvas
attention at this workload: its MFMA flops over its average launch time, measured live with HIP
events on its launch stream) and the CPU oracle timed on a bounded sample of the same step.

Other workloads (--workload): full_canvas_loop (one canvas, prefix 2048), single_layer (one
layer at d 2048, 64 experts top-4, prefix 4096, no head, no sampler), tiny_loop (the two-layer
d 256 model through its whole sampling loop), prefill_batch8_32k (the causal prefill of the eight
~32 k prompts), long_generation, full_canvas_loop_fp8, continuous_serving.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
SEED = 20260610


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- work per launch

def expert_gemm1_bytes(shape, routes: int, experts_touched: int) -> float:
    """Algorithmic HBM bytes of one gate/up expert GEMM launch: each touched expert's gate and up
    matrices once (bf16, or E4M3 bytes plus one float32 scale per output channel), each routed
    row's activations once, the SwiGLU output once."""
    if getattr(shape, "expert_fp8", False):
        w = experts_touched * 2 * shape.d_ff_expert * (shape.d_model * 1 + 4)
    else:
        w = experts_touched * 2 * shape.d_ff_expert * shape.d_model * 2
    x = routes * shape.d_model * 2
    out = routes * shape.d_ff_expert * 2
    return float(w + x + out)


def attention_flops(shape, lens) -> float:
    """Algorithmic MFMA flops of one canvas-attention launch: QK^T and PV of every canvas query
    over its request's cached prefix plus the canvas, 2 flops per multiply-add each."""
    C = shape.canvas
    return float(4 * shape.n_q_heads * shape.head_dim * sum(C * (L + C) for L in lens))


def attention_bytes(shape, lens) -> float:
    """Algorithmic HBM bytes of one canvas-attention launch: each request's cached K and V and
    canvas K and V once (bf16), the queries in and the output out (bf16)."""
    C, D = shape.canvas, shape.head_dim
    kv = 2 * 2 * shape.n_kv_heads * D * sum(L + C for L in lens)
    qo = 2 * 2 * shape.n_q_heads * D * C * len(lens)
    return float(kv + qo)


def causal_attention_flops(shape, n: int, chunk: int) -> float:
    """MFMA flops of the causal prefill attention of one n-token prompt processed in chunks: a
    query at position p sees p + 1 keys."""
    return float(4 * shape.n_q_heads * shape.head_dim * (n * (n + 1) // 2))


# HBM traffic of a roofline kernel from hardware counters (rocprofv3 --pmc FETCH_SIZE, then
# WRITE_SIZE, in separate runs of this script), per launch, each scaled by the ratio
# true bytes / counter bytes that the same counter gives for a plain 1 GiB device copy.  Valid
# only for the kernel source it was taken on: a changed source reports traffic null.
PMC_TRAFFIC = {
    "moe_gemm1_swiglu": {
        "kernel": "expert_stream_kernel<true, 3, 1, 1, false, true, 1>", "workload": "full_canvas_loop",
        "source": "block_discrete_diffusion_amd/csrc/k_moe.hip", "sha": "929cf7488c01e500",
        "fetch_kib": 202120.2, "fetch_scale": 1048576.0 / 524315.2,  # copy of 1 GiB reads 524315 KiB
        "write_kib": 1487.8, "write_scale": 1048576.0 / 1048576.0,   # and writes 1048576 KiB
    },
    "attention": {
        "kernel": "attention_pipe_kernel<8>", "workload": "batch8_ragged_32k",
        "source": "block_discrete_diffusion_amd/csrc/k_attn.hip", "sha": "c847875a1b63d4d7",
        "fetch_kib": 571288.7, "fetch_scale": 1048576.0 / 524315.2,
        "write_kib": 33826.4, "write_scale": 1048576.0 / 1048576.0,
    },
}


def source_digest(rel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(family: str, workload: str):
    t = PMC_TRAFFIC.get(family)
    if t is None or t["workload"] != workload or source_digest(t["source"]) != t["sha"]:
        return None
    return t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]


def copy_calibration(mib: int):
    """One plain device-to-device copy of `mib` MiB (float32), for scaling the HBM counters."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4}), flush=True)


def _host(t):
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def _threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def roofline_entry(bound, family, kt, work, unit_work, workload, extra=None):
    """`work` algorithmic bytes (bound hbm) or flops (bound mfma) per launch of `family`, over its
    average HIP-event launch time on the launch stream."""
    t = kt[family]["avg_ms"] * 1e-3
    if bound == "hbm":
        ach = work / t / 1e9
        e = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = work / t / 1e12
        e = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    e["traffic"] = measured_traffic(family, workload)
    e.update({"kernel": family, "avg_launch_us": round(kt[family]["avg_ms"] * 1e3, 2),
              f"algorithmic_{unit_work}_per_launch": work})
    if extra:
        e.update(extra)
    return e


# ----------------------------------------------------------------------------- the canvas loop

class CanvasLoop:
    """Denoise + sampler steps on B canvases over a prefilled cache, cycling through the
    schedule (a canvas restarts after the step cap)."""

    def __init__(self, dg, m, kv, cfg, B, shape):
        import torch
        self.m, self.kv, self.cfg, self.dg = m, kv, cfg, dg
        self.st = dg.Canvas(B, shape.canvas)
        self.stats = dg.Stats(B, shape.canvas)
        self.status = torch.zeros((B, 8), dtype=torch.int32, device="cuda")
        m.canvas_init(self.st, kv, cfg)
        self.s = 0

    def step(self):
        if self.s == self.cfg.max_steps:
            self.m.canvas_init(self.st, self.kv, self.cfg)
            self.s = 0
        self.m.denoise_step(self.st.tokens, self.kv, self.cfg, self.s, self.stats)
        self.m.sample_commit(self.st, self.stats, self.cfg, self.s, self.kv, self.status)
        self.s += 1


def time_steps(step, steps, warmup, m=None):
    """Warm up, then time `steps` steps with HIP events on the current stream; then, with m, one
    more pass with per-kernel HIP events on the launch stream.  Returns (ms per step, wall
    seconds of the timed region, per-kernel {family: {launches, total_ms, avg_ms}} or None)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    kt = None
    if m is not None:
        m.timing(True)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        kt = m.timing_read()
        m.timing(False)
    return ms, t_wall, kt


def per_step_us(kt, steps):
    return {k: round(v["total_ms"] / steps * 1e3, 2) for k, v in kt.items()}


def prefill_requests(dg, m, kv, shape, lens, tag0=1):
    import torch
    from block_discrete_diffusion_amd import synth
    B = len(lens)
    t0 = time.perf_counter()
    for b, L in enumerate(lens):  # one request at a time keeps progress visible
        n = [0] * B
        n[b] = L
        m.prefill(torch.from_numpy(synth.tokens(L, shape.vocab, SEED, tag0 + b)).cuda(), n, kv)
        torch.cuda.synchronize()
        log(f"  prefill request {b}: {L} tokens, {time.perf_counter() - t0:.1f} s")


# ----------------------------------------------------------------------------- CPU baselines

def cpu_baseline_batch(shape, weights, kv, lens, sample_rows: int):
    """The CPU oracle, as it stands, on a bounded sample of one step of B requests: layer 0 of
    the request of median prefix length over its 256 canvas rows (its GPU-prefilled bf16 K/V of
    layer 0 copied to the host, a synthetic residual input), scaled x B x n_layers; the fused
    head with Gumbel row statistics on `sample_rows` rows scaled to B x 256 rows; the sampler on
    one canvas scaled x B."""
    import numpy as np
    from block_discrete_diffusion_amd import synth
    from oracle import model as om
    from oracle import sampler as osm

    B = len(lens)
    order = sorted(range(B), key=lambda b: lens[b])
    b = order[B // 2]
    L = lens[b]
    d, V = shape.d_model, shape.vocab
    lw = {k: _host(v) for k, v in weights["layers"][0].items()}
    k = _host(kv.k[0, b, :, :L]).astype(np.float64)
    v = _host(kv.v[0, b, :, :L]).astype(np.float64)
    h = synth.hidden(256, d, SEED, 103)
    t0 = time.perf_counter()
    om.layer(h, lw, shape, L + np.arange(256), k, v, None)
    t_layer = time.perf_counter() - t0
    del lw, k, v
    head = _host(weights["lm_head"])
    f = synth.bf16_normal((sample_rows, d), SEED, 104)
    x = synth.tokens(sample_rows, V, SEED, 105)
    cfg = osm.SamplerConfig(seed=1)
    t0 = time.perf_counter()
    z = om.head_logits(f, head)
    st = osm.row_stats(z, x, osm.temperature(cfg, 0), cfg.seed, 0, L + np.arange(sample_rows), 0)
    t_head = (time.perf_counter() - t0) * B * 256 / sample_rows
    full = {kk: np.resize(vv, 256) for kk, vv in st.items()}
    t0 = time.perf_counter()
    osm.sample_commit(full, synth.tokens(256, V, SEED, 106), np.zeros(256, bool), 0, cfg, 0, 0,
                      L + np.arange(256), V)
    t_samp = (time.perf_counter() - t0) * B
    t_step = B * shape.n_layers * t_layer + t_head + t_samp
    return {
        "value": round(B * 256.0 / t_step, 3), "unit": "canvas positions/s", "cores": _threads(),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: layer 0 of request {b} (prefix {L}, its GPU-prefilled bf16 K/V) "
                   f"over 256 canvas rows scaled x{B * shape.n_layers} ({B} requests x {shape.n_layers} layers), "
                   f"head + Gumbel row stats on {sample_rows} rows scaled x{B * 256 // sample_rows}, "
                   f"sampler on 256 positions x{B}; est. {t_step:.1f} s/step (layer {t_layer:.2f} s, "
                   f"head {t_head:.1f} s, sampler {t_samp * 1e3:.1f} ms); "
                   f"host affinity {len(os.sched_getaffinity(0))} cpus"),
    }


def cpu_baseline_single_layer(shape, weights, h, k, v, L):
    """The whole config: the oracle's layer over the 256 canvas rows on the same inputs."""
    import numpy as np
    from oracle import model as om
    lw = {kk: _host(vv) for kk, vv in weights["layers"][0].items()}
    t0 = time.perf_counter()
    om.layer(h, lw, shape, L + np.arange(256), k, v, None)
    t = time.perf_counter() - t0
    return {"value": round(256.0 / t, 3), "unit": "canvas positions/s", "cores": _threads(), "kind": "oracle",
            "sample": f"the whole workload: float64 NumPy oracle layer over 256 rows, prefix {L}: {t * 1e3:.0f} ms; "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus"}


# ----------------------------------------------------------------------------- workloads

WORKLOADS = {
    "batch8_ragged_32k": "12 layers d2048 16q/8kv hd128, 64 experts top-4 d_ff 768 + shared FFN 4096, vocab 65536; "
                         "8 requests with prefixes round(32768*(1+U(-1/4,1/4))) prefilled causally, 8 canvases of "
                         "256 denoised together (2048 rows per step), sampler 48 steps 0.8->0.4 commit 16",
    "full_canvas_loop": "same model, prefix 2048, one canvas of 256, sampler 48 steps 0.8->0.4 commit 16",
    "single_layer": "one layer d2048 16q/8kv hd128, 64 experts top-4 d_ff 768 (no shared FFN), residual input "
                    "N(0,1) [256,2048], prefix K/V N(0,1) bf16 of 4096 positions; one dg_denoise_step, no head, "
                    "no sampler",
    "tiny_loop": "2 layers d256 4q/2kv hd64, 8 experts top-2 d_ff 512, vocab 1024, prefix 64, one canvas of 256 "
                 "through its whole sampling loop (48-step cap, adaptive stop)",
    "prefill_batch8_32k": "the batch8_ragged_32k model and prompts: causal prefill of 8 prompts of "
                          "round(32768*(1+U(-1/4,1/4))) tokens in 2048-row chunks",
    "long_generation": "same model, prefix 8192, 8 consecutive canvases each denoised until the sampler "
                       "stops and then committed to the KV cache (final length 10240)",
    "full_canvas_loop_fp8": "the full canvas loop with the routed experts quantized to OCP E4M3 "
                            "(per-channel float32 scales); everything else bf16",
    "continuous_serving": "same model, 24 requests (prompts round(2048*(1+U(-1/2,1/2))), 1-3 blocks each) "
                          "arriving one every 6 scheduler iterations, served on 8 cache slots with up to "
                          "8 live canvases per call; prefill, sampling loop and block commits all timed",
}


def base_line(metric, value, unit, steps, warmup, ms, dtype, workload, B, seq_len, **extra):
    out = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded device RNG weights, uniform random tokens)",
           "config": {"workload": f"{workload}: {WORKLOADS[workload]}", "global_batch": B, "seq_len": seq_len,
                      "parallelism": "single GPU"}}
    out.update(extra)
    return out


def canvas_workload(args, dg, shape, w, cfg, workload):
    """batch8_ragged_32k (with the one-canvas loop as extra keys) and full_canvas_loop[_fp8]."""
    import torch
    from block_discrete_diffusion_amd import synth

    batch = workload == "batch8_ragged_32k"
    lens = synth.ragged_lengths(8, 32768, 0.25, SEED) if batch else [2048]
    B = len(lens)
    m = dg.Model(shape, w, max_batch=B, max_prefill_rows=2048)
    kv = dg.KV(shape, B, max(lens) + shape.canvas)
    log(f"prefill {B} request(s), lengths {lens}")
    prefill_requests(dg, m, kv, shape, lens)
    loop = CanvasLoop(dg, m, kv, cfg, B, shape)
    log(f"timing {args.steps} steps (+{args.warmup} warm-up) on {B} canvas(es)")
    ms, wall, kt = time_steps(loop.step, args.steps, args.warmup, None if args.no_kernel_timing else m)
    value = B * shape.canvas / (ms * 1e-3)
    extra = {}
    roofline = None
    if kt is not None:
        extra["kernel_us_per_step"] = per_step_us(kt, args.steps)
        routes = B * shape.canvas * shape.top_k
        gemm1 = roofline_entry("hbm", "moe_gemm1_swiglu", kt, expert_gemm1_bytes(shape, routes, shape.n_experts),
                               "bytes", workload)
        fl = attention_flops(shape, lens)
        attn = roofline_entry("mfma", "attention", kt, fl, "flops", workload,
                              {"kv_bytes_per_launch": attention_bytes(shape, lens)})
        if "attn_split_combine" in kt:
            t2 = (kt["attention"]["avg_ms"] + kt["attn_split_combine"]["avg_ms"]) * 1e-3
            attn["with_split_combine"] = {"avg_us": round(t2 * 1e6, 2),
                                          "frac": round(fl / t2 / 1e12 / BF16_PEAK_TFLOPS, 4)}
        roofline = attn if batch else gemm1
        extra["attention_roofline"] = attn
        extra["expert_gemm1_roofline"] = gemm1
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline_batch(shape, w, kv, lens, args.cpu_sample_rows)
    out = base_line("canvas positions/s (denoise step, 1 GPU)", value, "canvas positions/s", args.steps,
                    args.warmup, ms, "bf16, routed experts e4m3" if shape.expert_fp8 else "bf16", workload, B,
                    max(lens) + shape.canvas, roofline=roofline, cpu_baseline=cpu, prefix_lengths=lens,
                    wall_s_timed=round(wall, 3), **extra)
    del loop
    if batch and not args.no_extra:
        # the one-canvas loop (prefix 2048) on the same model and context, as extra keys
        kv1 = dg.KV(shape, 1, 2048 + shape.canvas)
        log("extra: one canvas, prefix 2048")
        prefill_requests(dg, m, kv1, shape, [2048])
        loop1 = CanvasLoop(dg, m, kv1, cfg, 1, shape)
        ms1, _, kt1 = time_steps(loop1.step, args.steps, args.warmup, None if args.no_kernel_timing else m)
        e = {"ms_per_step": round(ms1, 4), "value": round(shape.canvas / (ms1 * 1e-3), 1),
             "unit": "canvas positions/s", "config": WORKLOADS["full_canvas_loop"]}
        if kt1 is not None:
            e["expert_gemm1_roofline"] = roofline_entry(
                "hbm", "moe_gemm1_swiglu", kt1, expert_gemm1_bytes(shape, shape.canvas * shape.top_k, shape.n_experts),
                "bytes", "full_canvas_loop")
            e["kernel_us_per_step"] = per_step_us(kt1, args.steps)
        out["full_canvas_loop"] = e
    print(json.dumps(out), flush=True)
    m.close()


def single_layer(args, dg, cfg):
    """One dg_denoise_step of one layer on a given residual state (DG_STEP_HIDDEN_IN), no head."""
    import numpy as np
    import torch
    from block_discrete_diffusion_amd import synth

    shape = synth.MID_LAYER
    L = 4096
    w = synth.torch_model_weights(shape, "cuda", SEED)
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=256)
    kv = dg.KV(shape, 1, L + shape.canvas, fill=None)
    dims = (shape.n_layers, 1, shape.n_kv_heads, L, shape.head_dim)
    kv.k[:, :, :, :L] = synth.torch_bf16_normal(dims, "cuda", SEED, 201)
    kv.v[:, :, :, :L] = synth.torch_bf16_normal(dims, "cuda", SEED, 202)
    kv.set_lengths([L])
    h = synth.hidden(256, shape.d_model, SEED, 203)
    hd = torch.from_numpy(h).cuda()
    step = lambda: m.denoise_step(None, kv, None, 0, None, flags=dg.DG_STEP_HIDDEN_IN | dg.DG_STEP_NO_HEAD,
                                  hidden_in=hd)
    log(f"timing {args.steps} single-layer steps")
    ms, wall, kt = time_steps(step, args.steps, args.warmup, None if args.no_kernel_timing else m)
    extra, roofline = {}, None
    if kt is not None:
        extra["kernel_us_per_step"] = per_step_us(kt, args.steps)
        roofline = roofline_entry("hbm", "moe_gemm1_swiglu", kt,
                                  expert_gemm1_bytes(shape, 256 * shape.top_k, shape.n_experts), "bytes", "single_layer")
        extra["attention_roofline"] = roofline_entry("mfma", "attention", kt, attention_flops(shape, [L]), "flops",
                                                     "single_layer")
        # the whole step against its bound: sum over kernels of max(flops / peak, bytes / BW)
        extra["step_bound_us"] = 84.5
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (the whole layer)")
        k = _host(kv.k[0, 0, :, :L]).astype(np.float64)
        v = _host(kv.v[0, 0, :, :L]).astype(np.float64)
        cpu = cpu_baseline_single_layer(shape, w, h, k, v, L)
    out = base_line("canvas positions/s (one-layer denoise step, 1 GPU)", 256 / (ms * 1e-3), "canvas positions/s",
                    args.steps, args.warmup, ms, "bf16", "single_layer", 1, L + shape.canvas, roofline=roofline,
                    cpu_baseline=cpu, wall_s_timed=round(wall, 3), **extra)
    print(json.dumps(out), flush=True)
    m.close()


def tiny_loop(args, dg):
    """The small model's whole sampling loop, GPU against the oracle's loop on the host."""
    import numpy as np
    import torch
    from block_discrete_diffusion_amd import synth
    from oracle import model as om
    from oracle import sampler as osm

    shape = synth.TINY
    L = 64
    w = synth.model_weights(shape, SEED)
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=256)
    kv = dg.KV(shape, 1, L + shape.canvas)
    prefix = synth.tokens(L, shape.vocab, SEED, 1)
    m.prefill(torch.from_numpy(prefix).cuda(), [L], kv)
    cfg = dg.sampler_cfg(seed=SEED)
    stats = dg.Stats(1, shape.canvas)

    def run_loop():
        st = dg.Canvas(1, shape.canvas)
        m.canvas_init(st, kv, cfg)
        return m.denoise_canvas(st, kv, cfg, stats)["steps"]

    for _ in range(args.warmup):
        run_loop()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_loops = max(1, args.steps // 8)
    t_wall = time.perf_counter()
    e0.record()
    n_steps = sum(run_loop() for _ in range(n_loops))
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / n_steps
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline: the oracle's whole sampling loop")
        ck = [np.zeros((shape.n_kv_heads, L, shape.head_dim)) for _ in range(shape.n_layers)]
        cv = [np.zeros((shape.n_kv_heads, L, shape.head_dim)) for _ in range(shape.n_layers)]
        om.prefill(w, shape, prefix, ck, cv, 0)
        oc = osm.SamplerConfig(seed=SEED)
        pos = L + np.arange(shape.canvas)
        x = osm.canvas_init(oc.seed, 0, pos, shape.vocab)
        com, sr = np.zeros(shape.canvas, bool), 0
        t0 = time.perf_counter()
        o_steps = 0
        for s in range(oc.max_steps):
            fw = om.denoise_forward(w, shape, x, ck, cv, L)
            rs = osm.row_stats(fw["logits"], x, osm.temperature(oc, s), oc.seed, 0, pos, s)
            x, com, sr, status = osm.sample_commit(rs, x, com, sr, oc, s, 0, pos, shape.vocab)
            o_steps += 1
            if status["stop"]:
                break
        t = time.perf_counter() - t0
        cpu = {"value": round(shape.canvas * o_steps / t, 1), "unit": "canvas positions/s", "cores": _threads(),
               "kind": "oracle",
               "sample": f"the whole workload: the oracle's sampling loop, {o_steps} steps in {t:.2f} s "
                         f"({t / o_steps * 1e3:.1f} ms/step); host affinity {len(os.sched_getaffinity(0))} cpus"}
    out = base_line("canvas positions/s (small-model sampling loop, 1 GPU)", shape.canvas / (ms * 1e-3),
                    "canvas positions/s", n_steps, args.warmup, ms, "bf16", "tiny_loop", 1, L + shape.canvas,
                    roofline=None, cpu_baseline=cpu, loops=n_loops, wall_s_timed=round(t_wall, 3))
    print(json.dumps(out), flush=True)
    m.close()


def prefill_workload(args, dg, shape, w):
    """Causal prefill of the eight ~32 k prompts: prompt tokens/s, with the causal attention's
    MFMA fraction measured per launch."""
    import numpy as np
    import torch
    from block_discrete_diffusion_amd import synth
    from oracle import model as om

    lens = synth.ragged_lengths(8, 32768, 0.25, SEED)
    chunk = 2048
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=chunk)
    kv = dg.KV(shape, 1, max(lens))
    toks = [torch.from_numpy(synth.tokens(L, shape.vocab, SEED, 1 + b)).cuda() for b, L in enumerate(lens)]
    log("warm-up: one 4096-token prompt")
    m.prefill(toks[0][:4096], [4096], kv)
    torch.cuda.synchronize()
    kv.set_lengths([0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for b, L in enumerate(lens):
        kv.set_lengths([0])
        m.prefill(toks[b], [L], kv)
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    n_tok = sum(lens)
    extra, roofline = {}, None
    if not args.no_kernel_timing:
        # per-kernel durations from a second pass over the same prompts (the events around each
        # kernel would otherwise count in the timed one)
        log("per-kernel timing: a second pass over the prompts")
        m.timing(True)
        for b, L in enumerate(lens):
            kv.set_lengths([0])
            m.prefill(toks[b], [L], kv)
        torch.cuda.synchronize()
        kt = m.timing_read()
        m.timing(False)
        extra["kernel_ms_total"] = {k: round(v["total_ms"], 2) for k, v in kt.items()}
        fl = sum(causal_attention_flops(shape, L, chunk) for L in lens) * shape.n_layers
        t_att = kt["attention"]["total_ms"] * 1e-3
        ach = fl / t_att / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "attention (causal prefill)", "launches": kt["attention"]["launches"],
                    "algorithmic_flops_total": fl,
                    "note": "flops and time summed over every causal attention launch of the prefill"}
        gem = {}
        for fam, flop_tok in (("gemm_qkv_rope", 2 * shape.d_model * (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim),
                              ("shared_gate_up_swiglu", 2 * 2 * shape.d_model * shape.d_ff_shared),
                              ("shared_down_residual", 2 * shape.d_model * shape.d_ff_shared),
                              ("gemm_o_residual", 2 * shape.d_model * shape.n_q_heads * shape.head_dim)):
            if fam in kt:
                f_all = flop_tok * n_tok * shape.n_layers
                gem[fam] = round(f_all / (kt[fam]["total_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        extra["gemm_mfma_frac"] = gem
    cpu = None
    if not args.no_cpu_baseline:
        # trapezoid over the prompt: the oracle's per-token cost of one layer at the start and at
        # the end of a prompt (attention cost grows linearly with the position)
        log("CPU oracle baseline: one layer, 256-token chunks at both ends of a prompt")
        lw = {k: _host(v) for k, v in w["layers"][0].items()}
        sub = {"embed": _host(w["embed"]), "layers": [lw]}
        one = dataclasses.replace(shape, n_layers=1)
        Lr, tr = lens[-1], toks[-1]  # the cache holds the last prompt after the timed loop
        n = 256
        t = []
        for start in (0, Lr - n):
            ck = [np.zeros((shape.n_kv_heads, start + n, shape.head_dim))]
            cv = [np.zeros((shape.n_kv_heads, start + n, shape.head_dim))]
            if start:
                ck[0][:, :start] = _host(kv.k[0, 0, :, :start])
                cv[0][:, :start] = _host(kv.v[0, 0, :, :start])
            t0 = time.perf_counter()
            om.prefill(sub, one, tr[start:start + n].cpu().numpy().astype(np.int64), ck, cv, start)
            t.append((time.perf_counter() - t0) / n)
        per_tok = 0.5 * (t[0] + t[1]) * shape.n_layers
        cpu = {"value": round(1.0 / per_tok, 2), "unit": "prompt tokens/s", "cores": _threads(), "kind": "oracle",
               "sample": f"float64 NumPy oracle prefill of one layer on 256 tokens at positions 0 and {Lr - n} "
                         f"of a {Lr}-token prompt ({t[0] * 1e3:.2f} and {t[1] * 1e3:.2f} ms/token), mean x "
                         f"{shape.n_layers} layers; host affinity {len(os.sched_getaffinity(0))} cpus"}
    out = base_line("prompt tokens/s (causal prefill, 1 GPU)", n_tok / (total_ms * 1e-3), "prompt tokens/s",
                    len(lens), 1, total_ms / len(lens), "bf16", "prefill_batch8_32k", 8, max(lens),
                    roofline=roofline, cpu_baseline=cpu, prompt_tokens=n_tok, prefix_lengths=lens,
                    wall_s_timed=round(t_wall, 3), **extra)
    out["ms_per_step"] = round(total_ms / len(lens), 3)  # per prompt
    print(json.dumps(out), flush=True)
    m.close()


def long_generation(args, dg, shape, w, cfg):
    """Prefill 8192 tokens, then 8 canvases, each denoised until the sampler stops and then
    committed (dg_commit_block), the next canvas attending to the grown cache.  The timed region
    is the whole block loop; one pinned status read per step is its only host synchronisation."""
    import torch
    from block_discrete_diffusion_amd import synth

    L0, n_blocks = 8192, 8
    m = dg.Model(shape, w, max_batch=1, max_prefill_rows=2048)
    kv = dg.KV(shape, 1, L0 + n_blocks * shape.canvas)
    log(f"prefill {L0}")
    m.prefill(torch.from_numpy(synth.tokens(L0, shape.vocab, SEED, 1)).cuda(), [L0], kv)
    torch.cuda.synchronize()
    stats = dg.Stats(1, shape.canvas)

    def one_block():
        st = dg.Canvas(1, shape.canvas)
        m.canvas_init(st, kv, cfg)
        res = m.denoise_canvas(st, kv, cfg, stats)
        m.commit_block(st.tokens, kv, any(d["changed"] for d in res["status"]))
        return res["steps"]

    log("warmup: one canvas (rolled back)")
    one_block()
    kv.set_lengths([L0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = []
    t_wall = time.perf_counter()
    e0.record()
    for j in range(n_blocks):
        steps.append(one_block())
        log(f"  canvas {j}: {steps[-1]} steps")
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    n_steps = sum(steps)
    final_len = kv.lengths[0]
    extra = {}
    if not args.no_kernel_timing:
        # per-kernel timing of the last canvas again (outside the timed region): its cache is
        # rolled back to the last block's prefix and the block re-run with the events on
        L_last = L0 + (n_blocks - 1) * shape.canvas
        kv.set_lengths([L_last])
        m.timing(True)
        one_block()
        torch.cuda.synchronize()
        kt = m.timing_read()
        m.timing(False)
        extra["attention_roofline"] = roofline_entry("mfma", "attention", kt, attention_flops(shape, [L_last]),
                                                     "flops", "long_generation", {"prefix": L_last})
        roofline = roofline_entry("hbm", "moe_gemm1_swiglu", kt,
                                  expert_gemm1_bytes(shape, shape.canvas * shape.top_k, shape.n_experts), "bytes",
                                  "long_generation")
    else:
        roofline = None
    cpu = None
    if not args.no_cpu_baseline:
        # one denoise step of the oracle over the last canvas's prefix (its GPU-filled bf16 K/V),
        # as for the batched workload with one request, then per finalised position: a canvas
        # took the mean steps per canvas of the GPU run
        log("CPU oracle baseline (bounded sample)")
        L_last = L0 + (n_blocks - 1) * shape.canvas
        cpu = cpu_baseline_batch(shape, w, kv, [L_last], args.cpu_sample_rows)
        spc = n_steps / n_blocks
        cpu["value"] = round(cpu["value"] / spc, 4)
        cpu["unit"] = "finalised canvas positions/s"
        cpu["sample"] += f"; per finalised position: divided by the {spc:g} steps per canvas of the GPU run"
    out = base_line("canvas positions/s (block-autoregressive generation, 1 GPU)",
                    n_blocks * shape.canvas / (total_ms * 1e-3), "finalised canvas positions/s", n_steps, 1,
                    total_ms / n_steps, "bf16", "long_generation", 1, L0 + n_blocks * shape.canvas,
                    steps_per_canvas=steps, canvas_ms=round(total_ms / n_blocks, 3), final_kv_len=final_len,
                    roofline=roofline, cpu_baseline=cpu, wall_s_timed=round(t_wall, 3), **extra)
    print(json.dumps(out), flush=True)
    m.close()


def continuous_serving(args, dg, shape, w, cfg):
    """Requests arrive over time and are served by the continuous batcher on a pool of slots: each
    scheduler iteration admits arrivals into free slots (causal prefill), runs one denoise +
    sampler step on every live canvas (each at its own step), and commits, restarts or releases
    the canvases that stopped.  The timed region is the whole serving run, host loop included."""
    import numpy as np
    import torch
    from block_discrete_diffusion_amd import synth
    from block_discrete_diffusion_amd.scheduler import ContinuousBatcher

    n_req, n_slots, gap = 24, 8, 6
    lens = synth.ragged_lengths(n_req, 2048, 0.5, SEED + 7)
    blocks = [1 + int(x) for x in np.random.default_rng(SEED + 8).integers(0, 3, n_req)]
    cap = max(lens) + max(blocks) * shape.canvas
    m = dg.Model(shape, w, max_batch=n_slots, max_prefill_rows=2048)
    prompts = [synth.tokens(L, shape.vocab, SEED, 100 + i) for i, L in enumerate(lens)]

    def serve(reqs, kv):
        t_arr, t_fin, rid_of = {}, {}, {}

        def on_event(ev, info):
            if ev == "finish":
                t_fin[info["rid"]] = time.perf_counter()

        b = ContinuousBatcher(m, kv, cfg, max_active=n_slots, trace=on_event)
        arrive = {i * gap: i for i in range(len(reqs))}
        while len(b.done) < len(reqs):
            i = arrive.get(b.iteration)
            if i is not None and i not in rid_of:
                rid_of[i] = b.submit(*reqs[i])
                t_arr[rid_of[i]] = time.perf_counter()
            if b.idle():  # nothing live before the next arrival: skip ahead
                b.iteration += 1
                continue
            b.step()
        torch.cuda.synchronize()
        return b, sorted(1e3 * (t_fin[r] - t_arr[r]) for r in t_fin)

    log("warmup: two short requests")
    kv_w = dg.KV(shape, n_slots, cap)
    serve([(prompts[0][:512], 1), (prompts[1][:300], 1)], kv_w)
    del kv_w
    kv = dg.KV(shape, n_slots, cap)
    reqs = list(zip(prompts, blocks))
    log(f"serving {n_req} requests, prompt lengths {min(lens)}-{max(lens)}, {sum(blocks)} blocks")
    t0 = time.perf_counter()
    b, lat = serve(reqs, kv)
    wall = time.perf_counter() - t0
    steps = [k for r in b.done.values() for k in r.steps_per_block]
    finals = sum(blocks) * shape.canvas
    out = base_line("canvas positions/s (continuous serving, 1 GPU)", finals / wall, "finalised canvas positions/s",
                    b.n_denoise_calls, 1, wall * 1e3 / b.n_denoise_calls, "bf16", "continuous_serving", n_slots, cap,
                    denoised_positions_per_s=round(b.n_positions / wall, 1),
                    mean_live_canvases=round(b.n_positions / shape.canvas / b.n_denoise_calls, 3),
                    prompt_tokens=int(sum(lens)), blocks=int(sum(blocks)),
                    steps_per_canvas_mean=round(float(np.mean(steps)), 2),
                    request_latency_ms={"p50": round(lat[len(lat) // 2], 1), "p90": round(lat[(9 * len(lat)) // 10], 1),
                                        "max": round(lat[-1], 1)},
                    roofline=None, cpu_baseline=None, wall_s_timed=round(wall, 3))
    print(json.dumps(out), flush=True)
    m.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="batch8_ragged_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the one-canvas extra keys of the default line")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the HIP-event per-kernel pass (e.g. under a profiler)")
    ap.add_argument("--cpu-sample-rows", type=int, default=64)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run one plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}). "
              "Independent requests would shard across GPUs with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_discrete_diffusion_amd import dg, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    cfg = dg.sampler_cfg(seed=SEED)
    if args.workload == "single_layer":
        return single_layer(args, dg, cfg)
    if args.workload == "tiny_loop":
        return tiny_loop(args, dg)
    shape = synth.FULL
    if args.workload == "full_canvas_loop_fp8":
        shape = dataclasses.replace(shape, expert_fp8=True)
    log("drawing weights on the device")
    w = synth.torch_model_weights(shape, "cuda", SEED)
    if args.workload == "prefill_batch8_32k":
        return prefill_workload(args, dg, shape, w)
    if args.workload == "long_generation":
        return long_generation(args, dg, shape, w, cfg)
    if args.workload == "continuous_serving":
        return continuous_serving(args, dg, shape, w, cfg)
    return canvas_workload(args, dg, shape, w, cfg, args.workload)


if __name__ == "__main__":
    main()
