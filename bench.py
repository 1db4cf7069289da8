#!/usr/bin/env python3
"""Benchmark of the denoise step: canvas positions/s and ms per step on one MI355X.

Workload (default "full_canvas_loop"): the 12-layer MoE model (d 2048, 16 q / 8 kv heads,
head_dim 128, 64 experts top-4, d_ff 768, shared SwiGLU FFN 4096, vocab 65536), a prefix of 2048
random tokens prefilled causally (untimed), and one 256-token canvas run through the sampling
schedule (48-step cap, temperature 0.8 -> 0.4, commit 16, re-noise below 0.1).  A step is one
dg_denoise_step (embedding, 12 layers, final norm, fused vocab head) plus one dg_sample_commit;
steps cycle through the 48-step schedule (the canvas restarts after the cap).  Weights and
tokens are seeded synthetic data (no checkpoint exists), drawn on the device.

Output: one JSON line with the metric, a roofline entry for the dominant kernel (the expert
gate/up grouped GEMM, measured live with HIP events on its launch stream) and the CPU oracle
timed on a bounded sample of the same step.
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


# HBM traffic of the dominant kernel from hardware counters (rocprofv3 --pmc FETCH_SIZE, then
# WRITE_SIZE, in separate runs of this script), per launch, each scaled by the ratio
# true bytes / counter bytes that the same counter gives for a plain 1 GiB device copy.  Valid
# only for the kernel source it was taken on: a changed source reports traffic null.
PMC_TRAFFIC = {
    "kernel": "expert_stream_kernel<true, 3, 1, 1, false>", "source": "block_discrete_diffusion_amd/csrc/k_moe.hip",
    "sha": "b37d0147617978a9",
    "fetch_kib": 202317.0, "fetch_scale": 1048576.0 / 524307.7,  # copy of 1 GiB reads 524308 KiB
    "write_kib": 1550.0, "write_scale": 1048576.0 / 1048576.0,   # and writes 1048576 KiB
}


def source_digest(rel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    if PMC_TRAFFIC is None or source_digest(PMC_TRAFFIC["source"]) != PMC_TRAFFIC["sha"]:
        return None
    return PMC_TRAFFIC["fetch_kib"] * 1024 * PMC_TRAFFIC["fetch_scale"] + \
        PMC_TRAFFIC["write_kib"] * 1024 * PMC_TRAFFIC["write_scale"]


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


def cpu_baseline(shape, weights, prefix_len: int, sample_rows: int):
    """The CPU oracle, as it stands, on a bounded sample of one step: layer 0 over the 256 canvas
    rows (synthetic residual state and random bf16 prefix K/V), the fused head on `sample_rows`
    rows, and the sampler on 256 positions; scaled to a full step (n_layers layers, 256 head rows).
    The oracle gets the same synthetic weights the GPU uses (copied from the device RNG draw)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from block_discrete_diffusion_amd import synth
    from oracle import model as om
    from oracle import sampler as osm

    d, D, V = shape.d_model, shape.head_dim, shape.vocab
    lw = {k: _host(v) for k, v in weights["layers"][0].items()}
    k = synth.bf16_normal((shape.n_kv_heads, prefix_len, D), SEED, 101)
    v = synth.bf16_normal((shape.n_kv_heads, prefix_len, D), SEED, 102)
    h = synth.hidden(256, d, SEED, 103)
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        om.layer(h, lw, shape, prefix_len + np.arange(256), k, v, None)
    t_layer = (time.perf_counter() - t0) / reps
    del lw
    head = _host(weights["lm_head"])
    f = synth.bf16_normal((sample_rows, d), SEED, 104)
    x = synth.tokens(sample_rows, V, SEED, 105)
    cfg = osm.SamplerConfig(seed=1)
    t0 = time.perf_counter()
    z = om.head_logits(f, head)
    st = osm.row_stats(z, x, osm.temperature(cfg, 0), cfg.seed, 0, prefix_len + np.arange(sample_rows), 0)
    t_head = (time.perf_counter() - t0) * 256 / sample_rows
    full = {kk: np.resize(vv, 256) for kk, vv in st.items()}
    t0 = time.perf_counter()
    osm.sample_commit(full, synth.tokens(256, V, SEED, 106), np.zeros(256, bool), 0, cfg, 0, 0,
                      prefix_len + np.arange(256), V)
    t_samp = time.perf_counter() - t0
    t_step = shape.n_layers * t_layer + t_head + t_samp
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": 256.0 / t_step, "unit": "canvas positions/s", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: 1 layer x 256 canvas rows (prefix {prefix_len}, mean of {reps}) "
                   f"scaled x{shape.n_layers}, "
                   f"head + Gumbel row stats on {sample_rows} rows scaled x{256 // sample_rows}, sampler on 256; "
                   f"est. {t_step * 1e3:.0f} ms/step (layer {t_layer * 1e3:.0f} ms, head {t_head * 1e3:.0f} ms, "
                   f"sampler {t_samp * 1e3:.1f} ms); host affinity {len(os.sched_getaffinity(0))} cpus"),
    }


WORKLOADS = {
    "full_canvas_loop": "12 layers d2048 16q/8kv hd128, 64 experts top-4 d_ff 768 + shared FFN 4096, "
                        "vocab 65536, prefix 2048, canvas 256, sampler 48 steps 0.8->0.4 commit 16",
    "batch8_ragged_32k": "same model, 8 requests with prefixes round(32768*(1+U(-1/4,1/4))) prefilled "
                         "causally, 8 canvases of 256 denoised together (2048 rows per step)",
    "long_generation": "same model, prefix 8192, 8 consecutive canvases each denoised until the sampler "
                       "stops and then committed to the KV cache (final length 10240)",
    "full_canvas_loop_fp8": "the full canvas loop with the routed experts quantized to OCP E4M3 "
                            "(per-channel float32 scales); everything else bf16",
    "continuous_serving": "same model, 24 requests (prompts round(2048*(1+U(-1/2,1/2))), 1-3 blocks each) "
                          "arriving one every 6 scheduler iterations, served on 8 cache slots with up to "
                          "8 live canvases per call; prefill, sampling loop and block commits all timed",
}


def attention_flops(shape, lens) -> float:
    """Algorithmic MFMA flops of one canvas-attention launch: QK^T and PV over the cached prefix
    plus the canvas, 2 flops per multiply-add each."""
    C = shape.canvas
    return float(4 * shape.n_q_heads * shape.head_dim * sum(C * (L + C) for L in lens))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="full_canvas_loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    shape = synth.FULL
    if args.workload == "full_canvas_loop_fp8":
        shape = dataclasses.replace(shape, expert_fp8=True)
    log("drawing weights on the device")
    w = synth.torch_model_weights(shape, "cuda", SEED)
    cfg = dg.sampler_cfg(seed=SEED)
    if args.workload == "long_generation":
        return long_generation(args, shape, w, cfg)
    if args.workload == "continuous_serving":
        return continuous_serving(args, shape, w, cfg)

    if args.workload == "batch8_ragged_32k":
        lens = synth.ragged_lengths(8, 32768, 0.25, SEED)
    else:
        lens = [2048]
    B = len(lens)
    m = dg.Model(shape, w, max_batch=B, max_prefill_rows=2048)
    kv = dg.KV(shape, B, max(lens) + shape.canvas)
    log(f"prefill {B} request(s), lengths {lens}")
    t0 = time.perf_counter()
    for b, L in enumerate(lens):  # one request at a time keeps progress visible
        n = [0] * B
        n[b] = L
        m.prefill(torch.from_numpy(synth.tokens(L, shape.vocab, SEED, 1 + b)).cuda(), n, kv)
        torch.cuda.synchronize()
        log(f"  request {b}: {L} tokens, {time.perf_counter() - t0:.1f} s")
    st = dg.Canvas(B, shape.canvas)
    stats = dg.Stats(B, shape.canvas)
    status = torch.zeros((B, 8), dtype=torch.int32, device="cuda")
    m.canvas_init(st, kv, cfg)
    counter = {"s": 0}

    def step():
        s = counter["s"]
        if s == cfg.max_steps:
            m.canvas_init(st, kv, cfg)
            s = 0
        m.denoise_step(st.tokens, kv, cfg, s, stats)
        m.sample_commit(st, stats, cfg, s, kv, status)
        counter["s"] = s + 1

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    value = B * shape.canvas / (ms * 1e-3)

    roofline = None
    kernels = None
    extra = {}
    if not args.no_kernel_timing:
        m.timing(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        kt = m.timing_read()
        m.timing(False)
        kernels = {k: round(v["total_ms"] / args.steps * 1e3, 2) for k, v in kt.items()}  # us per step
        g1 = kt["moe_gemm1_swiglu"]
        routes = B * shape.canvas * shape.top_k
        nbytes = expert_gemm1_bytes(shape, routes, shape.n_experts)
        ach = nbytes / (g1["avg_ms"] * 1e-3) / 1e9
        gemm1 = {"bound": "hbm", "kernel": "moe_gemm1_swiglu", "achieved": round(ach, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                 "traffic": measured_traffic() if args.workload == "full_canvas_loop" else None,
                 "avg_launch_us": round(g1["avg_ms"] * 1e3, 2), "algorithmic_bytes_per_launch": nbytes}
        at = kt["attention"]
        fl = attention_flops(shape, lens)
        tf = fl / (at["avg_ms"] * 1e-3) / 1e12
        attn = {"bound": "mfma", "kernel": "attention (+ split combine)", "achieved": round(tf, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": None, "avg_launch_us": round(at["avg_ms"] * 1e3, 2),
                "algorithmic_flops_per_launch": fl}
        roofline = gemm1 if args.workload.startswith("full_canvas_loop") else attn
        extra["attention_roofline"] = attn
        extra["expert_gemm1_roofline"] = gemm1
    cpu = None
    if not args.no_cpu_baseline and args.workload == "full_canvas_loop":
        log("CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(shape, w, lens[0], args.cpu_sample_rows)
    out = {
        "metric": "canvas positions/s (denoise step, 1 GPU)", "value": round(value, 1),
        "unit": "canvas positions/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16, routed experts e4m3" if shape.expert_fp8 else "bf16",
        "data": "synthetic (seeded device RNG weights, uniform random tokens)",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}",
                   "global_batch": B, "seq_len": max(lens) + shape.canvas, "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "kernel_us_per_step": kernels,
        "wall_s_timed": round(t_wall, 3), **extra,
    }
    print(json.dumps(out), flush=True)
    m.close()


def long_generation(args, shape, w, cfg):
    """Prefill 8192 tokens, then 8 canvases, each denoised until the sampler stops and then
    committed (dg_commit_block), the next canvas attending to the grown cache.  The timed region
    is the whole block loop; one pinned status read per step is its only host synchronisation."""
    import torch
    from block_discrete_diffusion_amd import dg, synth

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

    # warm-up on a scratch copy of the lengths: run one canvas, then roll the cache length back
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
    out = {
        "metric": "canvas positions/s (block-autoregressive generation, 1 GPU)",
        "value": round(n_blocks * shape.canvas / (total_ms * 1e-3), 1), "unit": "finalised canvas positions/s",
        "n_gpus": 1, "steps": n_steps, "warmup": 1, "ms_per_step": round(total_ms / n_steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded device RNG weights, uniform random tokens)",
        "config": {"workload": f"long_generation: {WORKLOADS['long_generation']}", "global_batch": 1,
                   "seq_len": L0 + n_blocks * shape.canvas, "parallelism": "single GPU"},
        "steps_per_canvas": steps, "canvas_ms": round(total_ms / n_blocks, 3),
        "final_kv_len": kv.lengths[0], "roofline": None, "cpu_baseline": None,
        "wall_s_timed": round(t_wall, 3),
    }
    print(json.dumps(out), flush=True)
    m.close()


def continuous_serving(args, shape, w, cfg):
    """Requests arrive over time and are served by the continuous batcher on a pool of slots: each
    scheduler iteration admits arrivals into free slots (causal prefill), runs one denoise +
    sampler step on every live canvas (each at its own step), and commits, restarts or releases
    the canvases that stopped.  The timed region is the whole serving run, host loop included."""
    import numpy as np
    import torch
    from block_discrete_diffusion_amd import dg, synth
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
    out = {
        "metric": "canvas positions/s (continuous serving, 1 GPU)",
        "value": round(finals / wall, 1), "unit": "finalised canvas positions/s",
        "n_gpus": 1, "steps": b.n_denoise_calls, "warmup": 1,
        "ms_per_step": round(wall * 1e3 / b.n_denoise_calls, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded device RNG weights, uniform random tokens)",
        "config": {"workload": f"continuous_serving: {WORKLOADS['continuous_serving']}",
                   "global_batch": n_slots, "seq_len": cap, "parallelism": "single GPU"},
        "denoised_positions_per_s": round(b.n_positions / wall, 1),
        "mean_live_canvases": round(b.n_positions / shape.canvas / b.n_denoise_calls, 3),
        "prompt_tokens": int(sum(lens)), "blocks": int(sum(blocks)),
        "steps_per_canvas_mean": round(float(np.mean(steps)), 2),
        "request_latency_ms": {"p50": round(lat[len(lat) // 2], 1), "p90": round(lat[(9 * len(lat)) // 10], 1),
                               "max": round(lat[-1], 1)},
        "roofline": None, "cpu_baseline": None, "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    m.close()


if __name__ == "__main__":
    main()
