"""Host-side checks of bench.py (no GPU): the per-launch work its rooflines divide by, the
HBM-counter guard, and the one-GPU refusal."""
import dataclasses
import os
import subprocess
import sys

import pytest

import bench
from block_discrete_diffusion_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_flops_count_every_query_key_pair():
    """4 D flops per (head, canvas query, key) triple (QK^T and PV, 2 flops per multiply-add),
    counted by enumerating the triples of a small ragged batch."""
    shape = dataclasses.replace(synth.TINY, canvas=3, n_q_heads=2, head_dim=4)
    lens = [0, 5, 2]
    triples = sum(1 for _ in range(shape.n_q_heads) for L in lens for _q in range(shape.canvas)
                  for _k in range(L + shape.canvas))
    assert bench.attention_flops(shape, lens) == 4 * shape.head_dim * triples


def test_attention_flops_of_the_ragged_workload():
    """The 8 x ~32 k workload's canvas attention: 593.9 GFLOP per launch (16 heads x 256 queries
    x (L_b + 256) keys x 512 flops)."""
    lens = synth.ragged_lengths(8, 32768, 0.25, bench.SEED)
    assert lens == [31672, 37674, 32010, 32993, 36578, 39977, 38367, 31878]
    assert bench.attention_flops(synth.FULL, lens) == 593907154944.0


def test_expert_gemm1_bytes_at_one_canvas_and_at_eight():
    """Gate and up matrices of all 64 experts (2 x 768 x 2048 bf16 each), the routed rows in
    (2048 bf16) and the SwiGLU rows out (768 bf16): 408.4 MB at 1024 routes, 448.8 MB at 8192."""
    w = 64 * 2 * 768 * 2048 * 2
    assert bench.expert_gemm1_bytes(synth.FULL, 1024, 64) == w + 1024 * 2048 * 2 + 1024 * 768 * 2 == 408420352
    assert bench.expert_gemm1_bytes(synth.FULL, 8192, 64) == w + 8192 * 2048 * 2 + 8192 * 768 * 2 == 448790528


def test_counter_traffic_only_for_its_workload_and_source(monkeypatch):
    """The stored HBM counters count only for the workload they were taken on and only while the
    kernel's source file is the one they were taken with."""
    fam = "attention"
    t = dict(bench.PMC_TRAFFIC[fam])
    want = t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]
    monkeypatch.setitem(bench.PMC_TRAFFIC, fam, dict(t, sha=bench.source_digest(t["source"])))
    assert bench.measured_traffic(fam, t["workload"]) == pytest.approx(want)
    assert bench.measured_traffic(fam, "full_canvas_loop") is None
    monkeypatch.setitem(bench.PMC_TRAFFIC, fam, dict(t, sha="0" * 16))
    assert bench.measured_traffic(fam, t["workload"]) is None
    assert bench.measured_traffic("no_such_kernel", t["workload"]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
