"""C-ABI checks that need no GPU: the library loads, exports every function include/dg.h declares,
rejects bad shapes before touching the device, and its host-side schedule matches the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_discrete_diffusion_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary_calls():
    names = _declared()
    for n in ("dg_prefill_causal", "dg_denoise_step", "dg_sample_commit", "dg_commit_block"):
        assert n in names


def test_library_exports_every_declared_symbol():
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    lib = ctypes.CDLL(dg.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(dg.EXPORTS) == _declared()


def _desc(dg, **kw):
    s = synth.TINY
    base = dict(n_layers=s.n_layers, d_model=s.d_model, n_q_heads=s.n_q_heads, n_kv_heads=s.n_kv_heads,
                head_dim=s.head_dim, n_experts=s.n_experts, top_k=s.top_k, d_ff_expert=s.d_ff_expert,
                d_ff_shared=s.d_ff_shared, vocab=s.vocab, canvas=256, rms_eps=1e-6, rope_theta=1e4,
                expert_fp8=0)
    base.update(kw)
    return dg.ModelDesc(*[base[n] for n, _ in dg.ModelDesc._fields_])


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), -2), (dict(canvas=128), -2), (dict(n_kv_heads=3), -2),
    (dict(top_k=9), -2), (dict(n_experts=65, top_k=2), -2), (dict(vocab=1000), -2),
    (dict(d_model=200), -2), (dict(rms_eps=0.0), -2), (dict(vocab=131072 + 128), -2),
])
def test_create_rejects_bad_shapes_before_any_device_work(bad, code):
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    desc = _desc(dg, **bad)
    layers = (dg.LayerWeights * 2)()
    w = dg.Weights(None, None, None, layers)
    h = ctypes.c_void_p()
    rc = dg._lib.dg_create(ctypes.byref(desc), ctypes.byref(w), 1, 256, ctypes.byref(h))
    assert rc == code
    assert b"unsupported model shape" in dg._lib.dg_last_error(None)
    assert not h.value


def test_create_rejects_null_weights():
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    desc = _desc(dg)
    layers = (dg.LayerWeights * 2)()
    w = dg.Weights(None, None, None, layers)
    h = ctypes.c_void_p()
    assert dg._lib.dg_create(ctypes.byref(desc), ctypes.byref(w), 1, 256, ctypes.byref(h)) == -1
    assert dg._lib.dg_create(ctypes.byref(desc), ctypes.byref(w), 0, 256, ctypes.byref(h)) == -1
    assert dg._lib.dg_create(None, ctypes.byref(w), 1, 256, ctypes.byref(h)) == -1


def test_null_context_is_rejected():
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    assert dg._lib.dg_denoise_step(None, None, None, None, None, None, None) == -1
    assert dg._lib.dg_sample_commit(None, None, None, None, 0, None, None, None, None) == -1
    assert dg._lib.dg_commit_block(None, None, None, 0, None) == -1
    assert dg._lib.dg_prefill_causal(None, None, None, 0, None, None) == -1
    assert dg._lib.dg_quantize_e4m3_rows(None, 4, 16, None, None, None) == -1
    assert b"null pointer" in dg._lib.dg_last_error(None)


def test_temperature_schedule_matches_oracle_bitexact():
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    from oracle import sampler
    for ms, t0, t1 in [(48, 0.8, 0.4), (10, 1.0, 0.25), (1, 0.7, 0.3)]:
        cfg = dg.sampler_cfg(max_steps=ms, temp_start=t0, temp_end=t1)
        oc = sampler.SamplerConfig(max_steps=ms, temp_start=float(np.float32(t0)), temp_end=float(np.float32(t1)))
        for s in range(ms):
            assert np.float32(dg.temperature(cfg, s)) == sampler.temperature(oc, s)


def test_binding_structs_match_the_header_layout(tmp_path):
    """Every ctypes structure of the binding has the size and field offsets that a C compiler
    gives the struct of the same role in include/dg.h."""
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    pairs = {"dg_model_desc": dg.ModelDesc, "dg_layer_weights": dg.LayerWeights,
             "dg_weights": dg.Weights, "dg_kv_cache": dg.KVCache,
             "dg_canvas_state": dg.CanvasState, "dg_row_stats": dg.RowStats,
             "dg_sampler_cfg": dg.SamplerCfg, "dg_debug": dg.Debug,
             "dg_step_params": dg.StepParams, "dg_kernel_time": dg.KernelTime}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dg.h"', "int main(void) {"]
    for cname, py in pairs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f in py._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ["return 0; }"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, val = ln.split()
        got[(cname, field)] = int(val)
    for cname, py in pairs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for f in py._fields_:
            assert got[(cname, f[0])] == getattr(py, f[0]).offset, (cname, f[0])


def test_binding_rejects_token_ids_outside_the_vocabulary():
    """The binding checks the token-range precondition of dg_prefill_causal / dg_denoise_step
    before anything reaches the device: host arrays and CPU tensors here."""
    import torch
    dg = pytest.importorskip("block_discrete_diffusion_amd.dg")
    dg.check_token_range(np.array([0, 5, 1023]), 1024)
    dg.check_token_range(torch.tensor([0, 1023], dtype=torch.int32), 1024)
    dg.check_token_range(np.zeros(0, np.int32), 1024)
    for bad in ([0, 1024], [-1, 3], [2 ** 31 - 1]):
        with pytest.raises(ValueError):
            dg.check_token_range(np.array(bad, np.int64), 1024)
        with pytest.raises(ValueError):
            dg.check_token_range(torch.tensor(bad, dtype=torch.int64), 1024)
