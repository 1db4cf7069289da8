"""ctypes binding of libdg (include/dg.h).  Argument marshalling only: every step of the denoise
path runs in the HIP kernels of libdg.so.  PyTorch supplies device memory and the stream.

Loading fails loudly (ImportError) when libdg.so has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m block_discrete_diffusion_amd.build_lib` (hipcc, gfx950)")
_lib = C.CDLL(LIB_PATH)

DG_OK, DG_ERR_ARG, DG_ERR_SHAPE, DG_ERR_CAPACITY, DG_ERR_HIP, DG_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
DG_STEP_HIDDEN_IN, DG_STEP_NO_HEAD, DG_STEP_HEAD_ONLY = 1, 2, 4

EXPORTS = ["dg_create", "dg_destroy", "dg_last_error", "dg_temperature", "dg_prefill_causal",
           "dg_canvas_init", "dg_denoise_step", "dg_sample_commit", "dg_commit_block",
           "dg_timing_enable", "dg_timing_read", "dg_debug_set_canvas_kv", "dg_quantize_e4m3_rows",
           "dg_device_errors", "dg_denoise_head_static"]
DG_DEVERR_TOKEN_RANGE = 1

vp = C.c_void_p


class ModelDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim",
                                         "n_experts", "top_k", "d_ff_expert", "d_ff_shared", "vocab",
                                         "canvas")] + [("rms_eps", C.c_float), ("rope_theta", C.c_float),
                                                       ("expert_fp8", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_router", "w_gate",
                                  "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class Weights(C.Structure):
    _fields_ = [("embed", vp), ("final_norm", vp), ("lm_head", vp), ("layers", C.POINTER(LayerWeights))]


class KVCache(C.Structure):
    _fields_ = [("k", vp), ("v", vp), ("cap", C.c_int32), ("batch", C.c_int32), ("len", C.POINTER(C.c_int32)),
                ("slot", C.POINTER(C.c_int32)), ("n_slots", C.c_int32)]


class CanvasState(C.Structure):
    _fields_ = [("tokens", vp), ("committed", vp), ("stable_run", vp), ("stopped", vp)]


class RowStats(C.Structure):
    _fields_ = [("cand", vp), ("t_cand", vp), ("t_cur", vp), ("lse", vp), ("entropy", vp)]


class SamplerCfg(C.Structure):
    _fields_ = [("max_steps", C.c_int32), ("temp_start", C.c_float), ("temp_end", C.c_float),
                ("commit_per_step", C.c_int32), ("renoise_conf", C.c_float), ("stable_steps", C.c_int32),
                ("entropy_stop", C.c_float), ("renoise_committed", C.c_int32), ("seed", C.c_uint64),
                ("select_mode", C.c_int32), ("entropy_budget", C.c_float)]


class Debug(C.Structure):
    _fields_ = [(n, vp) for n in ("hidden_out", "attn_out", "h_mid", "expert_idx", "gates", "logits",
                                  "canvas_k", "canvas_v", "layer_out", "route_offs", "route_perm",
                                  "route_inv")]


class StepParams(C.Structure):
    _fields_ = [("step", C.c_int32), ("flags", C.c_uint32), ("hidden_in", vp), ("debug", C.POINTER(Debug)),
                ("steps", C.POINTER(C.c_int32))]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char_p), ("launches", C.c_int32), ("total_ms", C.c_float)]


STATUS_FIELDS = ("changed", "n_committed", "n_new", "n_renoised", "stable_run", "stop", "nonfinite")

_lib.dg_create.argtypes = [C.POINTER(ModelDesc), C.POINTER(Weights), C.c_int32, C.c_int32, C.POINTER(vp)]
_lib.dg_create.restype = C.c_int
_lib.dg_destroy.argtypes = [vp]
_lib.dg_destroy.restype = None
_lib.dg_last_error.argtypes = [vp]
_lib.dg_last_error.restype = C.c_char_p
_lib.dg_temperature.argtypes = [C.POINTER(SamplerCfg), C.c_int32]
_lib.dg_temperature.restype = C.c_float
_lib.dg_prefill_causal.argtypes = [vp, vp, C.POINTER(C.c_int32), C.c_int32, C.POINTER(KVCache), vp]
_lib.dg_canvas_init.argtypes = [vp, C.POINTER(CanvasState), C.POINTER(KVCache), C.POINTER(SamplerCfg), vp]
_lib.dg_denoise_step.argtypes = [vp, vp, C.POINTER(KVCache), C.POINTER(SamplerCfg), C.POINTER(StepParams),
                                 C.POINTER(RowStats), vp]
_lib.dg_sample_commit.argtypes = [vp, C.POINTER(CanvasState), C.POINTER(RowStats), C.POINTER(SamplerCfg),
                                  C.c_int32, C.POINTER(C.c_int32), C.POINTER(KVCache), vp, vp]
_lib.dg_commit_block.argtypes = [vp, vp, C.POINTER(KVCache), C.c_int32, vp]
_lib.dg_debug_set_canvas_kv.argtypes = [vp, vp, vp, C.c_int32, vp]
_lib.dg_timing_enable.argtypes = [vp, C.c_int32]
_lib.dg_timing_read.argtypes = [vp, C.POINTER(KernelTime), C.c_int32]
_lib.dg_quantize_e4m3_rows.argtypes = [vp, C.c_int64, C.c_int32, vp, vp, vp]
_lib.dg_device_errors.argtypes = [vp, C.POINTER(C.c_uint32), vp]
_lib.dg_denoise_head_static.argtypes = [vp, vp, C.POINTER(KVCache), C.POINTER(SamplerCfg), C.POINTER(StepParams),
                                        C.POINTER(RowStats), vp]
for _n in ("dg_timing_enable", "dg_timing_read", "dg_prefill_causal", "dg_canvas_init", "dg_denoise_step", "dg_sample_commit",
           "dg_commit_block", "dg_debug_set_canvas_kv", "dg_quantize_e4m3_rows", "dg_device_errors",
           "dg_denoise_head_static"):
    getattr(_lib, _n).restype = C.c_int


class DGError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdg error {code}: {msg}")
        self.code = code


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def to_device_bf16(x, device) -> torch.Tensor:
    """float32 array of bf16-exact values (or a bf16 tensor) → contiguous bf16 device tensor."""
    if isinstance(x, torch.Tensor):
        return x.to(device=device, dtype=torch.bfloat16).contiguous()
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device).contiguous()


def check_token_range(tokens, vocab: int, what: str = "tokens") -> None:
    """Raise ValueError unless every id in `tokens` (numpy array, or torch tensor on any device)
    lies in [0, vocab): the precondition of dg_prefill_causal and dg_denoise_step.  A device
    tensor is checked with one reduction on the device and a host read."""
    if isinstance(tokens, torch.Tensor):
        if tokens.numel() == 0:
            return
        lo, hi = (int(v) for v in torch.aminmax(tokens.reshape(-1)))
    else:
        a = np.asarray(tokens)
        if a.size == 0:
            return
        lo, hi = int(a.min()), int(a.max())
    if lo < 0 or hi >= int(vocab):
        raise ValueError(f"{what}: token ids must lie in [0, {int(vocab)}), got [{lo}, {hi}]")


SELECT_TOP_M, SELECT_ENTROPY = 0, 1
COMMIT_LAST, COMMIT_REFRESH, COMMIT_CAUSAL = 0, 1, 2


def sampler_cfg(max_steps=48, temp_start=0.8, temp_end=0.4, commit_per_step=16, renoise_conf=0.1,
                stable_steps=2, entropy_stop=-1.0, renoise_committed=True, seed=0,
                select_mode=SELECT_TOP_M, entropy_budget=0.1) -> SamplerCfg:
    return SamplerCfg(int(max_steps), float(temp_start), float(temp_end), int(commit_per_step),
                      float(renoise_conf), int(stable_steps), float(entropy_stop),
                      int(bool(renoise_committed)), int(seed) & ((1 << 64) - 1), int(select_mode),
                      float(entropy_budget))


def temperature(cfg: SamplerCfg, step: int) -> float:
    return float(_lib.dg_temperature(C.byref(cfg), int(step)))


def quantize_e4m3_rows(w: torch.Tensor, q: torch.Tensor, scale: torch.Tensor) -> None:
    """dg_quantize_e4m3_rows on device tensors: w bf16 [rows, cols], q uint8 [rows, cols],
    scale float32 [rows] (all contiguous, on the GPU)."""
    if w.dtype != torch.bfloat16 or q.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise TypeError("quantize_e4m3_rows: w bf16, q uint8, scale float32")
    if w.dim() != 2 or tuple(q.shape) != tuple(w.shape) or tuple(scale.shape) != (w.shape[0],):
        raise ValueError("quantize_e4m3_rows: shapes w [rows, cols], q [rows, cols], scale [rows]")
    if not (w.is_contiguous() and q.is_contiguous() and scale.is_contiguous()):
        raise ValueError("quantize_e4m3_rows: contiguous tensors only")
    rc = _lib.dg_quantize_e4m3_rows(_ptr(w), int(w.shape[0]), int(w.shape[1]), _ptr(q), _ptr(scale), _stream())
    if rc != DG_OK:
        raise DGError(rc, _lib.dg_last_error(None).decode())


class KV:
    """bf16 KV cache [n_layers][batch][Hkv][cap][D] on the device + host lengths."""

    def __init__(self, shape, batch: int, cap: int, device="cuda", fill: Optional[float] = 0.0):
        dims = (shape.n_layers, batch, shape.n_kv_heads, cap, shape.head_dim)
        self.k = torch.empty(dims, dtype=torch.bfloat16, device=device)
        self.v = torch.empty(dims, dtype=torch.bfloat16, device=device)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)
        self.len = (C.c_int32 * batch)(*([0] * batch))
        self.n_slots = batch
        self.c = KVCache(_ptr(self.k), _ptr(self.v), cap, batch, C.cast(self.len, C.POINTER(C.c_int32)),
                         C.POINTER(C.c_int32)(), batch)

    @property
    def lengths(self) -> List[int]:
        return list(self.len)

    def set_lengths(self, lens: Sequence[int]):
        for b, v in enumerate(lens):
            self.len[b] = int(v)

    def view(self, slots: Optional[Sequence[int]]):
        """The cache as seen by a call on the requests in `slots` (all slots when None)."""
        return _KVView(self, slots)


class _KVView:
    """A dg_kv_cache for a call on some slots of a KV: its lengths are copied in, and back out
    after the call (prefill and commit advance them)."""

    def __init__(self, kv: "KV", slots: Optional[Sequence[int]]):
        self.kv = kv
        self.slots = None if slots is None else [int(x) for x in slots]
        if self.slots is None:
            self.c = kv.c
            return
        n = len(self.slots)
        self._len = (C.c_int32 * n)(*[kv.len[x] for x in self.slots])
        self._slot = (C.c_int32 * n)(*self.slots)
        self.c = KVCache(kv.c.k, kv.c.v, kv.c.cap, n, C.cast(self._len, C.POINTER(C.c_int32)),
                         C.cast(self._slot, C.POINTER(C.c_int32)), kv.n_slots)

    def done(self):
        if self.slots is not None:
            for i, x in enumerate(self.slots):
                self.kv.len[x] = self._len[i]


class Canvas:
    def __init__(self, batch: int, canvas: int, device="cuda"):
        self.tokens = torch.zeros((batch, canvas), dtype=torch.int32, device=device)
        self.committed = torch.zeros((batch, canvas), dtype=torch.uint8, device=device)
        self.stable_run = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.stopped = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.c = CanvasState(_ptr(self.tokens), _ptr(self.committed), _ptr(self.stable_run),
                             _ptr(self.stopped))


class Stats:
    def __init__(self, batch: int, canvas: int, device="cuda"):
        z = lambda dt: torch.zeros((batch, canvas), dtype=dt, device=device)
        self.cand = z(torch.int32)
        self.t_cand, self.t_cur, self.lse, self.entropy = (z(torch.float32) for _ in range(4))
        self.c = RowStats(_ptr(self.cand), _ptr(self.t_cand), _ptr(self.t_cur), _ptr(self.lse),
                          _ptr(self.entropy))


def status_dict(raw: torch.Tensor) -> List[Dict]:
    """Decode a [batch][8] int32 status tensor (dg_step_status) on the host."""
    a = raw.cpu().numpy()
    out = []
    for row in a:
        d = {k: int(row[i]) for i, k in enumerate(STATUS_FIELDS)}
        d["mean_entropy"] = float(row[7:8].view(np.float32)[0])
        out.append(d)
    return out


class Model:
    """Device weights + a libdg context.

    weights: dict as produced by synth.model_weights (float32 bf16-exact numpy arrays) or
    synth.torch_model_weights (device tensors)."""

    def __init__(self, shape, weights: Dict, max_batch: int = 1, max_prefill_rows: int = 2048,
                 device="cuda"):
        self.shape = shape
        self.device = device
        dev = torch.device(device)
        f32 = lambda x: (x if isinstance(x, torch.Tensor) else torch.from_numpy(np.asarray(x, np.float32))).to(
            dev, torch.float32).contiguous()
        self.t = {"embed": to_device_bf16(weights["embed"], dev), "final_norm": f32(weights["final_norm"]),
                  "lm_head": to_device_bf16(weights["lm_head"], dev), "layers": []}
        arr = (LayerWeights * shape.n_layers)()
        for l, lw in enumerate(weights["layers"]):
            t = {}
            for k, v in lw.items():
                t[k] = f32(v) if k.endswith("norm") else to_device_bf16(v, dev)
            self.t["layers"].append(t)
            get = lambda k: _ptr(t.get(k))
            arr[l] = LayerWeights(get("attn_norm"), get("wq"), get("wk"), get("wv"), get("wo"),
                                  get("ffn_norm"), get("w_router"), get("w_gate"), get("w_up"),
                                  get("w_down"), get("ws_gate"), get("ws_up"), get("ws_down"))
        self._layers = arr
        self.w = Weights(_ptr(self.t["embed"]), _ptr(self.t["final_norm"]), _ptr(self.t["lm_head"]), arr)
        self.desc = ModelDesc(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                              shape.n_experts, shape.top_k, shape.d_ff_expert, shape.d_ff_shared, shape.vocab,
                              shape.canvas, float(shape.rms_eps), float(shape.rope_theta),
                              int(bool(shape.expert_fp8)))
        h = C.c_void_p()
        rc = _lib.dg_create(C.byref(self.desc), C.byref(self.w), int(max_batch), int(max_prefill_rows),
                            C.byref(h))
        if rc != DG_OK:
            raise DGError(rc, _lib.dg_last_error(None).decode())
        self.ctx = h
        self.max_batch = max_batch

    def close(self):
        if getattr(self, "ctx", None):
            _lib.dg_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int):
        if rc != DG_OK:
            raise DGError(rc, _lib.dg_last_error(self.ctx).decode())

    # ---------------------------------------------------------------- entry points
    # `slots`: run the call on those slots of kv (and of the per-slot arrays) only; None = all.
    def prefill(self, tokens: torch.Tensor, n_new: Sequence[int], kv: KV, slots=None):
        check_token_range(tokens[:sum(int(v) for v in n_new)], self.shape.vocab, "prefill tokens")
        n = (C.c_int32 * len(n_new))(*[int(v) for v in n_new])
        view = kv.view(slots)
        self._check(_lib.dg_prefill_causal(self.ctx, _ptr(tokens), n, len(n_new), C.byref(view.c), _stream()))
        view.done()

    def canvas_init(self, state: Canvas, kv: KV, cfg: SamplerCfg, slots=None):
        view = kv.view(slots)
        self._check(_lib.dg_canvas_init(self.ctx, C.byref(state.c), C.byref(view.c), C.byref(cfg), _stream()))

    def denoise_step(self, canvas: Optional[torch.Tensor], kv: KV, cfg: Optional[SamplerCfg], step: int,
                     out: Optional[Stats], flags: int = 0, hidden_in: Optional[torch.Tensor] = None,
                     debug: Optional[Dict[str, torch.Tensor]] = None, slots=None):
        dbg = None
        if debug:
            dbg = Debug(*[_ptr(debug.get(n)) for n, _ in Debug._fields_])
        steps_arr = None
        if not isinstance(step, (int, np.integer)):  # one step per request of the call
            steps_arr = (C.c_int32 * len(step))(*[int(x) for x in step])
            step = 0
        p = StepParams(int(step), int(flags), _ptr(hidden_in), C.pointer(dbg) if dbg is not None else None,
                       C.cast(steps_arr, C.POINTER(C.c_int32)) if steps_arr is not None else None)
        view = kv.view(slots)
        self._check(_lib.dg_denoise_step(self.ctx, _ptr(canvas), C.byref(view.c),
                                         C.byref(cfg) if cfg is not None else None, C.byref(p),
                                         C.byref(out.c) if out is not None else None, _stream()))

    def sample_commit(self, state: Canvas, stats: Stats, cfg: SamplerCfg, step: int, kv: KV,
                      status: torch.Tensor, slots=None):
        view = kv.view(slots)
        steps_arr = None
        if not isinstance(step, (int, np.integer)):  # one step per request of the call
            steps_arr = (C.c_int32 * len(step))(*[int(x) for x in step])
            step = 0
        self._check(_lib.dg_sample_commit(self.ctx, C.byref(state.c), C.byref(stats.c), C.byref(cfg),
                                          int(step), steps_arr, C.byref(view.c), _ptr(status), _stream()))

    def commit_block(self, canvas: torch.Tensor, kv: KV, refresh, slots=None):
        """refresh: COMMIT_LAST (0 / False), COMMIT_REFRESH (1 / True) or COMMIT_CAUSAL (2)."""
        view = kv.view(slots)
        self._check(_lib.dg_commit_block(self.ctx, _ptr(canvas), C.byref(view.c), int(refresh), _stream()))
        view.done()

    def device_errors(self) -> int:
        """Sticky device-side error bits since the last read (DG_DEVERR_*); waits for the stream."""
        v = C.c_uint32(0)
        self._check(_lib.dg_device_errors(self.ctx, C.byref(v), _stream()))
        return int(v.value)

    def timing(self, enable: bool):
        self._check(_lib.dg_timing_enable(self.ctx, int(bool(enable))))

    def timing_read(self) -> Dict[str, Dict]:
        """{kernel family: {"launches": n, "total_ms": t, "avg_ms": t/n}} since the last read."""
        buf = (KernelTime * 64)()
        n = _lib.dg_timing_read(self.ctx, buf, 64)
        if n < 0:
            self._check(n)
        return {buf[i].name.decode(): {"launches": buf[i].launches, "total_ms": buf[i].total_ms,
                                       "avg_ms": buf[i].total_ms / max(1, buf[i].launches)} for i in range(n)}

    def set_canvas_kv(self, k: torch.Tensor, v: torch.Tensor, batch: int):
        self._check(_lib.dg_debug_set_canvas_kv(self.ctx, _ptr(k), _ptr(v), int(batch), _stream()))

    # ---------------------------------------------------------------- block-AR driver
    def denoise_canvas(self, state: Canvas, kv: KV, cfg: SamplerCfg, stats: Optional[Stats] = None,
                       on_step=None) -> Dict:
        """Run the sampling loop on every canvas of `state` until all requests stop.  One pinned
        32-byte-per-request status read per step is the only host synchronisation."""
        B = kv.c.batch
        stats = stats or Stats(B, self.shape.canvas, self.device)
        status = torch.zeros((B, 8), dtype=torch.int32, device=self.device)
        host = torch.zeros((B, 8), dtype=torch.int32, pin_memory=True)
        steps, last = 0, None
        for s in range(cfg.max_steps):
            self.denoise_step(state.tokens, kv, cfg, s, stats)
            self.sample_commit(state, stats, cfg, s, kv, status)
            host.copy_(status, non_blocking=True)
            torch.cuda.current_stream().synchronize()
            last = status_dict(host)
            steps += 1
            if on_step:
                on_step(s, last)
            if all(d["stop"] for d in last):
                break
        return {"steps": steps, "status": last}

    def generate(self, prefix: torch.Tensor, n_prefix: Sequence[int], n_blocks: int, cfg: SamplerCfg,
                 kv: KV) -> List[torch.Tensor]:
        """Prefill, then denoise and commit `n_blocks` canvases ([GUIDE] block-autoregressive)."""
        B = len(n_prefix)
        self.prefill(prefix, n_prefix, kv)
        blocks = []
        for _ in range(n_blocks):
            st = Canvas(B, self.shape.canvas, self.device)
            self.canvas_init(st, kv, cfg)
            res = self.denoise_canvas(st, kv, cfg)
            refresh = any(d["changed"] for d in res["status"])
            self.commit_block(st.tokens, kv, refresh)
            blocks.append(st.tokens.clone())
        return blocks
