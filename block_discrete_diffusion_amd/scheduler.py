"""Continuous block-autoregressive serving on a fixed pool of cache slots.

The generation loop is the block-autoregressive one ([GUIDE] "Arquitetura em Detalhes": the
prompt is prefilled causally, each 256-token canvas is denoised bidirectionally and then committed
to the cache before the next canvas starts; [NEWS] second paragraph).  What this adds is the
serving side that the pages only name (denoising loops over batched requests, [GUIDE] "Deploy com
vLLM"; the low-to-medium batch regime, [NEWS] fifth paragraph and [DOCS] "Compensação com modelos
tradicionais"; the per-canvas adaptive stop, [DOCS] table, adaptive-stop row): requests have their
own prompt length, number of blocks and stopping step, so they do not move in lockstep.  Each
request owns one slot of a cache of `n_slots` slots; every device call runs on the slots that are
live right now, each with its own step counter, and a slot is handed to the next queued request
as soon as its request has committed its last block.

Host-side bookkeeping only: every computation runs in libdg's kernels through the binding.  The
one host synchronisation per denoise step is the read of the 32-byte step status of the live
requests (needed to learn which canvases stopped).

A request's random draws are keyed by its slot and positions (canvas start, Gumbel noise,
re-noise tokens), so its output depends on the slot it lands in; with COMMIT_CAUSAL its cache
rows do not depend on which other requests share a call.
"""
from __future__ import annotations

import dataclasses
from collections import deque
from typing import Callable, Deque, Dict, List, Optional, Sequence

import numpy as np
import torch

from . import dg


@dataclasses.dataclass
class Request:
    rid: int
    prompt: np.ndarray            # int32 [n_prompt]
    n_blocks: int
    slot: int = -1
    step: int = 0                 # denoise step of the current canvas
    blocks: List[torch.Tensor] = dataclasses.field(default_factory=list)  # committed canvases
    steps_per_block: List[int] = dataclasses.field(default_factory=list)
    admitted_at: int = -1         # scheduler iteration of admission
    finished_at: int = -1


class ContinuousBatcher:
    """Serve queued requests on the slots of `kv` with at most `max_active` canvases per call.

    commit: dg.COMMIT_LAST (the K/V of the last forward pass, re-run first for the canvases whose
    last sampler step changed a token), dg.COMMIT_REFRESH (always re-run) or dg.COMMIT_CAUSAL
    (re-encode the canvas causally, like the prompt).
    trace: optional callable(event, info) for tests and measurement; events "admit", "denoise",
    "sample", "commit", "finish"."""

    def __init__(self, model: "dg.Model", kv: "dg.KV", cfg: "dg.SamplerCfg", max_active: Optional[int] = None,
                 commit: int = dg.COMMIT_LAST, trace: Optional[Callable[[str, Dict], None]] = None):
        if max_active is None:
            max_active = min(kv.n_slots, model.max_batch)
        if not 1 <= max_active <= min(kv.n_slots, model.max_batch):
            raise ValueError("max_active must be in [1, min(kv.n_slots, model.max_batch)]")
        if commit not in (dg.COMMIT_LAST, dg.COMMIT_REFRESH, dg.COMMIT_CAUSAL):
            raise ValueError("commit must be COMMIT_LAST, COMMIT_REFRESH or COMMIT_CAUSAL")
        self.m, self.kv, self.cfg = model, kv, cfg
        self.max_active, self.commit_mode, self.trace = max_active, commit, trace
        C, dev = model.shape.canvas, model.device
        self.C = C
        self.state = dg.Canvas(kv.n_slots, C, dev)
        self.stats = dg.Stats(kv.n_slots, C, dev)
        self.status = torch.zeros((kv.n_slots, 8), dtype=torch.int32, device=dev)
        self._gpu = torch.device(dev).type == "cuda"
        self.status_host = torch.zeros((kv.n_slots, 8), dtype=torch.int32, pin_memory=self._gpu)
        self.free: Deque[int] = deque(range(kv.n_slots))
        self.queue: Deque[Request] = deque()
        self.active: Dict[int, Request] = {}  # slot -> request
        self.done: Dict[int, Request] = {}
        self.iteration = 0
        self.n_denoise_calls = 0
        self.n_positions = 0  # canvas positions denoised (live canvases x canvas x steps)
        self._next_id = 0

    # ------------------------------------------------------------------ queue
    def submit(self, prompt: Sequence[int], n_blocks: int) -> int:
        p = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32).reshape(-1))
        if n_blocks < 1:
            raise ValueError("n_blocks must be >= 1")
        if len(p) + n_blocks * self.C > self.kv.c.cap:
            raise ValueError(f"prompt {len(p)} + {n_blocks} blocks of {self.C} exceed the cache capacity "
                             f"{self.kv.c.cap}")
        if len(p) and (p.min() < 0 or p.max() >= self.m.shape.vocab):
            raise ValueError("prompt tokens must lie in [0, vocab)")
        r = Request(self._next_id, p, int(n_blocks))
        self._next_id += 1
        self.queue.append(r)
        return r.rid

    def idle(self) -> bool:
        return not self.queue and not self.active

    # ------------------------------------------------------------------ one iteration
    def _admit(self):
        new: List[Request] = []
        while self.queue and self.free and len(self.active) + len(new) < self.max_active:
            r = self.queue.popleft()
            r.slot = self.free.popleft()
            r.admitted_at = self.iteration
            self.kv.len[r.slot] = 0
            new.append(r)
        if not new:
            return
        slots = [r.slot for r in new]
        toks = np.concatenate([r.prompt for r in new]) if any(len(r.prompt) for r in new) else np.zeros(1, np.int32)
        try:
            dev = torch.from_numpy(toks).to(self.m.device)
            self.m.prefill(dev, [len(r.prompt) for r in new], self.kv, slots=slots)
            self.m.canvas_init(self.state, self.kv, self.cfg, slots=slots)
        except Exception:
            # put the requests back at the head of the queue and free their slots, so the
            # batcher is left as it was before this admission
            for r in reversed(new):
                self.free.appendleft(r.slot)
                r.slot, r.admitted_at = -1, -1
                self.queue.appendleft(r)
            raise
        for r in new:
            r.step = 0
            self.active[r.slot] = r
        if self.trace:
            self.trace("admit", {"slots": slots, "rids": [r.rid for r in new]})

    def _commit(self, finished: List[Request], changed: Dict[int, bool]):
        mode = self.commit_mode
        if mode == dg.COMMIT_LAST:
            # K/V of the last forward pass are exact only where the sampler's last step left the
            # canvas unchanged; the others are re-run (which replaces the forward's K/V, so the
            # exact ones go first)
            exact = [r.slot for r in finished if not changed[r.slot]]
            stale = [r.slot for r in finished if changed[r.slot]]
            groups = [(exact, dg.COMMIT_LAST), (stale, dg.COMMIT_REFRESH)]
        else:
            groups = [([r.slot for r in finished], mode)]
        for slots, m in groups:
            if slots:
                self.m.commit_block(self.state.tokens, self.kv, m, slots=slots)
                if self.trace:
                    self.trace("commit", {"slots": slots, "mode": m})
        for r in finished:
            r.blocks.append(self.state.tokens[r.slot].clone())
            r.steps_per_block.append(r.step)
        # canvases of requests with blocks left start again; finished requests free their slot
        restart = [r.slot for r in finished if len(r.blocks) < r.n_blocks]
        if restart:
            self.m.canvas_init(self.state, self.kv, self.cfg, slots=restart)
            for s in restart:
                self.active[s].step = 0
        for r in finished:
            if len(r.blocks) == r.n_blocks:
                del self.active[r.slot]
                self.free.append(r.slot)
                r.finished_at = self.iteration
                self.done[r.rid] = r
                if self.trace:
                    self.trace("finish", {"slot": r.slot, "rid": r.rid})

    def step(self):
        """Admit queued requests into free slots, run one denoise + sampler step on every live
        canvas, and commit (and restart or release) the canvases that stopped."""
        self._admit()
        if not self.active:
            return
        slots = sorted(self.active)
        steps = [self.active[s].step for s in slots]
        self.m.denoise_step(self.state.tokens, self.kv, self.cfg, steps, self.stats, slots=slots)
        if self.trace:
            self.trace("denoise", {"slots": slots, "steps": steps})
        self.m.sample_commit(self.state, self.stats, self.cfg, steps, self.kv, self.status, slots=slots)
        self.status_host.copy_(self.status, non_blocking=self._gpu)
        if self._gpu:
            torch.cuda.current_stream().synchronize()
        st = dg.status_dict(self.status_host)
        if self.trace:
            self.trace("sample", {"slots": slots, "steps": steps, "status": {s: st[s] for s in slots}})
        self.n_denoise_calls += 1
        self.n_positions += len(slots) * self.C
        finished, changed = [], {}
        for s in slots:
            r = self.active[s]
            r.step += 1
            if st[s]["stop"]:
                finished.append(r)
                changed[s] = bool(st[s]["changed"])
        if finished:
            self._commit(finished, changed)
        self.iteration += 1

    def run(self, max_iterations: int = 1 << 30) -> Dict[int, Request]:
        """Step until every submitted request has committed all its blocks."""
        while not self.idle():
            if self.iteration >= max_iterations:
                raise RuntimeError("ContinuousBatcher.run: iteration limit reached")
            self.step()
        return self.done
