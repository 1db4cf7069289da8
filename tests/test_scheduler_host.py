"""Host logic of the continuous batcher, on the CPU: a stand-in model records the calls and
reports stops on a fixed rule, and the tests check admission, per-request step counters, the
commit grouping, slot reuse and the cache lengths.  No kernel runs here."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import dg, synth
from block_discrete_diffusion_amd.scheduler import ContinuousBatcher

C = 256
STATUS = {k: i for i, k in enumerate(dg.STATUS_FIELDS)}


class FakeModel:
    """Records every call; a canvas stops after 1 + (len // 7) % 4 steps (len = the request's
    committed length when the canvas started) and reports `changed` on odd final steps."""

    def __init__(self, shape, max_batch):
        self.shape, self.max_batch, self.device = shape, max_batch, "cpu"
        self.calls = []
        self.len_at_start = {}

    def prefill(self, tokens, n_new, kv, slots=None):
        assert tokens.dtype == torch.int32 and tokens.numel() >= sum(n_new)
        self.calls.append(("prefill", list(slots), list(n_new), tokens.clone(), [kv.len[s] for s in slots]))
        for s, n in zip(slots, n_new):
            assert kv.len[s] + n <= kv.c.cap
            kv.len[s] += n

    def canvas_init(self, state, kv, cfg, slots=None):
        self.calls.append(("canvas_init", list(slots)))
        for s in slots:
            self.len_at_start[s] = kv.len[s]
            state.tokens[s].fill_(kv.len[s])

    def denoise_step(self, canvas, kv, cfg, step, out, slots=None):
        assert len(slots) <= self.max_batch and len(set(slots)) == len(slots)
        self.calls.append(("denoise", list(slots), list(step)))

    def sample_commit(self, state, stats, cfg, step, kv, status, slots=None):
        self.calls.append(("sample", list(slots), list(step)))
        status.zero_()
        for s, k in zip(slots, step):
            last = 1 + (self.len_at_start[s] // 7) % 4
            if k + 1 >= last:
                status[s, STATUS["stop"]] = 1
                status[s, STATUS["changed"]] = k % 2

    def commit_block(self, canvas, kv, refresh, slots=None):
        self.calls.append(("commit", list(slots), int(refresh)))
        for s in slots:
            assert kv.len[s] + C <= kv.c.cap
            kv.len[s] += C


def _serve(requests, n_slots=3, max_active=2, commit=dg.COMMIT_LAST, cap=2000):
    fm = FakeModel(synth.TINY, max_batch=4)
    kv = dg.KV(synth.TINY, n_slots, cap, device="cpu", fill=None)
    events = []
    b = ContinuousBatcher(fm, kv, dg.sampler_cfg(seed=1), max_active=max_active, commit=commit,
                          trace=lambda e, i: events.append((e, i)))
    rids = [b.submit(p, n) for p, n in requests]
    done = b.run(max_iterations=10_000)
    return fm, kv, b, rids, done, events


REQS = [(np.arange(40) % 1024, 2), (np.arange(173) % 1024, 1), ([], 2), (np.arange(260) % 1024, 1),
        (np.arange(90) % 1024, 3)]


def test_every_request_gets_its_blocks_and_lengths():
    fm, kv, b, rids, done, events = _serve(REQS)
    assert sorted(done) == rids
    for rid, (p, n) in zip(rids, REQS):
        r = done[rid]
        assert len(r.blocks) == n and len(r.steps_per_block) == n
        assert all(t.shape == (C,) for t in r.blocks)
    fin = [i for e, i in events if e == "finish"]
    assert len(fin) == len(REQS)
    assert b.idle() and not b.active and sorted(b.free) == [0, 1, 2]


def test_live_canvases_never_exceed_max_active_and_slots_are_reused():
    fm, kv, b, rids, done, events = _serve(REQS, n_slots=3, max_active=2)
    den = [c for c in fm.calls if c[0] == "denoise"]
    assert den and all(1 <= len(c[1]) <= 2 for c in den)
    slots_used = {done[r].slot for r in rids}
    assert slots_used <= {0, 1, 2} and len(REQS) > 3  # some slot served two requests
    # requests are admitted first in, first out
    assert [done[r].admitted_at for r in rids] == sorted(done[r].admitted_at for r in rids)


def test_prefill_resets_the_slot_and_carries_each_prompt():
    fm, kv, b, rids, done, events = _serve(REQS)
    pre = [c for c in fm.calls if c[0] == "prefill"]
    seen = []
    for _, slots, n_new, toks, len_before in pre:
        assert len_before == [0] * len(slots)
        ofs = 0
        for s, n in zip(slots, n_new):
            seen.append((s, n, toks[ofs:ofs + n].numpy().tolist()))
            ofs += n
    assert len(seen) == len(REQS)  # in admission order, which is submission order
    for (s, n, toks), (rid, (p, _)) in zip(seen, zip(rids, REQS)):
        assert s == done[rid].slot and n == len(p) and toks == list(np.asarray(p, np.int32))


def test_steps_count_from_each_canvas_start():
    fm, kv, b, rids, done, events = _serve(REQS)
    step_of = {}
    for c in fm.calls:
        if c[0] == "canvas_init":
            for s in c[1]:
                step_of[s] = 0
        elif c[0] == "denoise":
            assert c[2] == [step_of[s] for s in c[1]]
        elif c[0] == "sample":
            for s in c[1]:
                step_of[s] += 1


def test_commit_groups_follow_the_last_step():
    """Canvases that stopped unchanged commit the last forward pass's K/V (first), the others
    re-run it; nothing else is committed."""
    fm, kv, b, rids, done, events = _serve(REQS)
    calls = fm.calls
    n_commits = 0
    for i, c in enumerate(calls):
        if c[0] != "sample":
            continue
        stopped = [(s, k) for s, k in zip(c[1], c[2]) if k + 1 >= 1 + (_len_at_start(calls, i, s) // 7) % 4]
        exact = [s for s, k in stopped if k % 2 == 0]
        stale = [s for s, k in stopped if k % 2 == 1]
        j, commits = i + 1, []
        while j < len(calls) and calls[j][0] == "commit":
            commits.append((calls[j][1], calls[j][2]))
            j += 1
        want = ([(exact, dg.COMMIT_LAST)] if exact else []) + ([(stale, dg.COMMIT_REFRESH)] if stale else [])
        assert commits == want, (i, commits, want)
        n_commits += sum(len(x) for x, _ in commits)
    assert n_commits == sum(n for _, n in REQS)


def _len_at_start(calls, i, s):
    """The committed length of slot s when its current canvas started (before call i)."""
    n = None
    lens = {}
    for c in calls[:i]:
        if c[0] == "prefill":
            for x, k in zip(c[1], c[2]):
                lens[x] = k
        elif c[0] == "commit":
            for x in c[1]:
                lens[x] += C
        elif c[0] == "canvas_init" and s in c[1]:
            n = lens[s]
    return n


def test_commit_modes_pass_through():
    for mode in (dg.COMMIT_REFRESH, dg.COMMIT_CAUSAL):
        fm, kv, b, rids, done, events = _serve(REQS, commit=mode)
        assert {c[2] for c in fm.calls if c[0] == "commit"} == {mode}


def test_final_lengths_of_each_slot():
    fm, kv, b, rids, done, events = _serve(REQS, n_slots=5, max_active=4)
    for rid, (p, n) in zip(rids, REQS):
        assert kv.len[done[rid].slot] == len(p) + n * C  # each slot served one request


def test_rejects_bad_requests_and_settings():
    fm = FakeModel(synth.TINY, max_batch=2)
    kv = dg.KV(synth.TINY, 2, 600, device="cpu", fill=None)
    with pytest.raises(ValueError):
        ContinuousBatcher(fm, kv, dg.sampler_cfg(), max_active=3)
    with pytest.raises(ValueError):
        ContinuousBatcher(fm, kv, dg.sampler_cfg(), commit=7)
    b = ContinuousBatcher(fm, kv, dg.sampler_cfg())
    with pytest.raises(ValueError):
        b.submit(np.zeros(100, np.int32), 2)  # 100 + 512 > 600
    with pytest.raises(ValueError):
        b.submit([5, 1024], 1)  # token outside the vocab
    with pytest.raises(ValueError):
        b.submit([1, 2], 0)
    assert b.idle()


def test_failed_admission_leaves_queue_and_slots_unchanged():
    class Failing(FakeModel):
        def prefill(self, tokens, n_new, kv, slots=None):
            raise RuntimeError("device error")

    fm = Failing(synth.TINY, max_batch=4)
    kv = dg.KV(synth.TINY, 3, 2000, device="cpu", fill=None)
    b = ContinuousBatcher(fm, kv, dg.sampler_cfg(seed=1), max_active=2)
    rids = [b.submit(p, n) for p, n in REQS]
    with pytest.raises(RuntimeError):
        b.step()
    assert [r.rid for r in b.queue] == rids and sorted(b.free) == [0, 1, 2] and not b.active
    assert all(r.slot == -1 for r in b.queue)
