"""Host-side drivers over the C-ABI: an engine that owns the device buffers of
one model, lockstep greedy generation, and the continuous-batching decode loop.

The decode loop follows "Fat-station continuous batching" (section
"Components", item 3): each step first fills free lanes with pending jobs
(lane cleared, position 0), gathers one token per live lane — the next prompt
token while the prompt lasts, else the lane's last generated token — runs one
batched decode step over the live lanes, then folds per lane: a lane that has
consumed its whole prompt takes the greedy argmax as its next generated token,
and a lane whose job has all its tokens retires and frees its lane for the
next job.  There is no stop token; a job ends after max_new_tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import Arena, Model, arena_block_bytes, arena_bytes


class Engine:
    """Model + arena + workspace + output buffers on one device and stream."""

    def __init__(self, cfg, dev_weights, n_lanes: int, max_seq: int, max_batch: Optional[int] = None,
                 device: str = "cuda", stream=None, kv_blocks: Optional[int] = None):
        """kv_blocks: size of the KV block pool (64 positions of one lane per
        block); by default every lane can reach max_seq at once."""
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = device
        self.max_batch = max_batch or n_lanes
        self.model = Model(cfg, dev_weights)
        nbytes = (arena_bytes(cfg, n_lanes, max_seq) if kv_blocks is None
                  else int(kv_blocks) * arena_block_bytes(cfg))
        self.arena_mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.arena = Arena(self.model, n_lanes, max_seq, self.arena_mem)
        self.ws_bytes = self.model.workspace_bytes(self.max_batch, max_seq)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.logits = torch.empty((self.max_batch, cfg.vocab), dtype=torch.float32, device=device)
        self.argmax = torch.empty(self.max_batch, dtype=torch.int32, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)

    def step(self, lanes: Sequence[int], positions: np.ndarray, tokens) -> None:
        """One decode step; positions (np.int32) advance in place.  Asynchronous."""
        self.model.decode_step_batch(self.arena, lanes, positions, tokens, self.logits, self.argmax, self.ws,
                                     self.ws_bytes, self.stream)

    def step_sync(self, lanes, positions, tokens, want_logits: bool = False):
        self.step(lanes, positions, tokens)
        B = len(lanes)
        am = self.argmax[:B].cpu().numpy()
        lg = self.logits[:B].cpu().numpy() if want_logits else None
        return am, lg

    def prefill_sync(self, lanes, positions, prompts, want_logits: bool = False):
        """Feed each lane its whole chunk of tokens in one batched prefill call; returns the argmax (and
        logits) of each lane's last token.  positions (np.int32) advance in place by the chunk lengths."""
        counts = [len(p) for p in prompts]
        toks = [int(t) for p in prompts for t in p]
        self.model.prefill_batch(self.arena, lanes, positions, counts, toks, self.logits, self.argmax, self.ws,
                                 self.ws_bytes, self.stream)
        n = len(lanes)
        am = self.argmax[:n].cpu().numpy()
        lg = self.logits[:n].cpu().numpy() if want_logits else None
        return am, lg

    def kv_export(self, lane: int):
        c = self.cfg
        n = self.arena.lane_length(lane)
        dt = np.uint16 if c.wtype == 1 else np.float32
        shape = (c.n_layers, c.n_kv_heads, n, c.head_dim)
        k = np.empty(shape, dtype=dt)
        v = np.empty(shape, dtype=dt)
        self.arena.kv_export(lane, k, v, self.stream)
        return k, v


def generate_lockstep(eng: Engine, prompts: Sequence[Sequence[int]], n_new, want_logits=False):
    """Greedy generation of B jobs in lockstep, one batched step over the lanes still live.

    want_logits: False, True (every step of every job), or a predicate
    keep(job, step) selecting the steps whose logits are copied back (the step
    index counts the job's own steps from 0).  Returns (tokens per job, logits
    per job per step or None; unselected steps hold None)."""
    B = len(prompts)
    n_new = [n_new] * B if np.isscalar(n_new) else list(n_new)
    keep = (lambda b, i: True) if want_logits is True else (want_logits or None)
    lanes = [eng.arena.lane_alloc() for _ in range(B)]
    pos = np.zeros(B, np.int32)
    feed = [0] * B
    last = [0] * B
    gen: List[List[int]] = [[] for _ in range(B)]
    logs: List[list] = [[] for _ in range(B)]
    while True:
        live = [b for b in range(B) if len(gen[b]) < n_new[b]]
        if not live:
            break
        toks = [int(prompts[b][feed[b]]) if feed[b] < len(prompts[b]) else last[b] for b in live]
        p = pos[live].copy()
        eng.step([lanes[b] for b in live], p, toks)
        am = eng.argmax[:len(live)].cpu().numpy()
        rows = [i for i, b in enumerate(live) if keep is not None and keep(b, feed[b])]
        lg = eng.logits[rows].cpu().numpy() if rows else None
        at = {i: j for j, i in enumerate(rows)}
        pos[live] = p
        for i, b in enumerate(live):
            if keep is not None:
                logs[b].append(lg[at[i]] if i in at else None)
            feed[b] += 1
            if feed[b] >= len(prompts[b]):
                last[b] = int(am[i])
                gen[b].append(last[b])
    for l in lanes:
        eng.arena.lane_evict(l)
    return gen, (logs if keep is not None else None)


@dataclass
class TraceStats:
    steps: int = 0           # decode steps issued
    idle_steps: int = 0      # steps with no live lane (clock advanced only)
    lane_steps: int = 0      # sum of live lanes over steps
    generated: int = 0       # generated tokens
    occupancy: List[int] = field(default_factory=list)
    positions: List[np.ndarray] = field(default_factory=list)  # per step, if recorded: positions before it
    logits: Dict[int, List[np.ndarray]] = field(default_factory=dict)  # job id -> logits of its kept steps
    kv: Dict[int, tuple] = field(default_factory=dict)  # job id -> (K, V) of its lane as it retired


def run_trace(eng: Engine, jobs, n_lanes: int, max_steps: int = 10 ** 7, record_positions: bool = False,
              keep_logits: Optional[Dict[int, int]] = None):
    """Continuous batching of `jobs` (arrival_step, prompt, max_new_tokens) over n_lanes lanes.

    FIFO admission at the start of each step into the lowest free lane.  Returns
    ({job_id: generated tokens}, TraceStats); with record_positions the stats keep
    every step's lane positions (before the step).  keep_logits {job_id: n}: the
    stats keep the logits of that job's first n steps, as taken inside the
    batched steps of the trace (st.logits[job_id], one row per step), and the
    job's whole KV cache as it retires (st.kv[job_id] = (K, V))."""
    pending = sorted(jobs, key=lambda j: (j.arrival_step, j.job_id))
    qi = 0
    lane_job: Dict[int, object] = {}
    feed: Dict[int, int] = {}
    last: Dict[int, int] = {}
    out: Dict[int, List[int]] = {}
    pos: Dict[int, int] = {}
    free = list(range(n_lanes))
    lane_ids: Dict[int, int] = {}
    st = TraceStats()
    clock = 0
    while (qi < len(pending) or lane_job) and clock < max_steps:
        # fill(): admit arrived jobs into free lanes, clearing them
        while qi < len(pending) and pending[qi].arrival_step <= clock and free:
            slot = free.pop(0)
            job = pending[qi]
            qi += 1
            if slot not in lane_ids:
                lane_ids[slot] = eng.arena.lane_alloc()
            else:
                eng.arena.lane_clear(lane_ids[slot])
            lane_job[slot], feed[slot], pos[slot] = job, 0, 0
            out[job.job_id] = []
        live = sorted(lane_job)
        if not live:
            st.idle_steps += 1
            clock += 1
            continue
        toks = [int(lane_job[s].prompt[feed[s]]) if feed[s] < len(lane_job[s].prompt) else last[s] for s in live]
        p = np.array([pos[s] for s in live], np.int32)
        if record_positions:
            st.positions.append(p.copy())
        am, _ = eng.step_sync([lane_ids[s] for s in live], p, toks)
        if keep_logits:
            rows = [i for i, s in enumerate(live)
                    if feed[s] < keep_logits.get(lane_job[s].job_id, 0)]
            if rows:
                lg = eng.logits[rows].cpu().numpy()
                for j, i in enumerate(rows):
                    st.logits.setdefault(lane_job[live[i]].job_id, []).append(lg[j])
        st.steps += 1
        st.lane_steps += len(live)
        st.occupancy.append(len(live))
        for i, s in enumerate(live):
            pos[s] = int(p[i])
            feed[s] += 1
            job = lane_job[s]
            if feed[s] >= len(job.prompt):
                last[s] = int(am[i])
                out[job.job_id].append(last[s])
                st.generated += 1
                if len(out[job.job_id]) >= job.max_new_tokens:
                    if keep_logits and job.job_id in keep_logits:
                        st.kv[job.job_id] = eng.kv_export(lane_ids[s])
                    del lane_job[s]
                    free.append(s)
                    free.sort()
        clock += 1
    for s, lid in lane_ids.items():
        eng.arena.lane_evict(lid)
    return out, st


def run_sched_trace(eng: Engine, jobs, n_lanes: int, prefill_tokens_per_tick: int, max_ticks: int = 10 ** 7):
    """The same jobs through the continuous-batching scheduler over the decode path (cbd_sched): each
    job is submitted once the tick count reaches its arrival step; ticks decode first, then prefill
    whole prompts (up to prefill_tokens_per_tick prompt tokens per tick, one prompt always) into the
    lanes that were free at the start of the tick.  The engine's workspace must hold the larger of
    n_lanes and prefill_tokens_per_tick rows (and the longest prompt).  Returns ({job_id: generated
    tokens}, scheduler telemetry, idle ticks)."""
    from . import Scheduler
    b = dict(weight_bytes=0, kv_budget_bytes=1 << 62, kv_bytes_per_token=1, scratch_per_session=0,
             scratch_budget_bytes=0, max_active=n_lanes, max_queue=max(1, len(jobs)), max_batch=n_lanes,
             max_prefill_tokens_per_tick=prefill_tokens_per_tick)
    s = Scheduler(b, device=(eng.model, eng.arena, eng.ws, eng.logits, eng.argmax, eng.stream))
    pending = sorted(jobs, key=lambda j: (j.arrival_step, j.job_id))
    qi, tick, idle = 0, 0, 0
    while tick < max_ticks:
        while qi < len(pending) and pending[qi].arrival_step <= tick:
            job = pending[qi]
            assert s.submit(job.job_id, job.prompt, job.max_new_tokens) == "QUEUED"
            qi += 1
        if not s.tick():
            if qi >= len(pending):
                break
            idle += 1
        tick += 1
    out = {j.job_id: s.job_tokens(j.job_id)[0] for j in jobs}
    tel = s.telemetry()
    s.close()
    return out, tel, idle
