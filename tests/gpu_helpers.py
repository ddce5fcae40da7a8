"""Helpers for the GPU parity tests: engine setup from seeded weights, teacher-
forced oracle comparison, and the comparison metrics with their tolerances.

Metrics (per lane and step): max relative error = ||g - o||_inf / ||o||_inf
over the vocab; the same norm for KV.  Greedy tokens must agree at every step
where the oracle's top-1 / top-2 gap is at least 4 x tolerance x ||o||_inf;
closer steps are near-ties, counted and reported, and the comparison stays
teacher-forced (the oracle is fed the tokens the GPU consumed) so one near-tie
cannot cascade.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

import oracle
import synth

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def top2_gap(o) -> float:
    s = np.sort(np.asarray(o, np.float64))
    return float(s[-1] - s[-2])


def engine_for(cfg, W, n_lanes, max_seq, max_batch=None, pack=None):
    import continuous_batching_decode_step_amd as cbd
    from continuous_batching_decode_step_amd.driver import Engine
    dw = cbd.upload_weights(W, pack=pack)
    return Engine(cfg, dw, n_lanes, max_seq, max_batch)


@dataclass
class LaneReport:
    max_rel: float = 0.0
    mismatches: int = 0   # decisive steps whose argmax differs
    near_ties: int = 0
    steps: int = 0
    cos: List[float] = field(default_factory=list)
    top1_agree: int = 0
    gen_steps: int = 0
    first_token_match: bool = True
    first_token_decisive: bool = True


def compare_lane_teacher_forced(M: "oracle.Model", prompt, gen, gpu_logits, tol, max_seq=None,
                                decisive_factor=4.0) -> LaneReport:
    """Feed the oracle the tokens the GPU lane consumed (prompt, then its own generated
    tokens but the last) and compare every step's logits and greedy choice.  gpu_logits
    may cover only the job's first steps; those are compared."""
    seq = list(prompt) + list(gen[:-1])
    assert 0 < len(gpu_logits) <= len(seq)
    seq = seq[:len(gpu_logits)]
    lane = M.lane(max_seq or len(seq))
    rep = LaneReport()
    for i, tok in enumerate(seq):
        o = M.step(lane, int(tok))
        g = gpu_logits[i]
        rep.steps += 1
        rep.max_rel = max(rep.max_rel, rel_err(g, o))
        go, oo = np.asarray(g, np.float64), np.asarray(o, np.float64)
        rep.cos.append(float(go @ oo / (np.linalg.norm(go) * np.linalg.norm(oo))))
        if i >= len(prompt) - 1:  # a generation step
            rep.gen_steps += 1
            oa = int(np.argmax(o))
            ga = int(gen[i - (len(prompt) - 1)])
            decisive = top2_gap(o) >= decisive_factor * tol * np.max(np.abs(oo))
            if ga == oa:
                rep.top1_agree += 1
            elif decisive:
                rep.mismatches += 1
            else:
                rep.near_ties += 1
            if i == len(prompt) - 1:
                rep.first_token_match = ga == oa
                rep.first_token_decisive = bool(decisive)
    return rep
