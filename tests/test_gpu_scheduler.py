"""The scheduler over the decode path on the GPU (cbd_sched_create_device):
the DGR-012 concurrency sweep (8 sessions, prompt 4, 8 new tokens, levels
1/2/4/8) with a 3-layer f32 model whose KV costs the page's 1536 bytes per
token reproduces the page's table cell for cell; every session's tokens equal
the job generated alone (lockstep, one token per step) at every level; the
arena ends empty; and the oracle, fed the GPU's tokens, picks the same greedy
token at every step whose top-two margin is decisive.
"""
import json
import os

import numpy as np
import pytest

import continuous_batching_decode_step_amd as cbd
import oracle
import synth
from gpu_helpers import TOL_F32, engine_for, say, top2_gap

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "dgr012_sweep.json")) as _f:
    SWEEP = json.load(_f)
CFG = synth.ModelConfig("sched-tiny-f32", d=64, n_layers=3, n_heads=4, n_kv_heads=4, head_dim=16, ffn=172,
                        vocab=256)


def test_device_scheduler_reproduces_the_sweep():
    from continuous_batching_decode_step_amd.driver import generate_lockstep
    W = synth.make_weights(CFG)
    n, plen, new = SWEEP["sessions"], SWEEP["prompt_len"], SWEEP["new_tokens"]
    P = [synth.uniform_int(1, 1200 + j, plen, 0, CFG.vocab - 1).tolist() for j in range(n)]
    eng = engine_for(CFG, W, n, plen + new, max_batch=n)
    assert cbd.lib().cbd_arena_n_blocks(eng.arena.h) >= n
    got = {}
    for level in sorted(SWEEP["levels"], key=int):
        c = int(level)
        want = SWEEP["levels"][level]
        b = dict(weight_bytes=0, kv_budget_bytes=1 << 40, kv_bytes_per_token=1, scratch_per_session=0,
                 scratch_budget_bytes=0, max_active=c, max_queue=n, max_batch=n, max_prefill_tokens_per_tick=plen)
        s = cbd.Scheduler(b, device=(eng.model, eng.arena, eng.ws, eng.logits, eng.argmax, eng.stream))
        for j, p in enumerate(P):
            assert s.submit(j, p, new) == "QUEUED"
        s.run()
        t = s.telemetry()
        tpt = (t["prefill_tokens"] + t["decode_tokens"]) / t["ticks"]
        say("level %d: ticks %d, occupancy avg %.3f max %d, tokens/tick %.3f, peak KV %d B" % (
            c, t["ticks"], t["occupancy_avg"], t["occupancy_max"], tpt, t["kv_peak_bytes"]))
        assert t["ticks"] == want["ticks"] and t["occupancy_max"] == want["occupancy_max"]
        assert round(t["occupancy_avg"], 3) == want["occupancy_avg"] and round(tpt, 3) == want["tokens_per_tick"]
        assert t["kv_peak_bytes"] == want["kv_peak_bytes"]      # the arena's own bytes per token
        assert t["kv_bytes"] == 0 and eng.arena.used_bytes == 0 and eng.arena.live_lanes == 0
        for j in range(n):
            toks, done = s.job_tokens(j)
            assert done and len(toks) == new
            if j in got:
                assert toks == got[j], (c, j)   # no cross-session corruption at any level
            got[j] = toks
        s.close()
    # each job alone, one token per step, on a fresh engine
    ref = engine_for(CFG, W, 1, plen + new, max_batch=1)
    for j in (0, 5):
        toks, _ = generate_lockstep(ref, [P[j]], new)
        assert list(toks[0]) == got[j], j
    # the oracle, teacher-forced on the GPU's tokens
    M = oracle.Model(W)
    for j in (0, 7):
        lane = M.lane(plen + new)
        seq = P[j] + got[j][:-1]
        for i, tok in enumerate(seq):
            o = M.step(lane, int(tok))
            if i >= plen - 1:
                g = got[j][i - (plen - 1)]
                if int(np.argmax(o)) != g:
                    assert top2_gap(o) < 4 * TOL_F32 * np.max(np.abs(o)), (j, i)
