"""The continuous-batching scheduler (cbd_sched_*) on the host, over a mock
engine: admission budgets and their reasons, decode first then bounded
prefill, positions isolated per session, KV returned on completion,
telemetry, and the concurrency sweep of the DGR-012 page reproduced cell for
cell (tests/golden/dgr012_sweep.json).

The mock engine's next token is a hash of the lane's whole token history, so
a token fed to the wrong lane, or a position skipped or repeated, changes
every later token of that session.
"""
import json
import os

import numpy as np
import pytest

import continuous_batching_decode_step_amd as cbd

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "dgr012_sweep.json")) as _f:
    SWEEP = json.load(_f)
VOCAB = 1000


class MockEngine:
    def __init__(self, n_lanes):
        self.hist = [None] * n_lanes   # per lane: tokens fed so far (None: free)
        self.calls = []                # ("prefill" | "decode", [(lane, position), ...])

    def _next(self, lane):
        h = 1469598103934665603
        for t in self.hist[lane]:
            h = ((h ^ t) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
        return h % VOCAB

    def _feed(self, lane, pos, tok):
        assert self.hist[lane] is not None and len(self.hist[lane]) == pos, (lane, pos)
        self.hist[lane].append(int(tok))

    def prefill(self, n, lanes, positions, counts, tokens, nxt):
        k, fed = 0, []
        for i in range(n):
            for _ in range(counts[i]):
                self._feed(lanes[i], positions[i], tokens[k])
                fed.append((lanes[i], positions[i]))
                positions[i] += 1
                k += 1
            nxt[i] = self._next(lanes[i])
        self.calls.append(("prefill", fed))
        return 0

    def decode(self, B, lanes, positions, tokens, nxt):
        fed = []
        for b in range(B):
            self._feed(lanes[b], positions[b], tokens[b])
            fed.append((lanes[b], positions[b]))
            positions[b] += 1
            nxt[b] = self._next(lanes[b])
        self.calls.append(("decode", fed))
        return 0

    def lane_alloc(self, out):
        i = self.hist.index(None)
        self.hist[i] = []
        out[0] = i
        return 0

    def lane_evict(self, lane):
        self.hist[lane] = None
        return 0

    def callbacks(self):
        return {"prefill": self.prefill, "decode": self.decode, "lane_alloc": self.lane_alloc,
                "lane_evict": self.lane_evict}


def budget(**kw):
    b = dict(weight_bytes=123456, kv_budget_bytes=1 << 40, kv_bytes_per_token=1536, scratch_per_session=0,
             scratch_budget_bytes=0, max_active=8, max_queue=64, max_batch=64, max_prefill_tokens_per_tick=4)
    b.update(kw)
    return b


def prompts(n, length, seed=7):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, VOCAB, length).tolist() for _ in range(n)]


def serial_reference(prompt, n_new):
    """The same job alone: the mock engine's greedy continuation."""
    e = MockEngine(1)
    out = [0]
    e.lane_alloc(out)
    for pos, t in enumerate(prompt):
        e._feed(0, pos, t)
    toks = [e._next(0)]
    while len(toks) < n_new:
        e._feed(0, len(e.hist[0]), toks[-1])
        toks.append(e._next(0))
    return toks


@pytest.mark.parametrize("level", sorted(SWEEP["levels"], key=int))
def test_concurrency_sweep_matches_the_pages_table(level):
    c = int(level)
    want = SWEEP["levels"][level]
    eng = MockEngine(c)
    s = cbd.Scheduler(budget(max_active=c, kv_bytes_per_token=SWEEP["kv_bytes_per_token"]), eng.callbacks())
    P = prompts(SWEEP["sessions"], SWEEP["prompt_len"])
    for j, p in enumerate(P):
        assert s.submit(j, p, SWEEP["new_tokens"]) == "QUEUED"
    s.run()
    t = s.telemetry()
    assert t["ticks"] == want["ticks"]
    assert round(t["occupancy_avg"], 3) == want["occupancy_avg"]
    assert t["occupancy_max"] == want["occupancy_max"]
    assert round((t["prefill_tokens"] + t["decode_tokens"]) / t["ticks"], 3) == want["tokens_per_tick"]
    assert t["kv_peak_bytes"] == want["kv_peak_bytes"]
    # corruption-free: every session's tokens equal the job run alone; KV back to zero
    for j, p in enumerate(P):
        toks, done = s.job_tokens(j)
        assert done and toks == serial_reference(p, SWEEP["new_tokens"]), j
    assert t["kv_bytes"] == 0 and t["active"] == 0 and t["finished"] == SWEEP["sessions"]
    assert t["rejected"] == 0


def test_admission_reasons_and_backpressure():
    eng = MockEngine(2)
    # KV: a session must fit its prompt + new tokens on its own (10 positions here)
    s = cbd.Scheduler(budget(kv_budget_bytes=10 * 1536, max_active=2, max_queue=2), eng.callbacks())
    assert s.submit(1, [1, 2, 3], 8) == "REJECTED_KV_BUDGET"        # 11 positions
    assert s.submit(2, [1, 2], 8) == "QUEUED"                       # 10 positions
    assert s.submit(2, [5], 1) == "REJECTED_DUPLICATE"
    assert s.submit(3, [1], 2) == "QUEUED"
    assert s.submit(4, [1], 2) == "REJECTED_QUEUE_FULL"              # backpressure
    t = s.telemetry()
    assert (t["rejected"], t["rejected_kv"], t["rejected_duplicate"], t["rejected_queue_full"]) == (3, 1, 1, 1)
    assert t["queued"] == 2 and t["weight_bytes"] == 123456
    s.tick()                      # job 2 prefilled; job 3 waits for KV (10 + 3 > 10 positions reserved)
    t = s.telemetry()
    assert (t["active"], t["queued"]) == (1, 1)
    assert s.submit(4, [1], 2) == "QUEUED"                           # the queue has room again
    s.run()
    assert s.telemetry()["finished"] == 3 and s.telemetry()["kv_bytes"] == 0
    # scratch: the active cap is the tighter of max_active and the envelope
    s2 = cbd.Scheduler(budget(max_active=8, scratch_per_session=100, scratch_budget_bytes=350), eng.callbacks())
    assert s2.telemetry()["effective_active_cap"] == 3
    s3 = cbd.Scheduler(budget(scratch_per_session=100, scratch_budget_bytes=99), eng.callbacks())
    assert s3.submit(1, [1], 1) == "REJECTED_SCRATCH_BUDGET"
    assert s3.telemetry()["rejected_scratch"] == 1


def test_decode_first_and_prefill_does_not_starve_decode():
    eng = MockEngine(8)
    s = cbd.Scheduler(budget(max_active=8, max_prefill_tokens_per_tick=4), eng.callbacks())
    s.submit(0, [1, 2, 3, 4], 12)
    s.tick()                                          # job 0 prefilled
    for j in range(1, 5):                             # a burst of four prompts
        s.submit(j, [j, j, j, j], 4)
    before = len(eng.calls)
    for _ in range(4):
        s.tick()
    calls = eng.calls[before:]
    # each tick: decode first (job 0 decodes on every tick), then one prefill (4-token cap)
    kinds = [k for k, _ in calls]
    assert kinds == ["decode", "prefill"] * 4
    assert all(len(fed) == 4 for k, fed in calls if k == "prefill")
    # a prompt longer than the cap still progresses (one session per tick always may)
    s.submit(9, list(range(10)), 1)
    s.run()
    assert s.job_tokens(9)[1]


def test_positions_isolated_across_prompt_lengths():
    eng = MockEngine(3)
    s = cbd.Scheduler(budget(max_active=3, max_prefill_tokens_per_tick=16), eng.callbacks())
    P = [[3], [4, 5, 6], [7, 8, 9, 10, 11, 12, 13]]
    for j, p in enumerate(P):
        s.submit(j, p, 5)
    s.run()
    for j, p in enumerate(P):
        toks, done = s.job_tokens(j)
        assert done and toks == serial_reference(p, 5)
    # every lane was fed positions 0, 1, 2, ... with no gap or repeat (the mock asserts it)
    assert s.telemetry()["decode_tokens"] == 3 * 4 and s.telemetry()["prefill_tokens"] == 11


def test_run_is_bounded_and_errors_are_reported():
    eng = MockEngine(1)
    s = cbd.Scheduler(budget(max_active=1), eng.callbacks())
    s.submit(0, [1, 2], 50)
    with pytest.raises(cbd.CbdError):
        s.run(max_ticks=10)
    with pytest.raises(cbd.CbdError):
        cbd.Scheduler(budget(max_batch=0), eng.callbacks())
    with pytest.raises(cbd.CbdError):
        s.submit(5, [], 3)
    with pytest.raises(cbd.CbdError):
        s.job_tokens(77)


def test_prefill_failure_requeues_and_still_releases_finished_sessions():
    # A tick whose decode finishes a session and whose prefill then fails: the
    # finished session's lane is released all the same, the picked sessions
    # wait again at the head of the queue with their lanes returned, and the
    # next tick prefills them.
    eng = MockEngine(3)
    fail = {"n": 0}
    good_prefill = eng.prefill

    def prefill(*a):
        if fail["n"] > 0:
            fail["n"] -= 1
            return -8  # CBD_E_HIP, as a device failure would report it
        return good_prefill(*a)

    cb = dict(eng.callbacks(), prefill=prefill)
    s = cbd.Scheduler(budget(max_active=3, max_prefill_tokens_per_tick=16), cb)
    assert s.submit(0, [1, 2], 2) == "QUEUED"
    s.tick()                                   # job 0 prefilled: first token
    assert s.submit(1, [3, 4, 5], 3) == "QUEUED"
    assert s.submit(2, [6], 2) == "QUEUED"
    fail["n"] = 1
    with pytest.raises(cbd.CbdError):
        s.tick()                               # decode finishes job 0; the prefill of jobs 1, 2 fails
    t = s.telemetry()
    assert s.job_tokens(0)[1] and t["finished"] == 1 and t["active"] == 0 and t["queued"] == 2
    assert eng.hist == [None, None, None]      # job 0's lane and the failed prefill's lanes are free
    s.run()
    for j, p, n in [(0, [1, 2], 2), (1, [3, 4, 5], 3), (2, [6], 2)]:
        toks, done = s.job_tokens(j)
        assert done and toks == serial_reference(p, n), j
    assert s.telemetry()["kv_bytes"] == 0

