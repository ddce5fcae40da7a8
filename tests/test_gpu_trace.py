"""Continuous batching at the Mistral-7B shape in bf16: 8 lanes, 64 seeded jobs
with Poisson arrivals (mean gap 4 steps), prompts of 32-1024 uniform tokens
fed one token per step, 16-256 new tokens per job (seed 4).

The decode loop is the one of "Fat-station continuous batching" (section
"Components", item 3): free lanes are filled first-come first-served, a lane
is cleared and reused when its job retires, and every step is one batched
decode step over the live lanes at mixed positions.  Gate: every job's greedy
tokens are identical to the same job run alone on a fresh lane (one-lane
steps, "Parity (CPU, before any deploy)" on the same page asks for exactly
this per-job equality).  Also checked: the arena's usage returns to zero, the
trace used every lane, and lanes were reused.

Against the oracle: two jobs' logits as taken inside the trace's batched
steps (other lanes live at other positions), teacher-forced (the oracle is fed
the tokens the GPU lane consumed): job 2 over all of its 66 steps (47-token
prompt, 20 new tokens, so its last step too) and job 16 over its first 64
steps (a 35-token prompt, then 29 steps that feed back generated tokens).
Bar: 2e-2 max relative logit error at every step (bf16), and the greedy
token equal to the oracle's at every decisive generation step.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, compare_lane_teacher_forced, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_LANES = 8


QUARTERS = 4  # the serial runs are checked in four tests, so progress shows between them
ORACLE_JOBS = {2: 10 ** 6, 16: 64}  # job id -> steps checked against the oracle (all of job 2)


@pytest.fixture(scope="module")
def trace_run(device_weights_7b):
    from continuous_batching_decode_step_amd.driver import Engine, run_trace
    cfg = synth.MISTRAL7B
    jobs = synth.make_trace(cfg)
    max_seq = max(len(j.prompt) + j.max_new_tokens for j in jobs)
    eng = Engine(cfg, device_weights_7b, N_LANES, max_seq, max_batch=N_LANES)
    say("trace: %d jobs, %d lane-steps" % (len(jobs), sum(len(j.prompt) + j.max_new_tokens - 1 for j in jobs)))
    out, st = run_trace(eng, jobs, N_LANES, keep_logits=ORACLE_JOBS)
    say("trace: %d steps (%d idle), %d lane-steps, mean occupancy %.2f" % (
        st.steps, st.idle_steps, st.lane_steps, np.mean(st.occupancy)))
    yield eng, jobs, out, st
    del eng


def test_trace_runs_every_job_and_frees_the_arena(trace_run):
    eng, jobs, out, st = trace_run
    assert st.lane_steps == sum(len(j.prompt) + j.max_new_tokens - 1 for j in jobs)
    assert max(st.occupancy) == N_LANES
    assert eng.arena.used_bytes == 0 and eng.arena.live_lanes == 0
    for j in jobs:
        assert len(out[j.job_id]) == j.max_new_tokens


@pytest.mark.parametrize("quarter", range(QUARTERS))
def test_trace_jobs_equal_serial_runs(trace_run, quarter):
    from continuous_batching_decode_step_amd.driver import generate_lockstep
    eng, jobs, out, _ = trace_run
    for j in jobs[quarter::QUARTERS]:
        gen, _ = generate_lockstep(eng, [j.prompt], j.max_new_tokens)
        same = gen[0] == out[j.job_id]
        if j.job_id % 8 == quarter or not same:
            say("trace: job %d (prompt %d, %d new) serial %s" % (
                j.job_id, len(j.prompt), j.max_new_tokens, "identical" if same else "DIFFERS"))
        assert same, j.job_id


def test_scheduler_with_prefill_gives_the_trace_tokens(trace_run, device_weights_7b):
    """The same jobs through the continuous-batching scheduler (cbd_sched over the decode path), whose
    ticks prefill whole prompts in batched calls: every job's tokens equal the one-token-per-step
    trace's, and the arena ends empty."""
    from continuous_batching_decode_step_amd.driver import Engine, run_sched_trace
    _, jobs, out, st = trace_run
    cfg = synth.MISTRAL7B
    max_seq = max(len(j.prompt) + j.max_new_tokens for j in jobs)
    rows = max(len(j.prompt) for j in jobs)
    eng = Engine(cfg, device_weights_7b, N_LANES, max_seq, max_batch=max(rows, 1024))
    got, tel, idle = run_sched_trace(eng, jobs, N_LANES, 1024)
    say("scheduler trace: %d ticks (%d idle, %d decoding), mean decode occupancy %.2f, against %d steps" % (
        tel["ticks"], idle, tel["decode_ticks"], tel["occupancy_avg"], st.steps))
    for j in jobs:
        assert got[j.job_id] == out[j.job_id], j.job_id
    assert tel["finished"] == len(jobs) and tel["kv_bytes"] == 0
    assert eng.arena.used_bytes == 0 and eng.arena.live_lanes == 0
    del eng


@pytest.mark.parametrize("job_id", sorted(ORACLE_JOBS))
def test_trace_job_teacher_forced_against_oracle(trace_run, weights_7b, job_id):
    eng, jobs, out, st = trace_run
    job = next(j for j in jobs if j.job_id == job_id)
    n_steps = len(job.prompt) + job.max_new_tokens - 1
    lg = st.logits[job_id]
    assert len(lg) == min(n_steps, ORACLE_JOBS[job_id])
    say("trace oracle: job %d (prompt %d, %d new), %d of its %d steps" % (
        job_id, len(job.prompt), job.max_new_tokens, len(lg), n_steps))
    M = oracle.Model(weights_7b)
    rep = compare_lane_teacher_forced(M, job.prompt, out[job_id], lg, TOL_BF16, max_seq=n_steps)
    say("trace oracle: job %d max rel err %.4g over %d steps, %d generation steps: %d agree, %d near-ties, "
        "%d decisive mismatches" % (job_id, rep.max_rel, rep.steps, rep.gen_steps, rep.top1_agree,
                                    rep.near_ties, rep.mismatches))
    assert rep.steps == len(lg)
    assert rep.max_rel <= TOL_BF16
    assert rep.mismatches == 0
