"""Full-size parity at the Mistral-7B shape in bf16, in the launch configuration
bench.py times: 64 lanes with KV lengths uniform in [128, 4096] (seed 2) and
synthetic post-rotary K/V (seed 3), one decode step over the first B lanes
for B in {1, 2, 4, 8, 16, 32, 64}.

Checked: sampled lanes' logits against the CPU oracle (teacher-forced: same
token, same cache); the same lane's logits are bit-identical at every B; the
GPU argmax equals the argmax of the GPU logits; the step writes the new K/V
at slot len_b and leaves the older slots untouched.

The bar.  The logits are compared by max relative error (||g - o||_inf /
||o||_inf).  At this depth bf16 activations turn any f32 rounding into flipped
bf16 roundings that grow through the 32 layers, so an evaluation of the same
definition with f32 accumulators (the oracle's own accumulate="f32" build,
tests/golden/bf16_7b_floor.json, written by tests/golden/make_bf16_7b_floor.py
from the oracle alone) lands 1.5-2.1% from the exact-sum oracle on these very
lanes, above 2e-2 on three of the eight.  So each lane is held to
max(2e-2, F), F the largest of those eight f32 distances (2.096%): no GPU lane
may sit further from the exact oracle than an f32 evaluation's worst lane
does; and the GPU must be at least as accurate as that evaluation on average
(mean over the lanes of its error <= mean of the f32 distances).  The K/V the
step appends in every layer is held to 2e-2, and layer 0's (one projection,
no attention) to 2^-8 (a flipped bf16 rounding of single elements at most).
Eight lanes are checked: the shortest (162 positions) and the longest (3997)
of the 64, and six others spread over the range.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BATCHES = [1, 2, 4, 8, 16, 32, 64]
# lanes 24 and 2 hold the shortest and the longest KV of the 64
SAMPLE = [0, 2, 4, 7, 14, 24, 40, 63]
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bf16_7b_floor.json")) as _f:
    FLOOR = json.load(_f)["lanes"]
LAYER0_TOL = 2.0 ** -8
# the largest and the mean distance of the f32-accumulating evaluation from the exact one over the lanes
FLOOR_MAX = max(FLOOR[str(b)]["max_rel"] for b in SAMPLE)
FLOOR_MEAN = float(np.mean([FLOOR[str(b)]["max_rel"] for b in SAMPLE]))
LOGIT_BAR = max(TOL_BF16, FLOOR_MAX)


def _floor_note(b):
    f = FLOOR.get(str(b))
    return "" if f is None else " (f32-accumulation floor %.4g)" % f["max_rel"]


@pytest.fixture(scope="module")
def setup7b(weights_7b, device_weights_7b):
    import torch
    from continuous_batching_decode_step_amd.driver import Engine
    cfg = synth.MISTRAL7B
    W = weights_7b
    lens = synth.kv_lengths(64)
    toks = synth.step_tokens(cfg, 64)
    eng = Engine(cfg, device_weights_7b, 64, int(lens.max()) + 1, max_batch=64)
    lanes = [eng.arena.lane_alloc() for _ in range(64)]
    kv = {}
    say("7B: loading KV of 64 lanes")
    for b in range(64):
        k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))
        eng.arena.kv_import(lanes[b], int(lens[b]), k, v, eng.stream)
        if b in SAMPLE:
            kv[b] = (k, v)
    torch.cuda.synchronize()
    return cfg, W, lens, toks, eng, lanes, kv


def test_mistral7b_bf16_ragged_step_matches_oracle(setup7b):
    cfg, W, lens, toks, eng, lanes, kv = setup7b
    got = {}
    for B in BATCHES:
        say("7B: step B=%d" % B)
        for b in range(B):
            eng.arena.lane_truncate(lanes[b], int(lens[b]))
        pos = lens[:B].astype(np.int32).copy()
        am, lg = eng.step_sync(lanes[:B], pos, toks[:B], want_logits=True)
        assert np.array_equal(pos, lens[:B] + 1)
        for b in range(B):
            assert int(am[b]) == int(np.argmax(lg[b]))
        for b in SAMPLE:
            if b < B:
                if b in got:  # bit-identical at every width
                    assert np.array_equal(got[b].view(np.uint32), lg[b].view(np.uint32)), (b, B)
                else:
                    got[b] = lg[b].copy()
    M = oracle.Model(W)
    errs = []
    for b in SAMPLE:
        k, v = kv[b]
        n = int(lens[b])
        lane = M.lane(n + 1)
        lane.set_kv(synth.bf16_to_f32(k), synth.bf16_to_f32(v))
        say("7B: oracle lane %d (len %d)" % (b, n))
        ref = M.step(lane, int(toks[b]))
        assert FLOOR[str(b)]["kv_len"] == n and FLOOR[str(b)]["token"] == int(toks[b])
        err = rel_err(got[b], ref)
        errs.append(err)
        say("7B: lane %d (len %d) max rel err %.4g, bar %.4g%s" % (b, n, err, LOGIT_BAR, _floor_note(b)))
        assert err <= LOGIT_BAR
        # KV: old slots untouched, new slot close to the oracle's
        gk, gv = eng.kv_export(lanes[b])
        assert gk.shape[2] == n + 1
        assert np.array_equal(gk[:, :, :n], k) and np.array_equal(gv[:, :, :n], v)
        ok, ov = lane.get_kv()
        gkn, gvn = synth.bf16_to_f32(gk[:, :, n]), synth.bf16_to_f32(gv[:, :, n])
        ek, ev = rel_err(gkn, ok[:, :, n]), rel_err(gvn, ov[:, :, n])
        ek0, ev0 = rel_err(gkn[0], ok[0, :, n]), rel_err(gvn[0], ov[0, :, n])
        say("7B: lane %d new K/V rel err %.3g / %.3g, layer 0 %.3g / %.3g" % (b, ek, ev, ek0, ev0))
        assert ek <= TOL_BF16 and ev <= TOL_BF16
        assert ek0 <= LAYER0_TOL and ev0 <= LAYER0_TOL
    say("7B: mean max rel err over the lanes %.4g (f32-accumulation mean %.4g)" % (float(np.mean(errs)), FLOOR_MEAN))
    assert float(np.mean(errs)) <= FLOOR_MEAN


WIDE_BATCHES = [128, 256, 512]
WIDE_SAMPLE = [0, 77, 127]


def test_mistral7b_wide_batches_bit_identical_to_lane_alone(device_weights_7b):
    """Above 64 lanes the projections run as 64- and 128-lane panels, in full
    or split mode, with one or two row blocks per wave (a choice per
    projection and B); one lane alone runs the split-K tiles.  All follow one
    reduction contract, so sampled lanes' logits must be bitwise equal to the
    lane stepped alone at B = 128, 256 and 512 (short KV, U[1, 48], so the
    arena stays small)."""
    import torch
    from continuous_batching_decode_step_amd.driver import Engine
    cfg = synth.MISTRAL7B
    nl = max(WIDE_BATCHES)
    lens = synth.kv_lengths(nl, lo=1, hi=48)
    toks = synth.step_tokens(cfg, nl)
    eng = Engine(cfg, device_weights_7b, nl, int(lens.max()) + 1, max_batch=nl)
    lanes = [eng.arena.lane_alloc() for _ in range(nl)]
    say("7B wide: loading KV of %d lanes" % nl)
    for b in range(nl):
        k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))
        eng.arena.kv_import(lanes[b], int(lens[b]), k, v, eng.stream)
    torch.cuda.synchronize()
    alone = {}
    for b in WIDE_SAMPLE:
        eng.arena.lane_truncate(lanes[b], int(lens[b]))
        p1 = np.array([lens[b]], np.int32)
        am1, lg1 = eng.step_sync([lanes[b]], p1, [int(toks[b])], want_logits=True)
        assert int(am1[0]) == int(np.argmax(lg1[0]))
        alone[b] = lg1[0].copy()
    for B in WIDE_BATCHES:
        say("7B wide: step B=%d" % B)
        for b in range(B):
            eng.arena.lane_truncate(lanes[b], int(lens[b]))
        pos = lens[:B].astype(np.int32).copy()
        am, lg = eng.step_sync(lanes[:B], pos, toks[:B], want_logits=True)
        assert np.array_equal(pos, lens[:B] + 1)
        assert np.array_equal(am, np.argmax(lg, axis=1))
        for b in WIDE_SAMPLE:
            assert np.array_equal(lg[b].view(np.uint32), alone[b].view(np.uint32)), (b, B)
    del eng


PREFILL_COUNTS = [512, 1, 700, 64, 65, 1000, 300, 1454]   # 4096 rows in one call
PREFILL_CHECK = [0, 1, 3, 4, 7]


def test_mistral7b_prefill_4096_rows_bit_identical_to_decode(device_weights_7b):
    """One batched prefill call of 4096 rows (eight lanes, ragged prompts from
    empty caches) at the 7B shape: the projections run as 128-lane panels over
    the rows.  Sampled lanes' last-token logits and caches must be bitwise
    equal to the same lane fed its prompt one decode step at a time."""
    import torch
    from continuous_batching_decode_step_amd.driver import Engine
    cfg = synth.MISTRAL7B
    n = len(PREFILL_COUNTS)
    R = sum(PREFILL_COUNTS)
    max_seq = max(PREFILL_COUNTS)
    prompts = [synth.uniform_int(1, 1000 + b, PREFILL_COUNTS[b], 0, cfg.vocab - 1) for b in range(n)]
    eng = Engine(cfg, device_weights_7b, n, max_seq, max_batch=R)
    lanes = [eng.arena.lane_alloc() for _ in range(n)]
    say("7B prefill: %d rows in one call" % R)
    pos = np.zeros(n, np.int32)
    am, lg = eng.prefill_sync(lanes, pos, prompts, want_logits=True)
    assert np.array_equal(pos, PREFILL_COUNTS) and np.array_equal(am, np.argmax(lg, axis=1))
    kv = {b: eng.kv_export(lanes[b]) for b in PREFILL_CHECK}
    ref = Engine(cfg, device_weights_7b, 1, max_seq, max_batch=1)
    for b in PREFILL_CHECK:
        say("7B prefill: lane %d (%d tokens) fed one step at a time" % (b, PREFILL_COUNTS[b]))
        l0 = ref.arena.lane_alloc()
        p = np.zeros(1, np.int32)
        for t in prompts[b][:-1]:
            ref.step([l0], p, [int(t)])
        _, lg1 = ref.step_sync([l0], p, [int(prompts[b][-1])], want_logits=True)
        assert np.array_equal(lg1[0].view(np.uint32), lg[b].view(np.uint32)), b
        rk, rv = ref.kv_export(l0)
        assert np.array_equal(rk, kv[b][0]) and np.array_equal(rv, kv[b][1]), b
        ref.arena.lane_evict(l0)
    del eng, ref
    torch.cuda.empty_cache()
