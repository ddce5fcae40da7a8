"""Full-size parity at the Mistral-7B shape in bf16, in the launch configuration
bench.py times: 64 lanes with KV lengths uniform in [128, 4096] (seed 2) and
synthetic post-rotary K/V (seed 3), one decode step over the first B lanes
for B in {1, 2, 4, 8, 16, 32, 64}.

Checked: sampled lanes' logits against the CPU oracle (teacher-forced: same
token, same cache) within 2e-2 max relative error; the same lane's logits are
bit-identical at every B; the GPU argmax equals the argmax of the GPU logits;
the step writes the new K/V at slot len_b (within 2e-2 of the oracle's) and
leaves the older slots untouched.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BATCHES = [1, 2, 4, 8, 16, 32, 64]
SAMPLE = [0, 7, 63]


@pytest.fixture(scope="module")
def setup7b():
    import torch
    import continuous_batching_decode_step_amd as cbd
    from continuous_batching_decode_step_amd.driver import Engine
    cfg = synth.MISTRAL7B
    say("7B: generating weights")
    W = synth.make_weights(cfg)
    lens = synth.kv_lengths(64)
    toks = synth.step_tokens(cfg, 64)
    eng = Engine(cfg, cbd.upload_weights(W), 64, int(lens.max()) + 1, max_batch=64)
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
    for b in SAMPLE:
        k, v = kv[b]
        n = int(lens[b])
        lane = M.lane(n + 1)
        lane.set_kv(synth.bf16_to_f32(k), synth.bf16_to_f32(v))
        say("7B: oracle lane %d (len %d)" % (b, n))
        ref = M.step(lane, int(toks[b]))
        err = rel_err(got[b], ref)
        say("7B: lane %d max rel err %.3g" % (b, err))
        assert err <= TOL_BF16
        # KV: old slots untouched, new slot close to the oracle's
        gk, gv = eng.kv_export(lanes[b])
        assert gk.shape[2] == n + 1
        assert np.array_equal(gk[:, :, :n], k) and np.array_equal(gv[:, :, :n], v)
        ok, ov = lane.get_kv()
        assert rel_err(synth.bf16_to_f32(gk[:, :, n]), ok[:, :, n]) <= TOL_BF16
        assert rel_err(synth.bf16_to_f32(gv[:, :, n]), ov[:, :, n]) <= TOL_BF16
