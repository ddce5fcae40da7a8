"""Ragged attention at long contexts on shapes that take the matrix-core
kernel (bf16 KV, head_dim 64 and 128, eight KV heads), two layers deep so the
oracle comparison is sharp: 64 lanes with KV lengths uniform in [128, 4000]
(seed 2) of synthetic post-rotary K/V (seed 3), one decode step.  The
head_dim-64 shapes take every query-head group size up to eight (2, 5, 6, 7).

At this size a wave takes several 64-key chunks of a lane, while a lane
stepped alone gets one chunk per wave: the lane's logits must be bitwise the
same either way (chunk results never depend on the grouping, "Correctness —
proven, not asserted" on "MODEL-BATCHING-RESULTS — multi-user batched decode,
measured").  Sampled lanes match the oracle within the bf16 bar, and the step
writes the new K/V at slot len_b.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, engine_for, rel_err, say

pytestmark = pytest.mark.gpu

SHAPES = [
    synth.ModelConfig("attn-hd64-bf16", d=1024, n_layers=2, n_heads=16, n_kv_heads=8, head_dim=64, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
    synth.ModelConfig("attn-hd128-bf16", d=4096, n_layers=2, n_heads=32, n_kv_heads=8, head_dim=128, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
    # 5, 6 and 7 query heads per KV head: the head_dim-64 kernels' two-column query parts
    synth.ModelConfig("attn-hd64-g5-bf16", d=1280, n_layers=2, n_heads=20, n_kv_heads=4, head_dim=64, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
    synth.ModelConfig("attn-hd64-g6-bf16", d=1536, n_layers=2, n_heads=24, n_kv_heads=4, head_dim=64, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
    synth.ModelConfig("attn-hd64-g7-bf16", d=1792, n_layers=2, n_heads=28, n_kv_heads=4, head_dim=64, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
]
N_LANES = 64
SAMPLE = [0, 31, 63]


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_long_ragged_attention_grouped_chunks(cfg):
    say("case: %s, %d lanes, KV U[128, 4000]" % (cfg.name, N_LANES))
    W = synth.make_weights(cfg)
    lens = synth.kv_lengths(N_LANES, hi=4000)
    toks = synth.step_tokens(cfg, N_LANES)
    eng = engine_for(cfg, W, N_LANES, int(lens.max()) + 1)
    lanes = [eng.arena.lane_alloc() for _ in range(N_LANES)]
    kv = {}
    for b in range(N_LANES):
        k, v = synth.lane_kv_bf16(cfg, b, int(lens[b]))
        eng.arena.kv_import(lanes[b], int(lens[b]), k, v, eng.stream)
        if b in SAMPLE:
            kv[b] = (k, v)
    pos = lens.astype(np.int32).copy()
    am, lg = eng.step_sync(lanes, pos, toks, want_logits=True)
    assert np.array_equal(pos, lens + 1)
    M = oracle.Model(W)
    for b in SAMPLE:
        k, v = kv[b]
        n = int(lens[b])
        gk, gv = eng.kv_export(lanes[b])
        assert np.array_equal(gk[:, :, :n], k) and np.array_equal(gv[:, :, :n], v)
        # the same lane alone (one chunk per wave): same bits
        eng.arena.lane_truncate(lanes[b], n)
        p1 = np.array([n], np.int32)
        am1, lg1 = eng.step_sync([lanes[b]], p1, [int(toks[b])], want_logits=True)
        assert np.array_equal(lg1[0].view(np.uint32), lg[b].view(np.uint32)), b
        assert int(am1[0]) == int(am[b]) == int(np.argmax(lg[b]))
        lane = M.lane(n + 1)
        lane.set_kv(synth.bf16_to_f32(k), synth.bf16_to_f32(v))
        ref = M.step(lane, int(toks[b]))
        err = rel_err(lg[b], ref)
        ok, ov = lane.get_kv()
        ek = rel_err(synth.bf16_to_f32(gk[:, :, n]), ok[:, :, n])
        ev = rel_err(synth.bf16_to_f32(gv[:, :, n]), ov[:, :, n])
        say("  lane %d (len %d): logits max rel %.3g, new K/V %.3g / %.3g" % (b, n, err, ek, ev))
        assert err <= TOL_BF16 and ek <= TOL_BF16 and ev <= TOL_BF16
