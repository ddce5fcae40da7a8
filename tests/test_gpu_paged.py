"""Paged KV: the arena is a pool of 64-position blocks, and a lane's chunks
live in whatever blocks the pool hands out.  Lanes whose blocks are scattered
over the pool (imports and evictions interleaved, steps that open new chunks
and so take blocks mid-run) must give bit-identical logits and KV to the same
lanes in a fresh arena, where every lane's blocks are consecutive: attention
reads a chunk from its block and nothing else about the layout matters.  Both
attention kernels are covered (bf16 head_dim 128, the matrix-core kernel; the
135M shape in f32, the general kernel).  A step that needs more blocks than
are free fails with CBD_E_KV_FULL and changes nothing; evicting every lane
returns every block.
"""
import numpy as np
import pytest

import continuous_batching_decode_step_amd as cbd
import oracle
import synth
from gpu_helpers import TOL_BF16, TOL_F32, engine_for, rel_err, say

pytestmark = pytest.mark.gpu

SHAPES = [
    synth.ModelConfig("paged-hd128-bf16", d=2048, n_layers=2, n_heads=16, n_kv_heads=4, head_dim=128, ffn=256,
                      vocab=512, wtype=synth.WTYPE_BF16),
    synth.SMOL135M,
]
# lengths at import: lanes 1 and 3 open a chunk while stepping, lane 4 ends on a
# chunk boundary, lane 5 spans three groups of chunks (only the last holds the
# new slot; the others must leave the pool alone)
LENS = [130, 61, 200, 64, 58, 600]
STEPS = 6


def _kv(cfg, b, n):
    if cfg.wtype == synth.WTYPE_BF16:
        return synth.lane_kv_bf16(cfg, b, n)
    return synth.lane_kv_f32(cfg, b, n)


def _run(eng, cfg, lanes, toks, steps):
    pos = np.array([eng.arena.lane_length(l) for l in lanes], np.int32)
    out = []
    for s in range(steps):
        _, lg = eng.step_sync(lanes, pos, [int(t[s]) for t in toks], want_logits=True)
        out.append(lg.copy())
    return out


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_scattered_blocks_match_consecutive_blocks(cfg):
    say("case: %s, lanes of lengths %s, %d steps" % (cfg.name, LENS, STEPS))
    W = synth.make_weights(cfg)
    n = len(LENS)
    max_seq = max(LENS) + STEPS
    toks = [synth.uniform_int(1, 700 + b, STEPS, 0, cfg.vocab - 1) for b in range(n)]
    kv = [_kv(cfg, b, LENS[b]) for b in range(n)]

    # reference: a fresh arena, each lane's blocks consecutive
    ref = engine_for(cfg, W, n, max_seq)
    rl = [ref.arena.lane_alloc() for _ in range(n)]
    for b in range(n):
        ref.arena.kv_import(rl[b], LENS[b], kv[b][0], kv[b][1], ref.stream)
    want = _run(ref, cfg, rl, toks, STEPS)
    want_kv = [ref.kv_export(l) for l in rl]

    # paged: a pool with exactly the blocks the run needs, handed out scattered
    need = sum((LENS[b] + STEPS + 63) // 64 for b in range(n))
    from continuous_batching_decode_step_amd.driver import Engine
    eng = Engine(cfg, cbd.upload_weights(W), n + 1, max_seq, kv_blocks=need)
    assert eng.arena.n_blocks == need
    lanes = [eng.arena.lane_alloc() for _ in range(n + 1)]
    spare = lanes.pop()   # a lane that takes blocks first, then gives them back
    eng.arena.kv_import(spare, 128, *_kv(cfg, 99, 128), eng.stream)
    for b in (4, 2, 0):
        eng.arena.kv_import(lanes[b], LENS[b], kv[b][0], kv[b][1], eng.stream)
    eng.arena.lane_evict(spare)
    for b in (3, 1, 5):
        eng.arena.kv_import(lanes[b], LENS[b], kv[b][0], kv[b][1], eng.stream)
    got = _run(eng, cfg, lanes, toks, STEPS)
    assert eng.arena.free_blocks == 0
    for s in range(STEPS):
        for b in range(n):
            assert np.array_equal(got[s][b].view(np.uint32), want[s][b].view(np.uint32)), (s, b)
    for b in range(n):
        gk, gv = eng.kv_export(lanes[b])
        assert np.array_equal(gk, want_kv[b][0]) and np.array_equal(gv, want_kv[b][1]), b
        # the imported slots are untouched by the steps, in both arenas
        m = LENS[b]
        assert np.array_equal(gk[:, :, :m], kv[b][0]) and np.array_equal(gv[:, :, :m], kv[b][1]), b

    # an exhausted pool: a step that opens a chunk fails and changes nothing
    assert eng.arena.lane_length(lanes[4]) == 64
    pos = np.array([64], np.int32)
    with pytest.raises(cbd.CbdError) as e:
        eng.step(lanes[4:5], pos, [1])
    assert e.value.name == "CBD_E_KV_FULL" and int(pos[0]) == 64 == eng.arena.lane_length(lanes[4])
    assert eng.arena.free_blocks == 0
    for l in lanes:
        eng.arena.lane_evict(l)
    assert eng.arena.free_blocks == eng.arena.n_blocks and eng.arena.used_bytes == 0


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_clone_prefix_continues_bitwise(cfg):
    """Prefix reuse: a lane cloned from another (whole, or a prefix that ends
    inside a block) continues exactly as the original would, and as a lane
    that imported the same prefix: same logits bits, same cache."""
    say("case: %s, clone prefixes" % cfg.name)
    W = synth.make_weights(cfg)
    L0, steps = 150, 3
    eng = engine_for(cfg, W, 4, L0 + steps + 4)
    a, b, c, d = [eng.arena.lane_alloc() for _ in range(4)]
    k, v = _kv(cfg, 3, L0)
    eng.arena.kv_import(a, L0, k, v, eng.stream)
    toks = synth.uniform_int(1, 1500, steps + 4, 0, cfg.vocab - 1)
    pos = np.array([L0], np.int32)
    for s in range(steps):
        eng.step_sync([a], pos, [int(toks[s])])
    n = L0 + steps
    eng.arena.lane_clone(a, b, n, eng.stream)      # the whole lane
    eng.arena.lane_clone(a, c, 100, eng.stream)    # a prefix ending inside a block
    ka, va = eng.kv_export(a)
    kb, vb = eng.kv_export(b)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    kc, vc = eng.kv_export(c)
    assert np.array_equal(kc, ka[:, :, :100]) and np.array_equal(vc, va[:, :, :100])
    # a and b continue in one step: same bits
    p2 = np.array([n, n], np.int32)
    _, lg = eng.step_sync([a, b], p2, [int(toks[steps])] * 2, want_logits=True)
    assert np.array_equal(lg[0].view(np.uint32), lg[1].view(np.uint32))
    # c continues as a lane that imported the same 100 positions
    eng.arena.kv_import(d, 100, np.ascontiguousarray(ka[:, :, :100]), np.ascontiguousarray(va[:, :, :100]),
                        eng.stream)
    p3 = np.array([100, 100], np.int32)
    _, lg = eng.step_sync([c, d], p3, [int(toks[steps + 1])] * 2, want_logits=True)
    assert np.array_equal(lg[0].view(np.uint32), lg[1].view(np.uint32))
    # eviction returns every block, the clones' included
    for l in (a, b, c, d):
        eng.arena.lane_evict(l)
    assert eng.arena.free_blocks == eng.arena.n_blocks


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_evict_span_matches_the_oracle(cfg):
    """Span eviction: the cache after dropping [37, 101) of a 200-position lane
    equals the oracle's (moved keys rotated by -64 positions with the same f32
    arithmetic, values moved), bit for bit; blocks past the new length return
    to the pool; and the next decode step matches the oracle's step on its
    evicted lane.  A second eviction of the tail is a truncation."""
    say("case: %s, span eviction" % cfg.name)
    W = synth.make_weights(cfg)
    n0, b, e = 200, 37, 101
    eng = engine_for(cfg, W, 1, n0 + 2)
    lane = eng.arena.lane_alloc()
    k, v = _kv(cfg, 5, n0)
    eng.arena.kv_import(lane, n0, k, v, eng.stream)
    free0 = eng.arena.free_blocks
    eng.arena.lane_evict_span(lane, b, e, eng.stream)
    n1 = n0 - (e - b)
    assert eng.arena.lane_length(lane) == n1
    assert eng.arena.free_blocks == free0 + (n0 + 63) // 64 - (n1 + 63) // 64
    M = oracle.Model(W)
    ol = M.lane(n0 + 2)
    f32 = (lambda a: synth.bf16_to_f32(a)) if cfg.wtype == synth.WTYPE_BF16 else (lambda a: a)
    ol.set_kv(f32(k), f32(v))
    ol.evict_span(b, e)
    ok, ov = ol.get_kv()
    gk, gv = eng.kv_export(lane)
    assert np.array_equal(f32(gv), ov)
    assert np.array_equal(f32(gk), ok), float(np.max(np.abs(f32(gk) - ok)))
    tok = int(synth.uniform_int(1, 1700, 1, 0, cfg.vocab - 1)[0])
    p = np.array([n1], np.int32)
    _, lg = eng.step_sync([lane], p, [tok], want_logits=True)
    ref = M.step(ol, tok)
    err = rel_err(lg[0], ref)
    say("  after eviction: logits max rel %.3g" % err)
    assert err <= (TOL_BF16 if cfg.wtype == synth.WTYPE_BF16 else TOL_F32)
    # the tail: a truncation
    eng.arena.lane_evict_span(lane, 50, n1 + 1, eng.stream)
    gk2, _ = eng.kv_export(lane)
    assert eng.arena.lane_length(lane) == 50 and np.array_equal(gk2, gk[:, :, :50])


def test_graph_replay_follows_the_arena_over_a_reused_buffer():
    """Graph replay captures the pool's addresses (the V region follows the K
    region, whose size is the block count) into the kernels' arguments.  Two
    arenas with different block counts over the same device buffer, one after
    the other, each with the same lanes and workspace: every replayed step must
    equal the same step launched plainly, bit for bit (a graph captured over the
    first arena must never serve the second)."""
    import torch
    cfg = SHAPES[0]
    W = synth.make_weights(cfg)
    dw = cbd.upload_weights(W)
    model = cbd.Model(cfg, dw)
    n, steps = 3, 3
    lens = [70, 5, 129]
    max_seq = max(lens) + steps
    bb = cbd.arena_block_bytes(cfg)
    per_lane = (max_seq + 63) // 64
    mem = torch.empty((n * per_lane + 5) * bb, dtype=torch.uint8, device="cuda")
    wsb = model.workspace_bytes(n, max_seq)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    logits = torch.empty((n, cfg.vocab), dtype=torch.float32, device="cuda")
    argmax = torch.empty(n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    toks = [synth.uniform_int(1, 900 + b, steps, 0, cfg.vocab - 1) for b in range(n)]
    kv = [synth.lane_kv_bf16(cfg, b, lens[b]) for b in range(n)]
    for blocks in (n * per_lane, n * per_lane + 5):
        say("case: arena of %d blocks over the shared buffer" % blocks)
        arena = cbd.Arena(model, n, max_seq, mem, dev_bytes=blocks * bb)
        assert arena.n_blocks == blocks
        lanes = [arena.lane_alloc() for _ in range(n)]
        for b in range(n):
            arena.kv_import(lanes[b], lens[b], kv[b][0], kv[b][1], stream)
        runs = []
        for graph in (True, False):
            model.set_graph_replay(graph)
            for b in range(n):
                arena.lane_truncate(lanes[b], lens[b])
            pos = np.array(lens, np.int32)
            out = []
            for s in range(steps):
                model.decode_step_batch(arena, lanes, pos, [int(t[s]) for t in toks], logits, argmax, ws, wsb,
                                        stream)
                out.append(logits.cpu().numpy().copy())
            runs.append(out)
        model.set_graph_replay(False)
        for s in range(steps):
            assert np.array_equal(runs[0][s].view(np.uint32), runs[1][s].view(np.uint32)), (blocks, s)
        arena.close()


def test_decode_steps_allocate_nothing():
    """Once the arena exists, decode steps of any width allocate no device or
    pinned host memory (their staging is sized at arena creation and the
    workspace is the caller's), including steps that open new KV blocks."""
    cfg = SHAPES[0]
    W = synth.make_weights(cfg)
    n = 6
    max_seq = 300
    eng = engine_for(cfg, W, n, max_seq)
    lanes = [eng.arena.lane_alloc() for _ in range(n)]
    for b, ln in enumerate(lanes):
        k, v = synth.lane_kv_bf16(cfg, b, 60 + 40 * b)
        eng.arena.kv_import(ln, 60 + 40 * b, k, v, eng.stream)
    pos = np.array([eng.arena.lane_length(l) for l in lanes], np.int32)
    before = cbd.alloc_count()
    for s, B in enumerate([1, 6, 3, 6, 2, 6, 6, 5]):
        idx = list(range(B))
        p = pos[idx].copy()
        eng.step([lanes[i] for i in idx], p, [int(s + i) % cfg.vocab for i in idx])
        pos[idx] = p
    eng.torch.cuda.synchronize()
    assert cbd.alloc_count() == before
    say("8 decode steps of 1-6 lanes, lanes at %s after: %d allocations" % (list(pos), cbd.alloc_count() - before))
