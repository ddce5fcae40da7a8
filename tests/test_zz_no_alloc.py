"""The allocation-free decode step (cbd_decode_step_batch_noalloc), through the C
ABI: two calls in a row, the second over fewer lanes, give logits, argmax and
KV bit-identical to the workspace entry point (cbd_decode_step_batch) on a
twin arena holding the same caches, and allocate nothing.  A step whose lanes
need more than the static scratch holds is refused before any GPU work."""
import numpy as np
import pytest

import continuous_batching_decode_step_amd as cbd
import synth
from gpu_helpers import say

pytestmark = pytest.mark.gpu

CFG = synth.ModelConfig("noalloc-hd128-bf16", d=2048, n_layers=2, n_heads=16, n_kv_heads=4, head_dim=128,
                        ffn=512, vocab=1000, wtype=synth.WTYPE_BF16)
LENS = [130, 61, 200, 64, 1, 300]
MAX_SEQ = 400
CALLS = [[0, 1, 2, 3, 4, 5], [5, 2, 0]]  # the second call has fewer lanes


def _kv_export(arena, lane, cfg):
    n = arena.lane_length(lane)
    shape = (cfg.n_layers, cfg.n_kv_heads, n, cfg.head_dim)
    k, v = np.empty(shape, np.uint16), np.empty(shape, np.uint16)
    arena.kv_export(lane, k, v)
    return k, v


def test_noalloc_step_equals_the_workspace_step():
    import torch
    say("case: noalloc vs workspace step, %s, lanes %s, calls %s" % (CFG.name, LENS, CALLS))
    W = synth.make_weights(CFG)
    dw = cbd.upload_weights(W)
    model = cbd.Model(CFG, dw)
    n = len(LENS)
    stream = torch.cuda.current_stream()
    mems, arenas, lanes = [], [], []
    for _ in range(2):
        mem = torch.empty(cbd.arena_bytes(CFG, n, MAX_SEQ), dtype=torch.uint8, device="cuda")
        ar = cbd.Arena(model, n, MAX_SEQ, mem)
        ls = [ar.lane_alloc() for _ in range(n)]
        for b in range(n):
            k, v = synth.lane_kv_bf16(CFG, b, LENS[b])
            ar.kv_import(ls[b], LENS[b], k, v, stream)
        mems.append(mem)
        arenas.append(ar)
        lanes.append(ls)
    wsb = model.workspace_bytes(n, MAX_SEQ)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = [(torch.empty((n, CFG.vocab), dtype=torch.float32, device="cuda"),
            torch.empty(n, dtype=torch.int32, device="cuda")) for _ in range(2)]
    pos = [np.array(LENS, np.int32), np.array(LENS, np.int32)]
    torch.cuda.synchronize()
    for c, sel in enumerate(CALLS):
        toks = [int(t) for t in synth.uniform_int(1, 500 + c, len(sel), 0, CFG.vocab - 1)]
        p0 = pos[0][sel].copy()
        model.decode_step_batch(arenas[0], [lanes[0][i] for i in sel], p0, toks, out[0][0], out[0][1], ws, wsb,
                                stream)
        pos[0][sel] = p0
        before = cbd.alloc_count()
        p1 = pos[1][sel].copy()
        model.decode_step_batch_noalloc(arenas[1], [lanes[1][i] for i in sel], p1, toks, out[1][0], out[1][1],
                                        stream)
        pos[1][sel] = p1
        torch.cuda.synchronize()
        assert cbd.alloc_count() == before
        B = len(sel)
        lg0, lg1 = out[0][0][:B].cpu().numpy(), out[1][0][:B].cpu().numpy()
        am0, am1 = out[0][1][:B].cpu().numpy(), out[1][1][:B].cpu().numpy()
        assert np.array_equal(pos[0], pos[1])
        assert np.array_equal(lg0.view(np.uint32), lg1.view(np.uint32)), c
        assert np.array_equal(am0, am1) and np.array_equal(am1, np.argmax(lg1, axis=1))
        say("call %d: %d lanes, logits and argmax bit-identical" % (c, B))
    for b in range(n):
        k0, v0 = _kv_export(arenas[0], lanes[0][b], CFG)
        k1, v1 = _kv_export(arenas[1], lanes[1][b], CFG)
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1), b
    for ar in arenas:
        ar.close()


def test_noalloc_step_refuses_lanes_beyond_the_scratch():
    import torch
    W = synth.make_weights(CFG)
    model = cbd.Model(CFG, cbd.upload_weights(W))
    max_seq = 1 << 20  # attention partials of such lanes: ~34 MB each at this shape
    need2 = model.workspace_bytes(2, max_seq)
    assert need2 > cbd.lib().cbd_noalloc_scratch_bytes() >= model.workspace_bytes(1, max_seq)
    mem = torch.empty(4 * cbd.arena_block_bytes(CFG), dtype=torch.uint8, device="cuda")
    ar = cbd.Arena(model, 2, max_seq, mem)
    ls = [ar.lane_alloc() for _ in range(2)]
    logits = torch.empty((2, CFG.vocab), dtype=torch.float32, device="cuda")
    pos = np.zeros(2, np.int32)
    with pytest.raises(cbd.CbdError) as e:
        model.decode_step_batch_noalloc(ar, ls, pos, [1, 2], logits)
    assert e.value.name == "CBD_E_WORKSPACE" and list(pos) == [0, 0]
    p1 = np.zeros(1, np.int32)
    model.decode_step_batch_noalloc(ar, ls[:1], p1, [3], logits)
    torch.cuda.synchronize()
    assert list(p1) == [1] and ar.lane_length(ls[0]) == 1
    ar.close()
