"""The C-ABI library on the host: it loads, exports every symbol include/cbd.h
declares, validates models, arenas and steps, and keeps lane accounting —
without any GPU call (fake device addresses are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import continuous_batching_decode_step_amd as cbd
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(cbd.LIB_PATH):
        from continuous_batching_decode_step_amd import build
        build.build()
    cbd.lib()


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "cbd.h")).read()
    declared = set(re.findall(r"\b(cbd_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(cbd.SYMBOLS)
    L = cbd.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert cbd.lib().cbd_version().decode().startswith("cbd")


FAKE = 1 << 24  # a 256-byte aligned address that is never dereferenced on the host


def fake_weights(cfg):
    fm = lambda: cbd.DeviceMatrix(FAKE, FAKE if cfg.wtype == synth.WTYPE_Q8_0 else None)
    L = cfg.n_layers
    return cbd.DeviceWeights(embed=fm(), lm_head=None if cfg.tied else fm(), final_norm=FAKE,
                             attn_norm=[FAKE] * L, ffn_norm=[FAKE] * L, w_qkv=[fm() for _ in range(L)],
                             w_o=[fm() for _ in range(L)], w_gu=[fm() for _ in range(L)],
                             w_down=[fm() for _ in range(L)])


class _P:  # DeviceMatrix holding raw ints
    pass


def test_model_create_validates_shapes():
    for cfg in (synth.TINY, synth.SMOL135M, synth.SMOL135M_Q8, synth.MISTRAL7B):
        m = cbd.Model(cfg, fake_weights(cfg))
        m.close()
    from dataclasses import replace
    with pytest.raises(cbd.CbdError) as e:
        cbd.Model(replace(synth.TINY, head_dim=24), fake_weights(synth.TINY))
    assert e.value.name == "CBD_E_UNSUPPORTED"
    with pytest.raises(cbd.CbdError) as e:
        cbd.Model(replace(synth.TINY, n_kv_heads=3), fake_weights(synth.TINY))
    assert e.value.name == "CBD_E_UNSUPPORTED"
    with pytest.raises(cbd.CbdError) as e:  # Q8_0 needs K % 32 == 0 (ffn 172)
        cbd.Model(synth.TINY.with_wtype(synth.WTYPE_Q8_0), fake_weights(synth.TINY.with_wtype(synth.WTYPE_Q8_0)))
    assert e.value.name == "CBD_E_UNSUPPORTED"
    w = fake_weights(synth.TINY)
    w.w_o[1] = cbd.DeviceMatrix(FAKE + 8)  # misaligned rows
    with pytest.raises(cbd.CbdError) as e:
        cbd.Model(synth.TINY, w)
    assert e.value.name == "CBD_E_ARG"
    w = fake_weights(synth.TINY)
    w.ffn_norm[1] = FAKE + 4  # gains are loaded 16 bytes at a time
    with pytest.raises(cbd.CbdError) as e:
        cbd.Model(synth.TINY, w)
    assert e.value.name == "CBD_E_ARG"
    wq = fake_weights(synth.SMOL135M_Q8)
    wq.w_gu[0] = cbd.DeviceMatrix(FAKE, None)  # Q8_0 without scales
    with pytest.raises(cbd.CbdError):
        cbd.Model(synth.SMOL135M_Q8, wq)


def test_arena_bytes_per_token():
    # K and V, every layer and KV head: 2 * L * Hkv * hd * bytes per position per
    # lane, for max_seq rounded up to whole 64-position chunks
    assert cbd.arena_bytes(synth.MISTRAL7B, 1, 64) == 64 * 131072
    assert cbd.arena_bytes(synth.MISTRAL7B, 1, 1) == 64 * 131072
    assert cbd.arena_bytes(synth.SMOL135M, 1, 128) == 128 * 46080
    assert cbd.arena_bytes(synth.SMOL135M, 1, 65) == 128 * 46080
    assert cbd.arena_bytes(synth.TINY, 3, 10) == 3 * 64 * 1024
    assert cbd.arena_bytes(synth.TINY, 0, 10) == 0


def make_model_arena(cfg=synth.TINY, n_lanes=4, max_seq=8):
    m = cbd.Model(cfg, fake_weights(cfg))
    a = cbd.Arena(m, n_lanes, max_seq, FAKE, cbd.arena_bytes(cfg, n_lanes, max_seq))
    return m, a


def test_lane_alloc_clear_evict_and_usage_returns_to_zero():
    m, a = make_model_arena()
    lanes = [a.lane_alloc() for _ in range(4)]
    assert lanes == [0, 1, 2, 3] and a.live_lanes == 4
    with pytest.raises(cbd.CbdError) as e:
        a.lane_alloc()
    assert e.value.name == "CBD_E_NO_FREE_LANE"
    assert a.used_bytes == 0
    a.lane_evict(2)
    with pytest.raises(cbd.CbdError) as e:
        a.lane_length(2)
    assert e.value.name == "CBD_E_LANE_NOT_LIVE"
    with pytest.raises(cbd.CbdError) as e:
        a.lane_clear(2)
    assert e.value.name == "CBD_E_LANE_NOT_LIVE"
    assert a.lane_alloc() == 2  # lowest free lane is reused
    for l in lanes:
        a.lane_evict(l)
    assert a.live_lanes == 0 and a.used_bytes == 0
    with pytest.raises(cbd.CbdError) as e:
        a.lane_evict(9)
    assert e.value.name == "CBD_E_ARG"


def test_arena_is_a_block_pool():
    # a block: 64 positions of one lane, every layer and KV head, K and V
    assert cbd.arena_block_bytes(synth.TINY) == 2 * 2 * 4 * 64 * 16 * 4
    assert cbd.arena_block_bytes(synth.MISTRAL7B) == 64 * 131072
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    need = cbd.arena_bytes(synth.TINY, 2, 8)  # two lanes of one chunk each
    a = cbd.Arena(m, 2, 8, FAKE, need)
    assert a.n_blocks == 2 and a.free_blocks == 2
    # less memory is a smaller pool, shared by the lanes
    a1 = cbd.Arena(m, 2, 8, FAKE, need - 1)
    assert a1.n_blocks == 1 and a1.free_blocks == 1


def test_arena_create_rejects_small_or_misaligned_memory():
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    bb = cbd.arena_block_bytes(synth.TINY)
    with pytest.raises(cbd.CbdError):
        cbd.Arena(m, 2, 8, FAKE, bb - 1)
    with pytest.raises(cbd.CbdError):
        cbd.Arena(m, 2, 8, FAKE + 64, 2 * bb)


def test_step_needing_more_blocks_than_the_pool_changes_nothing():
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    a = cbd.Arena(m, 2, 8, FAKE, cbd.arena_block_bytes(synth.TINY))  # one block for two lanes
    l0, l1 = a.lane_alloc(), a.lane_alloc()
    assert step_err(m, a, [l0, l1], [0, 0], [1, 2]) == "CBD_E_KV_FULL"
    assert a.free_blocks == 1


def test_arena_accepts_long_contexts():
    # no bound on max_seq beyond memory: 512k positions of the tiny model
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    n = 512 * 1024
    a = cbd.Arena(m, 1, n, FAKE, cbd.arena_bytes(synth.TINY, 1, n))
    assert a.max_seq == n


def step_err(m, a, lanes, pos, toks, ws=FAKE, wsb=None, logits=FAKE):
    pos = np.array(pos, np.int32)
    before = pos.copy()
    lens = {l: a.lane_length(l) for l in range(a.n_lanes) if _live(a, l)}
    wsb = m.workspace_bytes(max(1, len(lanes)), a.max_seq) if wsb is None else wsb
    with pytest.raises(cbd.CbdError) as e:
        m.decode_step_batch(a, lanes, pos, toks, logits, None, ws, wsb, stream=0)
    # a failed call changes nothing
    assert np.array_equal(pos, before)
    assert lens == {l: a.lane_length(l) for l in range(a.n_lanes) if _live(a, l)}
    return e.value.name


def _live(a, l):
    try:
        a.lane_length(l)
        return True
    except cbd.CbdError:
        return False


def test_step_validation_errors_change_nothing():
    m, a = make_model_arena()
    l0, l1, l2 = a.lane_alloc(), a.lane_alloc(), a.lane_alloc()
    a.lane_evict(l2)
    assert step_err(m, a, [l0, l0], [0, 0], [1, 2]) == "CBD_E_DUP_LANE"
    assert step_err(m, a, [l0, l2], [0, 0], [1, 2]) == "CBD_E_LANE_NOT_LIVE"
    assert step_err(m, a, [l0, 7], [0, 0], [1, 2]) == "CBD_E_ARG"
    assert step_err(m, a, [l0, l1], [0, 1], [1, 2]) == "CBD_E_POS_MISMATCH"
    assert step_err(m, a, [l0, l1], [0, 0], [1, 256]) == "CBD_E_TOKEN"
    assert step_err(m, a, [l0, l1], [0, 0], [-1, 2]) == "CBD_E_TOKEN"
    assert step_err(m, a, [], [], []) == "CBD_E_ARG"
    assert step_err(m, a, [l0, l1], [0, 0], [1, 2], ws=0) == "CBD_E_WORKSPACE"
    small = m.workspace_bytes(1, a.max_seq)
    assert step_err(m, a, [l0, l1], [0, 0], [1, 2], wsb=small) == "CBD_E_WORKSPACE"
    assert step_err(m, a, [l0, l1], [0, 0], [1, 2], logits=0) == "CBD_E_ARG"


def test_workspace_grows_with_batch_and_context():
    m = cbd.Model(synth.MISTRAL7B, fake_weights(synth.MISTRAL7B))
    w1 = m.workspace_bytes(1, 4097)
    w8 = m.workspace_bytes(8, 4097)
    assert 0 < w1 < w8 < m.workspace_bytes(64, 4097)
    assert m.workspace_bytes(8, 512) < w8
    assert m.workspace_bytes(0, 10) == 0
    with pytest.raises(cbd.CbdError):
        m.set_variant(5)
    m.set_variant(1)


def prefill_err(m, a, lanes, pos, counts, toks, ws=FAKE, wsb=None, logits=FAKE):
    pos = np.array(pos, np.int32)
    before = pos.copy()
    lens = {l: a.lane_length(l) for l in range(a.n_lanes) if _live(a, l)}
    free = a.free_blocks
    wsb = m.workspace_bytes(max(1, int(sum(counts))), a.max_seq) if wsb is None else wsb
    with pytest.raises(cbd.CbdError) as e:
        m.prefill_batch(a, lanes, pos, counts, toks, logits, None, ws, wsb, stream=0)
    # a failed call changes nothing
    assert np.array_equal(pos, before) and a.free_blocks == free
    assert lens == {l: a.lane_length(l) for l in range(a.n_lanes) if _live(a, l)}
    return e.value.name


def test_prefill_validation_errors_change_nothing():
    m, a = make_model_arena()  # 4 lanes of at most 8 positions
    l0, l1, l2 = a.lane_alloc(), a.lane_alloc(), a.lane_alloc()
    a.lane_evict(l2)
    assert prefill_err(m, a, [l0, l0], [0, 0], [1, 2], [1, 2, 3]) == "CBD_E_DUP_LANE"
    assert prefill_err(m, a, [l0, l2], [0, 0], [1, 2], [1, 2, 3]) == "CBD_E_LANE_NOT_LIVE"
    assert prefill_err(m, a, [l0, 9], [0, 0], [1, 2], [1, 2, 3]) == "CBD_E_ARG"
    assert prefill_err(m, a, [l0, l1], [0, 1], [1, 2], [1, 2, 3]) == "CBD_E_POS_MISMATCH"
    assert prefill_err(m, a, [l0, l1], [0, 0], [1, 0], [1]) == "CBD_E_ARG"
    assert prefill_err(m, a, [l0, l1], [0, 0], [1, 9], [1] * 10) == "CBD_E_KV_FULL"  # 9 > max_seq 8
    assert prefill_err(m, a, [l0, l1], [0, 0], [2, 2], [1, 2, 3, 256]) == "CBD_E_TOKEN"
    assert prefill_err(m, a, [], [], [], []) == "CBD_E_ARG"
    small = m.workspace_bytes(3, a.max_seq)  # 3 rows; the call has 4
    assert prefill_err(m, a, [l0, l1], [0, 0], [2, 2], [1, 2, 3, 4], wsb=small) == "CBD_E_WORKSPACE"
    assert prefill_err(m, a, [l0, l1], [0, 0], [2, 2], [1, 2, 3, 4], ws=0) == "CBD_E_WORKSPACE"


def test_prefill_needing_more_blocks_than_the_pool_changes_nothing():
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    a = cbd.Arena(m, 2, 200, FAKE, 2 * cbd.arena_block_bytes(synth.TINY))  # two blocks for two lanes
    l0, l1 = a.lane_alloc(), a.lane_alloc()
    # 65 tokens span two blocks, and the other lane needs one more
    assert prefill_err(m, a, [l0, l1], [0, 0], [65, 1], [1] * 66) == "CBD_E_KV_FULL"
    assert a.free_blocks == 2


def test_lane_clone_validation():
    m, a = make_model_arena()
    l0, l1, l2 = a.lane_alloc(), a.lane_alloc(), a.lane_alloc()
    a.lane_evict(l2)
    for args, name in (((l0, l0, 0), "CBD_E_ARG"), ((l0, l1, 1), "CBD_E_ARG"), ((l0, l2, 0), "CBD_E_LANE_NOT_LIVE"),
                       ((l2, l0, 0), "CBD_E_LANE_NOT_LIVE"), ((l0, 9, 0), "CBD_E_ARG")):
        with pytest.raises(cbd.CbdError) as e:
            a.lane_clone(*args, stream=0)
        assert e.value.name == name, args
    a.lane_clone(l0, l1, 0, stream=0)  # an empty prefix: no copy
    assert a.lane_length(l1) == 0 and a.free_blocks == a.n_blocks


def test_lane_evict_span_validation():
    m, a = make_model_arena()
    l0, l1 = a.lane_alloc(), a.lane_alloc()
    a.lane_evict(l1)
    a.lane_evict_span(l0, 0, 0, stream=0)  # empty span of an empty lane: nothing to do
    for args, name in (((l0, 0, 1), "CBD_E_ARG"), ((l0, 1, 0), "CBD_E_ARG"), ((l0, -1, 0), "CBD_E_ARG"),
                       ((l1, 0, 0), "CBD_E_LANE_NOT_LIVE")):
        with pytest.raises(cbd.CbdError) as e:
            a.lane_evict_span(*args, stream=0)
        assert e.value.name == name, args


class _FakeBuf:
    """Stands in for a device tensor: an address and a size, never dereferenced."""

    def __init__(self, addr, n):
        self.addr, self.n = addr, n

    def numel(self):
        return self.n

    def element_size(self):
        return 1

    def data_ptr(self):
        return self.addr


def test_device_scheduler_refuses_what_the_arena_or_workspace_cannot_hold():
    # The scheduler over the decode path bounds sessions by the arena's max_seq
    # (a session ends holding prompt + max_new - 1 positions) and prompts by the
    # workspace's rows (a prompt is prefilled in one call); refusals happen at
    # submission, so nothing here reaches the device.
    cfg = synth.TINY
    m = cbd.Model(cfg, fake_weights(cfg))
    max_seq, rows = 40, 8
    a = cbd.Arena(m, 2, max_seq, FAKE, cbd.arena_bytes(cfg, 2, max_seq))
    wsb = m.workspace_bytes(rows, max_seq)
    assert m.workspace_bytes(rows + 1, max_seq) > wsb
    b = dict(weight_bytes=0, kv_budget_bytes=1 << 40, kv_bytes_per_token=1, scratch_per_session=0,
             scratch_budget_bytes=0, max_active=2, max_queue=8, max_batch=2, max_prefill_tokens_per_tick=64)
    s = cbd.Scheduler(b, device=(m, a, _FakeBuf(FAKE, wsb), FAKE, FAKE, 0))
    assert s.submit(1, [1] * (rows + 1), 1) == "REJECTED_SCRATCH_BUDGET"
    assert s.submit(2, [1] * rows, max_seq - rows + 1) == "QUEUED"       # ends at max_seq positions
    assert s.submit(3, [1] * rows, max_seq - rows + 2) == "REJECTED_KV_BUDGET"
    t = s.telemetry()
    assert (t["rejected_scratch"], t["rejected_kv"], t["queued"]) == (1, 1, 1)
    s.close()
    a.close()
    m.close()


def test_arena_creation_needs_no_device():
    # Arenas are host bookkeeping over caller memory: created here without a
    # GPU (the pinned staging for their steps is sized when a device exists,
    # else by the first step), their lanes and blocks are all available.
    m = cbd.Model(synth.TINY, fake_weights(synth.TINY))
    a = cbd.Arena(m, 3, 100, FAKE, cbd.arena_bytes(synth.TINY, 3, 100))
    assert a.n_blocks == a.free_blocks == 3 * 2
    assert [a.lane_alloc() for _ in range(3)] == [0, 1, 2]
    assert cbd.lib().cbd_last_error().decode() == ""
    a.close()
    m.close()
