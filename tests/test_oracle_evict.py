"""Pins of the oracle's span eviction (orc_lane_evict_span): entries after the
span move down by its length d, keys rotated by -d positions, values
unchanged.  Pinned against the oracle's own rotary (an independent path: keys
built as R(t) k_raw must become R(t - d) k_raw), the empty span, the tail span
(a truncation), and the bf16 rounding of moved keys."""
import numpy as np
import pytest

import oracle
import synth

CFG = synth.ModelConfig("evict-tiny-f32", d=64, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                        vocab=64)


def _lane(cfg, length, seed=0):
    M = oracle.Model(synth.make_weights(cfg))
    rng = np.random.default_rng(seed)
    shape = (cfg.n_layers, cfg.n_kv_heads, length, cfg.head_dim)
    raw = rng.standard_normal(shape).astype(np.float32)
    k = raw.copy()
    for l in range(cfg.n_layers):
        for g in range(cfg.n_kv_heads):
            for t in range(length):
                k[l, g, t] = oracle.rope(raw[l, g, t], t, cfg.rope_theta)
    v = rng.standard_normal(shape).astype(np.float32)
    if cfg.wtype == synth.WTYPE_BF16:
        k, v = synth.bf16_to_f32(synth.f32_to_bf16(k)), synth.bf16_to_f32(synth.f32_to_bf16(v))
    lane = M.lane(length + 4)
    lane.set_kv(k, v)
    return M, lane, raw, k, v


def test_moved_keys_are_rotated_to_their_new_positions():
    M, lane, raw, k, v = _lane(CFG, 40)
    b, e = 7, 19
    lane.evict_span(b, e)
    d = e - b
    assert lane.length == 40 - d
    k2, v2 = lane.get_kv()
    assert np.array_equal(k2[:, :, :b], k[:, :, :b]) and np.array_equal(v2[:, :, :b], v[:, :, :b])
    assert np.array_equal(v2[:, :, b:], v[:, :, e:])
    for t in range(e, 40):  # R(-d) R(t) k_raw = R(t - d) k_raw, up to f32 rounding
        want = np.stack([[oracle.rope(raw[l, g, t], t - d, CFG.rope_theta) for g in range(CFG.n_kv_heads)]
                         for l in range(CFG.n_layers)])
        got = k2[:, :, t - d]
        assert np.max(np.abs(got - want)) <= 4e-6 * max(1.0, np.max(np.abs(want))), t
        # and not the rotation the other way (a sign slip would give R(t + d))
        if t > 0:
            wrong = oracle.rope(raw[0, 0, t], t + d, CFG.rope_theta)
            assert np.max(np.abs(k2[0, 0, t - d] - wrong)) > 1e-3


def test_empty_span_and_tail_span():
    M, lane, raw, k, v = _lane(CFG, 30)
    lane.evict_span(12, 12)
    k2, v2 = lane.get_kv()
    assert lane.length == 30 and np.array_equal(k2, k) and np.array_equal(v2, v)
    lane.evict_span(20, 30)  # the tail: a truncation, nothing moves
    k3, v3 = lane.get_kv()
    assert lane.length == 20 and np.array_equal(k3, k[:, :, :20]) and np.array_equal(v3, v[:, :, :20])
    with pytest.raises(ValueError):
        lane.evict_span(5, 21)
    with pytest.raises(ValueError):
        lane.evict_span(6, 5)


def test_bf16_moved_keys_are_rounded():
    cfg = CFG.with_wtype(synth.WTYPE_BF16)
    M, lane, raw, k, v = _lane(cfg, 24)
    lane.evict_span(3, 8)
    k2, v2 = lane.get_kv()
    assert np.array_equal(synth.bf16_to_f32(synth.f32_to_bf16(k2)), k2)  # every stored key is a bf16 value
    assert np.array_equal(v2[:, :, 3:], v[:, :, 8:])
