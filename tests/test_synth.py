"""The seeded input generator: determinism, slicing, distribution and the Q8_0 planes."""
import numpy as np

import synth


def test_draws_are_pure_functions_of_index():
    a = synth.normal_f32(0, 7, (1001,), 1.0)
    for first in (0, 1, 3, 4, 997):
        b = synth.normal_f32(0, 7, (4,), 1.0, first=first)
        assert np.array_equal(b, a[first:first + 4])
    assert not np.array_equal(a[:16], synth.normal_f32(0, 8, (16,), 1.0))
    assert not np.array_equal(a[:16], synth.normal_f32(1, 7, (16,), 1.0))
    assert np.array_equal(synth.normal_bf16(0, 7, (1001,), 1.0), synth.f32_to_bf16(a))


def test_normal_moments():
    z = synth.normal_f32(5, 0, (400_000,), 1.0).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.1  # Gaussian kurtosis


def test_uniform_int_range_and_coverage():
    t = synth.uniform_int(1, 3, 50_000, 128, 4096)
    assert t.min() >= 128 and t.max() <= 4096
    assert len(np.unique(synth.uniform_int(1, 3, 50_000, 0, 255))) == 256


def test_q8_0_planes_round_trip_bound_and_zero_block():
    w = synth.normal_f32(0, 9, (16, 128), 0.02)
    w[3, 32:64] = 0.0
    q, s = synth.q8_0_quantize(w)
    sc = s.view(np.float16).astype(np.float64)  # numpy's binary16 decode
    assert np.all(q[3, 32:64] == 0) and sc[3, 1] == 0
    blocks = np.abs(q.reshape(16, 4, 32)).max(-1)
    assert np.all((blocks == 127) | (sc == 0))
    deq = q.astype(np.float64).reshape(16, 4, 32) * sc[:, :, None]
    err = np.abs(deq.reshape(16, 128) - w)
    # half a quantisation step plus the f16 rounding of the scale (2^-11 relative)
    bound = np.repeat(sc * 0.5 + np.abs(sc) * 127 * 2.0 ** -11, 32, axis=1) + 1e-12
    assert np.all(err <= bound)


def test_f16_encode_matches_numpy():
    x = np.concatenate([synth.normal_f32(0, 11, (20000,), 1.0) * 10.0 ** e for e in range(-9, 5)])
    x = np.concatenate([x, [0.0, -0.0, 65504.0, 70000.0, 1e-8, 6.1e-5]]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(synth.f32_to_f16(x), ref)


def test_weight_shapes_and_streamed_bytes():
    W = synth.make_weights(synth.TINY)
    assert W.w_qkv[0].shape == (192, 64) and W.w_gu[1].shape == (344, 64) and W.w_down[0].shape == (64, 172)
    assert W.streamed_bytes() == 4 * (2 * 49408 + 256 * 64)
    trace = synth.make_trace(synth.MISTRAL7B, n_jobs=64)
    assert len(trace) == 64 and all(32 <= len(j.prompt) <= 1024 for j in trace)
    assert all(16 <= j.max_new_tokens <= 256 for j in trace)
    arr = [j.arrival_step for j in trace]
    assert arr == sorted(arr) and 120 < arr[-1] < 400  # mean gap 4 over 64 jobs
