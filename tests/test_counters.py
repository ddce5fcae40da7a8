"""The roofline counters against the pages' own figures for the SmolLM2-135M
shape ("MODEL-BATCHING-RESULTS — multi-user batched decode, measured", "The
lever" and "The honest ceiling"): about 150 MB of Q8_0 weights streamed per
token, a B=512 step of about 138 GFLOP including the LM head on all users,
about 100 MB of logits per step at B=512, and 0.50 flop/byte at batch 1 in
f32."""
import math

import synth
from continuous_batching_decode_step_amd import roofline as rf


def test_q8_weight_stream_about_150mb():
    b = rf.weight_bytes(synth.SMOL135M_Q8)
    assert rf.streamed_params(synth.SMOL135M) == 134_479_872
    assert abs(b - 142.9e6) < 0.1e6 and 130e6 < b < 160e6


def test_b512_step_about_138_gflop_and_100mb_logits():
    # matmul work only (2 flops per weight per user), as the page counts it
    f = 2.0 * rf.streamed_params(synth.SMOL135M) * 512
    assert abs(f / 1e9 - 137.7) < 0.1 and abs(f / 1e9 - 138) < 1
    assert abs(512 * synth.SMOL135M.vocab * 4 / 1e6 - 100.7) < 0.1


def test_batch1_f32_intensity_half_flop_per_byte():
    cfg = synth.SMOL135M
    assert 2.0 * rf.streamed_params(cfg) / rf.weight_bytes(cfg) == 0.5


def test_step_bytes_and_flops_7b():
    cfg = synth.MISTRAL7B
    assert rf.streamed_params(cfg) == 7_110_393_856
    assert rf.weight_bytes(cfg) == 14_220_787_712
    assert rf.kv_bytes_per_token(cfg) == 131072
    # one lane at 2112 cached positions: weights + history + new slot + logits + embedding row
    b = rf.step_bytes(cfg, [2112])
    assert abs(b - (14_220_787_712 + 2112 * 131072 + 131072 + 32000 * 4 + 4096 * 2)) < 1
    t = rf.roofline_time_s(cfg, [2112])
    assert abs(t - b / 8e12) < 1e-12 and abs(1 / t - 552) < 1
    # per-kernel bytes sum over the layer classes + head ~ the step's weight stream
    per = sum(rf.kernel_bytes(cfg, c, [0]) for c in ("gemm_qkv", "gemm_o", "gemm_gu", "gemm_down"))
    assert per * cfg.n_layers + rf.kernel_bytes(cfg, "gemm_head", [0]) > rf.weight_bytes(cfg)
