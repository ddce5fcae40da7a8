"""Whole-step pins of the oracle.

* Special weights whose decode step has a closed form: zero projections (the
  step reduces to head @ rmsnorm(E[token])), a uniform-attention averaging
  layer (the step reduces to a running mean of the normalised embeddings), and
  a key projection that selects one input so the stored key is cos/sin of the
  position.  These catch a dropped residual, an off-by-one in the attended
  range, a key stored before rotation or at the wrong slot, and a wrong GQA map.
* A SwiGLU block with selector weights and distinct norm gains per norm and
  layer: x_out = x + silu(sg * xf_i) * (su * xf_j) e_k per hidden unit, in
  closed form.  This catches silu on the up rows, the gate/up row order
  reversed, a dropped FFN residual, and one norm's gain used for another
  (checked by planting each mistake in the oracle: every one fails a pin).
* The invariants the pages state for the method ("MODEL-BATCHING-RESULTS",
  section "Correctness — proven, not asserted"): the panel step is bit-for-bit
  the serial step per user, logits and the whole KV cache, across distinct
  prompt lengths; lockstep greedy generation equals serial generation.  Lanes
  are isolated across prompt lengths 1/3/7 (DGR-012 evidence, "Acceptance
  criteria → evidence"), and a cleared lane behaves like a fresh one
  ("Fat-station continuous batching", "Components", fill()).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import Matrix, ModelConfig, Weights, WTYPE_BF16, WTYPE_F32, WTYPE_Q8_0


def _weights_from(cfg, embed, head, qkv, o, gu, down):
    W = Weights(cfg=cfg, embed=Matrix(WTYPE_F32, np.ascontiguousarray(embed, np.float32)),
                lm_head=None if cfg.tied else Matrix(WTYPE_F32, np.ascontiguousarray(head, np.float32)),
                final_norm=np.ones(cfg.d, np.float32))
    for l in range(cfg.n_layers):
        W.attn_norm.append(np.ones(cfg.d, np.float32))
        W.ffn_norm.append(np.ones(cfg.d, np.float32))
        W.w_qkv.append(Matrix(WTYPE_F32, np.ascontiguousarray(qkv[l], np.float32)))
        W.w_o.append(Matrix(WTYPE_F32, np.ascontiguousarray(o[l], np.float32)))
        W.w_gu.append(Matrix(WTYPE_F32, np.ascontiguousarray(gu[l], np.float32)))
        W.w_down.append(Matrix(WTYPE_F32, np.ascontiguousarray(down[l], np.float32)))
    return W


def _rms64(x, eps):
    x = np.asarray(x, np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps)


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / np.max(np.abs(b)))


def test_zero_projections_reduce_to_head_of_normalised_embedding():
    cfg = ModelConfig("t", d=32, n_layers=3, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=40)
    r = np.random.default_rng(11)
    E = r.standard_normal((cfg.vocab, cfg.d)) * 0.5
    H = r.standard_normal((cfg.vocab, cfg.d)) * 0.1
    L = cfg.n_layers
    # q/k/v and gate/up projections random: only W_o and W_down feed the residual.
    qkv = [r.standard_normal((cfg.n_qkv, cfg.d)) for _ in range(L)]
    gu = [r.standard_normal((2 * cfg.ffn, cfg.d)) for _ in range(L)]
    o = [np.zeros((cfg.d, cfg.q_dim)) for _ in range(L)]
    down = [np.zeros((cfg.d, cfg.ffn)) for _ in range(L)]
    M = oracle.Model(_weights_from(cfg, E, H, qkv, o, gu, down))
    lane = M.lane(8)
    for tok in [3, 17, 39, 0]:
        lg = M.step(lane, tok)
        ref = H @ _rms64(E[tok].astype(np.float32), cfg.rms_eps)
        assert _rel(lg, ref) < 2e-6
    assert lane.length == 4


def test_uniform_attention_layer_is_running_mean_with_gqa():
    # d = Hq*hd = 8, Hq = 2, Hkv = 1, hd = 4.  Wq = 0 -> all scores 0 -> uniform softmax
    # over t = 0..p; Wv selects xn[:4]; Wo = I; FFN zero.  Then
    # x_p = E[tok_p] + [m, m] with m = mean_{t<=p} rmsnorm(E[tok_t])[:4].
    cfg = ModelConfig("t", d=8, n_layers=1, n_heads=2, n_kv_heads=1, head_dim=4, ffn=8, vocab=16)
    r = np.random.default_rng(12)
    E = r.standard_normal((cfg.vocab, cfg.d))
    H = r.standard_normal((cfg.vocab, cfg.d))
    qkv = np.zeros((cfg.n_qkv, cfg.d))
    qkv[8:12] = r.standard_normal((4, 8))  # k rows: arbitrary, scores stay 0 because q = 0
    qkv[12:16, :4] = np.eye(4)             # v = xn[:4]
    M = oracle.Model(_weights_from(cfg, E, H, [qkv], [np.eye(8)], [np.zeros((16, 8))], [np.zeros((8, 8))]))
    toks = [5, 9, 9, 2, 15, 0, 7]
    lane = M.lane(len(toks))
    xn_hist = []
    for p, tok in enumerate(toks):
        lg = M.step(lane, tok)
        e = E[tok].astype(np.float32).astype(np.float64)
        xn_hist.append(_rms64(e, cfg.rms_eps)[:4])
        m = np.mean(xn_hist, axis=0)
        x = e + np.concatenate([m, m])
        ref = H.astype(np.float32).astype(np.float64) @ _rms64(x, cfg.rms_eps)
        assert _rel(lg, ref) < 1e-5, p


def test_stored_key_is_rotated_at_its_own_position():
    # k = xn[1] * e0 in the single KV head (hd = 4): the stored key at slot p must be
    # xn[1] * (cos p, 0, sin p, 0) (pair (0, 2), theta_0 = 1); v = xn[:4] stored as is.
    cfg = ModelConfig("t", d=8, n_layers=2, n_heads=1, n_kv_heads=1, head_dim=4, ffn=8, vocab=16)
    r = np.random.default_rng(13)
    E = r.standard_normal((cfg.vocab, cfg.d))
    H = r.standard_normal((cfg.vocab, cfg.d))
    qkv = np.zeros((cfg.n_qkv, cfg.d))
    qkv[0:4] = r.standard_normal((4, 8))
    qkv[4, 1] = 1.0
    qkv[8:12, :4] = np.eye(4)
    zeros_o = np.zeros((cfg.d, cfg.q_dim))
    M = oracle.Model(_weights_from(cfg, E, H, [qkv, qkv], [zeros_o, zeros_o],
                                   [np.zeros((16, 8))] * 2, [np.zeros((8, 8))] * 2))
    toks = [1, 4, 4, 11, 6]
    lane = M.lane(8)
    for tok in toks:
        M.step(lane, tok)
    K, V = lane.get_kv()
    assert K.shape == (2, 1, len(toks), 4)
    for p, tok in enumerate(toks):
        xn = _rms64(E[tok].astype(np.float32), cfg.rms_eps)  # residual unchanged: W_o = W_down = 0
        for l in range(2):
            assert np.allclose(K[l, 0, p], xn[1] * np.array([math.cos(p), 0, math.sin(p), 0]), atol=2e-6)
            assert np.allclose(V[l, 0, p], xn[:4], atol=2e-6)


def test_bf16_mode_rounds_projection_inputs_and_kv():
    # Zero projections in bf16 mode: logits = head @ bf16(rmsnorm(E[tok])); stored K/V
    # are bf16 values.
    cfg = ModelConfig("t", d=32, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=16, ffn=32, vocab=24,
                      wtype=WTYPE_BF16)
    r = np.random.default_rng(14)
    Eb = synth.f32_to_bf16(r.standard_normal((cfg.vocab, cfg.d)).astype(np.float32))
    Hb = synth.f32_to_bf16((0.1 * r.standard_normal((cfg.vocab, cfg.d))).astype(np.float32))
    qkvb = synth.f32_to_bf16(r.standard_normal((cfg.n_qkv, cfg.d)).astype(np.float32))
    zo = np.zeros((cfg.d, cfg.q_dim), np.uint16)
    zgu = synth.f32_to_bf16(r.standard_normal((2 * cfg.ffn, cfg.d)).astype(np.float32))
    zd = np.zeros((cfg.d, cfg.ffn), np.uint16)
    W = Weights(cfg=cfg, embed=Matrix(WTYPE_BF16, Eb), lm_head=Matrix(WTYPE_BF16, Hb),
                final_norm=np.ones(cfg.d, np.float32))
    for l in range(cfg.n_layers):
        W.attn_norm.append(np.ones(cfg.d, np.float32))
        W.ffn_norm.append(np.ones(cfg.d, np.float32))
        W.w_qkv.append(Matrix(WTYPE_BF16, qkvb))
        W.w_o.append(Matrix(WTYPE_BF16, zo))
        W.w_gu.append(Matrix(WTYPE_BF16, zgu))
        W.w_down.append(Matrix(WTYPE_BF16, zd))
    M = oracle.Model(W)
    up = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    lane = M.lane(4)
    for tok in [2, 7, 19]:
        lg = M.step(lane, tok)
        xn = _rms64(up(Eb[tok]), cfg.rms_eps).astype(np.float32)
        # independent round-to-nearest-even to bf16 by integer arithmetic
        u = xn.view(np.uint32).astype(np.uint64)
        xnb = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)
        ref = up(Hb).astype(np.float64) @ xnb.astype(np.float64)
        assert _rel(lg, ref) < 2e-6
    K, V = lane.get_kv()
    assert np.all((K.view(np.uint32) & 0xFFFF) == 0) and np.all((V.view(np.uint32) & 0xFFFF) == 0)


# ---- the pages' invariants -----------------------------------------------------------

SMALL_GQA = ModelConfig("small-gqa", d=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=32, ffn=96,
                        vocab=300)


@pytest.mark.parametrize("cfg", [synth.TINY, SMALL_GQA, SMALL_GQA.with_wtype(WTYPE_BF16),
                                 SMALL_GQA.with_wtype(WTYPE_Q8_0)], ids=lambda c: "%s-%d" % (c.name, c.wtype))
def test_batched_step_is_bitwise_serial_logits_and_kv(cfg):
    W = synth.make_weights(cfg)
    M = oracle.Model(W)
    plens = [3, 5, 7, 9]
    prompts = [synth.prompt_tokens(cfg, b, n) for b, n in enumerate(plens)]
    max_seq = 16
    # serial: each lane alone
    ser_lanes = [M.lane(max_seq) for _ in plens]
    ser_logits = [[M.step(ser_lanes[b], t) for t in prompts[b]] for b in range(4)]
    # batched: lockstep over the lanes still feeding
    bat_lanes = [M.lane(max_seq) for _ in plens]
    bat_logits = [[] for _ in plens]
    for s in range(max(plens)):
        live = [b for b in range(4) if s < plens[b]]
        lg = M.step_batch([bat_lanes[b] for b in live], [prompts[b][s] for b in live])
        for i, b in enumerate(live):
            bat_logits[b].append(lg[i])
    for b in range(4):
        for s in range(plens[b]):
            assert np.array_equal(ser_logits[b][s].view(np.uint32), bat_logits[b][s].view(np.uint32))
        ks, vs = ser_lanes[b].get_kv()
        kb, vb = bat_lanes[b].get_kv()
        assert ks.shape[2] == plens[b]
        assert np.array_equal(ks.view(np.uint32), kb.view(np.uint32))
        assert np.array_equal(vs.view(np.uint32), vb.view(np.uint32))


def test_lockstep_greedy_equals_serial_generation_tiny():
    cfg = synth.TINY
    M = oracle.Model(synth.make_weights(cfg))
    prompts = [synth.prompt_tokens(cfg, b, n) for b, n in enumerate([3, 5, 7, 9])]
    lock = oracle.generate_lockstep(M, prompts, 8)
    ser = [oracle.generate(M, p, 8) for p in prompts]
    assert lock == ser
    assert all(len(g) == 8 for g in lock)


def test_positions_isolated_across_prompt_lengths_1_3_7():
    cfg = SMALL_GQA
    M = oracle.Model(synth.make_weights(cfg))
    prompts = [synth.prompt_tokens(cfg, 10 + b, n) for b, n in enumerate([1, 3, 7])]
    gen_l, logs_l = oracle.generate_lockstep(M, prompts, 5, return_logits=True)
    for b, p in enumerate(prompts):
        gen_s, logs_s = oracle.generate(M, p, 5, return_logits=True)
        assert gen_s == gen_l[b]
        assert len(logs_s) == len(p) + 5 - 1
        for a, c in zip(logs_s, logs_l[b]):
            assert np.array_equal(a, c)


def test_cleared_lane_behaves_like_a_fresh_lane():
    cfg = SMALL_GQA
    M = oracle.Model(synth.make_weights(cfg))
    a = synth.prompt_tokens(cfg, 20, 6)
    b = synth.prompt_tokens(cfg, 21, 4)
    used = M.lane(12)
    for t in a:
        M.step(used, t)
    used.clear()
    assert used.length == 0
    fresh = M.lane(12)
    for t in b:
        assert np.array_equal(M.step(used, t), M.step(fresh, t))


def test_lane_full_and_bad_token_are_rejected():
    cfg = synth.TINY
    M = oracle.Model(synth.make_weights(cfg))
    lane = M.lane(2)
    M.step(lane, 1)
    M.step(lane, 2)
    with pytest.raises(ValueError):
        M.step(lane, 3)
    with pytest.raises(ValueError):
        M.step(M.lane(2), cfg.vocab)
    l1 = M.lane(4)
    with pytest.raises(ValueError):
        M.step_batch([l1, l1], [1, 2])


def test_q8_0_oracle_is_faithful_to_f32_oracle():
    # The Q8_0 model quantises the same f32 draws; its logits stay close to the f32
    # model's (the pages report mean cosine 0.99939 on a trained model).
    cfg = SMALL_GQA
    Mf = oracle.Model(synth.make_weights(cfg, wtype=WTYPE_F32))
    Mq = oracle.Model(synth.make_weights(cfg.with_wtype(WTYPE_Q8_0)))
    prompt = synth.prompt_tokens(cfg, 30, 8)
    lf, lq = Mf.lane(8), Mq.lane(8)
    cos = []
    for t in prompt:
        a, b = Mf.step(lf, t).astype(np.float64), Mq.step(lq, t).astype(np.float64)
        cos.append(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
    assert min(cos) > 0.999


def test_f32_accumulation_build_is_the_same_definition():
    # The accumulate="f32" build differs from the exact-sum oracle only by the
    # rounding of its sums: on a small f32 model the logits agree to ~1e-6, and
    # the two builds are not bit-identical (the flag took effect).
    cfg = synth.TINY
    W = synth.make_weights(cfg)
    prompts = [synth.prompt_tokens(cfg, b, n) for b, n in enumerate([3, 5])]
    exact = oracle.generate_lockstep(oracle.Model(W), prompts, 4, return_logits=True)
    f32 = oracle.generate_lockstep(oracle.Model(W, accumulate="f32"), prompts, 4, return_logits=True)
    assert exact[0] == f32[0]
    worst, same = 0.0, True
    for la, lb in zip(exact[1], f32[1]):
        for x, y in zip(la, lb):
            worst = max(worst, float(np.max(np.abs(x - y)) / np.max(np.abs(x))))
            same = same and np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert worst < 1e-5
    assert not same


# ---- the SwiGLU block and the three norm gains ------------------------------------------

def _ffn_weights(cfg, r, gates, ups, outs, sg, su, gains, swap=False):
    """Special weights whose decode step has a closed form (d = 8, Hq = 2, Hkv = 1, hd = 4,
    F = 4).  Wq = 0, so every score is 0 and attention is the plain mean of the values; Wv
    selects four entries of the attention-normalised input (layer l: xa[4l .. 4l+3]); Wo
    is 0.5 x a permutation; hidden unit j takes gate = sg * xf[gates[j]] and up =
    su * xf[ups[j]] from the FFN-normalised input, and W_down adds unit j into
    x[outs[j]].  swap=True stores the up rows where the gate rows belong and vice versa."""
    d, F, L = cfg.d, cfg.ffn, cfg.n_layers
    E = r.standard_normal((cfg.vocab, d))
    H = r.standard_normal((cfg.vocab, d))
    qkv, o, gu, down, perms = [], [], [], [], []
    for l in range(L):
        w = np.zeros((cfg.n_qkv, d))
        w[8:12] = r.standard_normal((4, d))  # key rows: any values, the scores stay 0
        for i in range(4):
            w[12 + i, 4 * l + i] = 1.0
        qkv.append(w)
        p = r.permutation(d)
        perms.append(p)
        wo = np.zeros((d, cfg.q_dim))
        wo[np.arange(d), p] = 0.5
        o.append(wo)
        g = np.zeros((2 * F, d))
        for j in range(F):
            g[j, gates[j]] = sg
            g[F + j, ups[j]] = su
        if swap:
            g = np.concatenate([g[F:], g[:F]])
        gu.append(g)
        wd = np.zeros((d, F))
        for j in range(F):
            wd[outs[j], j] = 1.0
        down.append(wd)
    W = _weights_from(cfg, E, H, qkv, o, gu, down)
    ga, gf, gfin = gains
    W.attn_norm[:] = [np.ascontiguousarray(a, np.float32) for a in ga]
    W.ffn_norm[:] = [np.ascontiguousarray(a, np.float32) for a in gf]
    W.final_norm = np.ascontiguousarray(gfin, np.float32)
    return W, E.astype(np.float32).astype(np.float64), H.astype(np.float32).astype(np.float64), perms


def _ffn_closed_form(cfg, E, H, perms, gains, toks, gates, ups, outs, sg, su, silu_on="gate",
                     ffn_residual=True):
    """Logits of each step of one lane under the special weights of _ffn_weights, in f64.
    silu_on / ffn_residual describe plausible mistakes, for the negative checks."""
    ga, gf, gfin = [[np.asarray(g, np.float32).astype(np.float64) for g in gs] for gs in gains[:2]] + \
        [np.asarray(gains[2], np.float32).astype(np.float64)]
    eps = cfg.rms_eps
    silu = lambda u: u / (1.0 + math.exp(-u))
    hist = [[] for _ in range(cfg.n_layers)]
    res = []
    for tok in toks:
        x = E[tok].copy()
        for l in range(cfg.n_layers):
            xa = _rms64(x, eps) * ga[l]
            hist[l].append(xa[4 * l:4 * l + 4])
            m = np.mean(hist[l], axis=0)           # uniform attention: mean of the values
            o = np.concatenate([m, m])             # both query heads read the one KV head
            upd = np.zeros(cfg.d)
            upd[np.arange(cfg.d)] = 0.5 * o[perms[l]]
            x = x + upd
            xf = _rms64(x, eps) * gf[l]
            add = np.zeros(cfg.d)
            for j in range(cfg.ffn):
                g, u = sg * xf[gates[j]], su * xf[ups[j]]
                add[outs[j]] += silu(g) * u if silu_on == "gate" else silu(u) * g
            x = x + add if ffn_residual else add
        res.append(H @ (_rms64(x, eps) * gfin))
    return res


FFN_CFG = ModelConfig("ffn-pin", d=8, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=4, ffn=4, vocab=16)
FFN_GATES, FFN_UPS, FFN_OUTS = [0, 3, 5, 6], [2, 7, 1, 4], [1, 4, 6, 3]


def _ffn_gains(r, cfg):
    ga = [0.5 + r.random(cfg.d) for _ in range(cfg.n_layers)]
    gf = [0.5 + r.random(cfg.d) for _ in range(cfg.n_layers)]
    return ga, gf, 0.5 + r.random(cfg.d)


@pytest.mark.parametrize("batched", [False, True])
def test_swiglu_block_and_norm_gains_have_their_closed_form(batched):
    # x_out = x + W_down (silu(W_g xf) * (W_u xf)) with xf the FFN-normalised input times
    # that layer's FFN gain; attention reads the attention-normalised input times that
    # layer's attention gain; the head reads the final-normalised state times the final gain.
    cfg = FFN_CFG
    r = np.random.default_rng(21)
    gains = _ffn_gains(r, cfg)
    sg, su = 3.0, 2.0
    W, E, H, perms = _ffn_weights(cfg, r, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su, gains)
    M = oracle.Model(W)
    toks = [5, 11, 5, 0, 14, 9]
    if batched:
        lanes = [M.lane(8), M.lane(8)]
        got = [M.step_batch(lanes, [t, toks[0]])[0] for t in toks]
    else:
        lane = M.lane(8)
        got = [M.step(lane, t) for t in toks]
    want = _ffn_closed_form(cfg, E, H, perms, gains, toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su)
    for p in range(len(toks)):
        assert _rel(got[p], want[p]) < 1e-5, p
    # The pin rejects the plausible mistakes: each alternative closed form is far from
    # what the oracle computes.
    alts = {
        "silu on the up rows": _ffn_closed_form(cfg, E, H, perms, gains, toks, FFN_GATES, FFN_UPS, FFN_OUTS,
                                                sg, su, silu_on="up"),
        "no FFN residual": _ffn_closed_form(cfg, E, H, perms, gains, toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su,
                                            ffn_residual=False),
        "attention and FFN gains exchanged": _ffn_closed_form(
            cfg, E, H, perms, (gains[1], gains[0], gains[2]), toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su),
        "final gain = last FFN gain": _ffn_closed_form(
            cfg, E, H, perms, (gains[0], gains[1], gains[1][-1]), toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su),
        "layers' gains in reverse": _ffn_closed_form(
            cfg, E, H, perms, (gains[0][::-1], gains[1][::-1], gains[2]), toks, FFN_GATES, FFN_UPS, FFN_OUTS,
            sg, su),
    }
    for name, alt in alts.items():
        assert max(_rel(got[p], alt[p]) for p in range(len(toks))) > 1e-3, name


def test_gate_and_up_rows_are_not_interchangeable():
    # Storing the up rows first (the gate/up order reversed) must give the closed form
    # with silu on what is now the second half, a different result.
    cfg = FFN_CFG
    r = np.random.default_rng(22)
    gains = _ffn_gains(r, cfg)
    sg, su = 3.0, 2.0
    W, E, H, perms = _ffn_weights(cfg, r, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su, gains, swap=True)
    M = oracle.Model(W)
    toks = [3, 8, 15, 1]
    lane = M.lane(8)
    got = [M.step(lane, t) for t in toks]
    swapped = _ffn_closed_form(cfg, E, H, perms, gains, toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su,
                               silu_on="up")
    plain = _ffn_closed_form(cfg, E, H, perms, gains, toks, FFN_GATES, FFN_UPS, FFN_OUTS, sg, su)
    for p in range(len(toks)):
        assert _rel(got[p], swapped[p]) < 1e-5, p
    assert max(_rel(got[p], plain[p]) for p in range(len(toks))) > 1e-3
