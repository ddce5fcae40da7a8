"""The Q8_0 path at the SmolLM2-135M shape: 16-token prompts, 12 greedy decode
steps, B in {1, 64, 256, 512, 960} lanes in lockstep.

The gate ("Correctness — proven, not asserted" on "MODEL-BATCHING-RESULTS —
multi-user batched decode, measured": Q8 batched decode keeps the decisive
first-token argmax of the f32 model and near-f32 teacher-forced agreement):

* first generated token of a lane == the f32 oracle's, on every sampled lane
  whose f32 top-1/top-2 margin is decisive, i.e. exceeds 3*sqrt(2) x the RMS
  of that lane's (Q8 - f32) logit difference at that step (a margin the
  quantisation noise cannot close); the rest are counted and reported;
* teacher-forced over every step of the sampled lanes: mean logit cosine
  against the f32 oracle >= 0.999 and top-1 agreement >= 80%;
* against the Q8_0 oracle (same quantised weights, f32 activations): max
  relative error <= 2e-2 and cosine > 0.9999 (the kernel computes in binary16
  operands: weights dequantised as q * scale, activations rounded);
* lane b's tokens and logits are bit-identical at every B.

Oracle cost bounds the sample: 64 lanes spread over [0, 960) for the first
token (f32 oracle, lockstep over the prompt), six lanes teacher-forced at
every step.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, engine_for, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BATCHES = [1, 64, 256, 512, 960]
N_PROMPT, N_NEW = 16, 12
FIRST_LANES = sorted(set(np.linspace(0, 959, 64).astype(int).tolist()))
TF_LANES = [0, 63, 255, 300, 511, 959]


def _cos(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _teacher_forced(M, seqs):
    """Oracle logits of every step for lanes fed the given token sequences (equal lengths)."""
    lanes = [M.lane(len(s)) for s in seqs]
    out = [[] for _ in seqs]
    for t in range(len(seqs[0])):
        lg = M.step_batch(lanes, [int(s[t]) for s in seqs])
        for i in range(len(seqs)):
            out[i].append(lg[i])
    return out


def test_q8_0_135m_gate():
    from continuous_batching_decode_step_amd.driver import generate_lockstep
    cfgq = synth.SMOL135M_Q8
    say("Q8: weights")
    Wq = synth.make_weights(cfgq)
    prompts = [synth.prompt_tokens(cfgq, b, N_PROMPT) for b in range(max(BATCHES))]
    eng = engine_for(cfgq, Wq, max(BATCHES), N_PROMPT + N_NEW, max(BATCHES))
    sample = set(FIRST_LANES) | set(TF_LANES)
    first_step = N_PROMPT - 1  # the step that feeds the last prompt token yields the first token
    seen = {}
    for B in BATCHES:
        say("Q8: B=%d" % B)
        keep = lambda b, i: b in sample and (i == first_step or b in TF_LANES)
        gen, logs = generate_lockstep(eng, prompts[:B], N_NEW, want_logits=keep)
        for b in range(B):
            if b not in sample:
                continue
            if b in seen:  # the same lane at a narrower step: same bits
                g0, l0 = seen[b]
                assert g0 == gen[b], (b, B)
                for x, y in zip(l0, logs[b]):
                    if x is not None:
                        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), (b, B)
            else:
                seen[b] = (gen[b], logs[b])
    del eng

    # first token against the f32 oracle on the sampled lanes
    W32 = synth.make_weights(cfgq, wtype=synth.WTYPE_F32)
    M32 = oracle.Model(W32)
    say("Q8: f32 oracle over %d prompts" % len(FIRST_LANES))
    ref = _teacher_forced(M32, [prompts[b] for b in FIRST_LANES])
    decisive = agree = 0
    for i, b in enumerate(FIRST_LANES):
        o = np.asarray(ref[i][first_step], np.float64)
        g = np.asarray(seen[b][1][first_step], np.float64)
        s = np.sort(o)
        margin = s[-1] - s[-2]
        noise = np.sqrt(np.mean((g - o) ** 2))
        gpu_tok = seen[b][0][0]
        assert gpu_tok == int(np.argmax(g))
        if margin > 3 * np.sqrt(2) * noise:
            decisive += 1
            assert gpu_tok == int(np.argmax(o)), "lane %d: decisive first token differs" % b
        agree += gpu_tok == int(np.argmax(o))
    say("Q8: first token: %d/%d sampled lanes decisive (all match), %d/%d agree overall" % (
        decisive, len(FIRST_LANES), agree, len(FIRST_LANES)))
    assert decisive >= 8  # the gate is not vacuous

    # teacher-forced on every step of a few lanes, against the f32 and the Q8_0 oracle
    seqs = [list(prompts[b]) + list(seen[b][0][:-1]) for b in TF_LANES]
    say("Q8: teacher-forced f32 and Q8_0 oracles, lanes %s" % TF_LANES)
    r32 = _teacher_forced(M32, seqs)
    del M32, W32
    rq = _teacher_forced(oracle.Model(Wq), seqs)
    cos32, top1, n_gen, worst_q, cos_q = [], 0, 0, 0.0, 1.0
    for i, b in enumerate(TF_LANES):
        for t, g in enumerate(seen[b][1]):
            cos32.append(_cos(g, r32[i][t]))
            worst_q = max(worst_q, rel_err(g, rq[i][t]))
            cos_q = min(cos_q, _cos(g, rq[i][t]))
            if t >= first_step:
                n_gen += 1
                top1 += int(np.argmax(g)) == int(np.argmax(r32[i][t]))
    say("Q8: vs f32 oracle mean cos %.5f, top-1 %d/%d; vs Q8_0 oracle max rel %.3g, min cos %.6f" % (
        np.mean(cos32), top1, n_gen, worst_q, cos_q))
    assert np.mean(cos32) >= 0.999
    assert top1 >= 0.8 * n_gen
    assert worst_q <= TOL_BF16 and cos_q > 0.9999
