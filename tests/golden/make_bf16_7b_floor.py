"""Write bf16_7b_floor.json: how far a plain f32-accumulating evaluation of the
decode step drifts from the exact-sum oracle at the Mistral-7B shape in bf16.

Workload (the full-size GPU parity test's): seeded weights (seed 0), 64 lanes
with KV lengths uniform in [128, 4096] (seed 2), synthetic post-rotary K/V
(seed 3), the step's input tokens (seed 1); one decode step on each sampled
lane.  Both evaluations are the CPU oracle (oracle/): the default build sums
in double, the accumulate="f32" build in f32; everything else, including
every bf16 rounding point, is the same code.  The bf16 activations turn tiny
accumulation differences into flipped roundings, which grow through the 32
layers; the figures recorded per lane are the max relative logit difference
(max |a - b| / max |a|), the relative l2 difference, and the max relative
difference of the K and V the step appends (slot kv_len), over all layers
and for layer 0 alone.

Run from the repository root:  python tests/golden/make_bf16_7b_floor.py
(about 10 minutes and 40 GB of host memory).
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

SAMPLE = [0, 2, 4, 7, 14, 24, 40, 63]  # the full-size GPU parity test's sampled lanes


def main():
    cfg = synth.MISTRAL7B
    t0 = time.time()
    W = synth.make_weights(cfg)
    print("weights %.0fs" % (time.time() - t0), flush=True)
    lens = synth.kv_lengths(64)
    toks = synth.step_tokens(cfg, 64)
    exact, f32 = oracle.Model(W), oracle.Model(W, accumulate="f32")
    out = {}
    for b in SAMPLE:
        n = int(lens[b])
        k, v = synth.lane_kv_bf16(cfg, b, n)
        kf, vf = synth.bf16_to_f32(k), synth.bf16_to_f32(v)
        res, kvs = [], []
        for M in (exact, f32):
            lane = M.lane(n + 1)
            lane.set_kv(kf, vf)
            res.append(M.step(lane, int(toks[b])).astype(np.float64))
            ok, ov = lane.get_kv()
            kvs.append((ok[:, :, n].astype(np.float64), ov[:, :, n].astype(np.float64)))
            del lane
        a, c = res
        rel = lambda x, y: float(np.max(np.abs(x - y)) / np.max(np.abs(x)))
        out[str(b)] = {"kv_len": n, "token": int(toks[b]),
                       "max_rel": float(np.max(np.abs(a - c)) / np.max(np.abs(a))),
                       "l2_rel": float(np.linalg.norm(a - c) / np.linalg.norm(a)),
                       "argmax_exact": int(np.argmax(a)), "argmax_f32": int(np.argmax(c)),
                       "k_new_max_rel": rel(kvs[0][0], kvs[1][0]), "v_new_max_rel": rel(kvs[0][1], kvs[1][1]),
                       "k_new_layer0_max_rel": rel(kvs[0][0][0], kvs[1][0][0]),
                       "v_new_layer0_max_rel": rel(kvs[0][1][0], kvs[1][1][0])}
        print("lane %d: %s" % (b, out[str(b)]), flush=True)
    doc = {"what": "exact-sum oracle vs f32-accumulating oracle, Mistral-7B shape bf16, one decode step",
           "command": "python tests/golden/make_bf16_7b_floor.py", "lanes": out}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "bf16_7b_floor.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
