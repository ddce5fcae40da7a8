"""Pins of the oracle's pieces to closed forms, special cases, brute force and
independent number-format implementations (numpy's binary16, bit shifts).

Each test names the mistake it is there to catch.  None of these re-types the
oracle's own formula and compares it with itself: the expected values come
from the mathematics (identities, special inputs with known answers) or from
an independent implementation of a number format.
"""
import math

import numpy as np
import pytest

import oracle
import synth

EPS32 = 2.0 ** -24


def _rng(seed):
    return np.random.default_rng(seed)


# ---- number formats ---------------------------------------------------------------

def test_f16_decode_matches_numpy_binary16_all_patterns():
    # Catches a wrong exponent bias, a missing subnormal branch or a sign error in the
    # Q8_0 scale decode: numpy's float16 is an independent binary16 implementation.
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isinf(got[np.isinf(ref)])) and np.all(np.isnan(got[np.isnan(ref)]))


def test_round_bf16_properties():
    # bf16 values are fixed points; otherwise the result is one of the two bf16
    # neighbours, the nearer one, with exact ties going to the even neighbour.
    r = _rng(1)
    x = r.standard_normal(5000).astype(np.float32)
    xb = synth.bf16_to_f32(synth.f32_to_bf16(x))  # bf16-representable values
    for v in xb[:200]:
        assert oracle.round_bf16(float(v)) == v
    for v in x[:500]:
        u = np.float32(v).view(np.uint32)
        lo = np.uint32(u & 0xFFFF0000).view(np.float32)
        hi = np.uint32((u & 0xFFFF0000) + 0x10000).view(np.float32)
        got = np.float32(oracle.round_bf16(float(v)))
        assert got in (lo, hi)
        assert abs(float(got) - float(v)) <= min(abs(float(lo) - float(v)), abs(float(hi) - float(v)))
    # exact ties: bf16 value with mantissa lsb 0 / 1, plus half an ulp
    even = np.uint32(0x3F800000).view(np.float32)  # 1.0, lsb even
    tie_up = np.uint32(0x3F808000).view(np.float32)  # 1.0 + half ulp -> 1.0 (even)
    assert oracle.round_bf16(float(tie_up)) == float(even)
    odd = np.uint32(0x3F810000).view(np.float32)
    tie_odd = np.uint32(0x3F818000).view(np.float32)  # odd + half ulp -> next even (0x3F820000)
    assert np.float32(oracle.round_bf16(float(tie_odd))).view(np.uint32) == 0x3F820000
    assert oracle.round_bf16(float(odd)) == float(odd)


# ---- projections --------------------------------------------------------------------

def _dot_bound(W64, x64):
    K = W64.shape[1]
    return 1.01 * K * EPS32 * (np.abs(W64) @ np.abs(x64)) + 1e-30


@pytest.mark.parametrize("K", [172, 576, 1000])
def test_matvec_f32_within_rounding_bound_of_f64(K):
    # Catches a transposed operand, a wrong row offset or a dropped term: the f32
    # in-order dot must sit within K*2^-24*sum|w||x| of the exact f64 product.
    r = _rng(K)
    W = (0.02 * r.standard_normal((37, K))).astype(np.float32)
    x = r.standard_normal(K).astype(np.float32)
    y = oracle.matvec(W, x)
    ref = W.astype(np.float64) @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= _dot_bound(W.astype(np.float64), x.astype(np.float64)))
    # row offset: rows [5, 17)
    y2 = oracle.matvec(W, x, row0=5, nrows=12)
    assert np.array_equal(y2, y[5:17])


def test_matvec_bf16_upcasts_exactly():
    r = _rng(2)
    Wf = (0.02 * r.standard_normal((19, 256))).astype(np.float32)
    Wb = synth.f32_to_bf16(Wf)
    W64 = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # independent upcast
    x = r.standard_normal(256).astype(np.float32)
    y = oracle.matvec(Wb, x, wtype=oracle.ORC_BF16)
    ref = W64 @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= _dot_bound(W64, x.astype(np.float64)))


def test_matvec_q8_0_dequantises_per_block_of_32():
    # Catches a scale indexed by the wrong block (i instead of i/32) or by the wrong row.
    r = _rng(3)
    K = 128
    q = r.integers(-127, 128, size=(9, K)).astype(np.int8)
    s = (r.uniform(0.5, 2.0, size=(9, K // 32)) * 1e-3).astype(np.float16)
    W64 = q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)
    x = r.standard_normal(K).astype(np.float32)
    y = oracle.matvec(q, x, wtype=oracle.ORC_Q8_0, scale=s.view(np.uint16))
    ref = W64 @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= _dot_bound(W64, x.astype(np.float64)))
    # one block's scale changed moves only the outputs of that row
    s2 = s.copy()
    s2[4, 2] *= 2
    y2 = oracle.matvec(q, x, wtype=oracle.ORC_Q8_0, scale=s2.view(np.uint16))
    changed = np.nonzero(y2 != y)[0]
    assert list(changed) == [4]


# ---- RMSNorm, SiLU -----------------------------------------------------------------

@pytest.mark.parametrize("c", [0.5, 1.0, 3.0, -2.0])
def test_rmsnorm_constant_vector_closed_form(c):
    # rmsnorm(c * 1) = c / sqrt(c^2 + eps) * g
    n, eps = 64, 1e-5
    g = np.linspace(0.5, 1.5, n).astype(np.float32)
    out = oracle.rmsnorm(np.full(n, c, np.float32), g, eps)
    ref = c / math.sqrt(c * c + eps) * g.astype(np.float64)
    assert np.allclose(out, ref, rtol=4e-7, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    # With eps -> 0 the output has unit mean square and ignores the input scale;
    # catches a mean replaced by a sum or a missing square root.
    r = _rng(4)
    x = r.standard_normal(576).astype(np.float32)
    g = np.ones(576, np.float32)
    out = oracle.rmsnorm(x, g, 1e-30)
    assert abs(float(np.mean(out.astype(np.float64) ** 2)) - 1.0) < 1e-5
    out2 = oracle.rmsnorm(8.0 * x, g, 1e-30)
    assert np.allclose(out, out2, rtol=1e-6)


def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    for u in [0.1, 0.7, 1.3, 2.9, 5.0]:
        # silu(u) - silu(-u) = u (sigmoid(u) + sigmoid(-u) = 1)
        assert abs((oracle.silu(u) - oracle.silu(-u)) - u) < 4e-7 * max(1.0, u)
        # silu(u) = u * sigmoid(u) with sigmoid(u) = 1/(1+e^-u)
        assert abs(oracle.silu(u) - u / (1 + math.exp(-u))) < 2e-7 * max(1.0, u)
    assert abs(oracle.silu(30.0) - 30.0) < 1e-5 and abs(oracle.silu(-30.0)) < 1e-10


# ---- rotary positions ------------------------------------------------------------

def test_rope_position_zero_is_identity():
    v = _rng(5).standard_normal(128).astype(np.float32)
    assert np.array_equal(oracle.rope(v, 0, 10000.0), v)


def test_rope_pairing_and_frequencies_special_vectors():
    # Rotate-half pairing (j, j + hd/2); theta_0 = 1 (angle = pos), theta_{hd/4} = theta^-1/2.
    hd, pos, theta = 8, 3, 10000.0
    e0 = np.zeros(hd, np.float32)
    e0[0] = 1
    out = oracle.rope(e0, pos, theta)
    exp = np.zeros(hd)
    exp[0], exp[hd // 2] = math.cos(3.0), math.sin(3.0)
    assert np.allclose(out, exp, atol=1e-7)
    e_half = np.zeros(hd, np.float32)
    e_half[hd // 2] = 1  # second member of pair 0 -> (-sin, cos)
    out = oracle.rope(e_half, pos, theta)
    exp = np.zeros(hd)
    exp[0], exp[hd // 2] = -math.sin(3.0), math.cos(3.0)
    assert np.allclose(out, exp, atol=1e-7)
    e2 = np.zeros(hd, np.float32)
    e2[hd // 4] = 1  # pair j = hd/4: angle = pos * theta^(-1/2) = 0.03
    out = oracle.rope(e2, pos, theta)
    exp = np.zeros(hd)
    exp[hd // 4], exp[hd // 4 + hd // 2] = math.cos(0.03), math.sin(0.03)
    assert np.allclose(out, exp, atol=1e-7)
    c, s = oracle.rope_cs(hd, pos, theta)
    assert abs(c[0] - math.cos(3.0)) < 1e-7 and abs(s[0] - math.sin(3.0)) < 1e-7


def test_rope_preserves_pair_norms_and_relative_dot():
    r = _rng(6)
    hd, theta = 64, 10000.0
    q = r.standard_normal(hd).astype(np.float32)
    k = r.standard_normal(hd).astype(np.float32)
    for p in (1, 17, 1000, 4095):
        rq = oracle.rope(q, p, theta).astype(np.float64)
        n_in = q[:hd // 2].astype(np.float64) ** 2 + q[hd // 2:].astype(np.float64) ** 2
        n_out = rq[:hd // 2] ** 2 + rq[hd // 2:] ** 2
        assert np.allclose(n_in, n_out, rtol=1e-5)
    # <R_a q, R_b k> depends on a - b only
    d1 = float(np.dot(oracle.rope(q, 10, theta).astype(np.float64), oracle.rope(k, 3, theta)))
    d2 = float(np.dot(oracle.rope(q, 107, theta).astype(np.float64), oracle.rope(k, 100, theta)))
    d0 = float(np.dot(oracle.rope(q, 7, theta).astype(np.float64), k))
    assert abs(d1 - d2) < 1e-4 and abs(d1 - d0) < 1e-4


# ---- attention ----------------------------------------------------------------------

def test_attention_single_key_returns_v_exactly():
    r = _rng(7)
    Hq, Hkv, hd = 6, 2, 16
    q = r.standard_normal(Hq * hd).astype(np.float32)
    K = r.standard_normal((1, Hkv * hd)).astype(np.float32)
    V = r.standard_normal((1, Hkv * hd)).astype(np.float32)
    out = oracle.attention(q, K, V, Hq, Hkv, hd).reshape(Hq, hd)
    Vh = V.reshape(Hkv, hd)
    for h in range(Hq):
        assert np.array_equal(out[h], Vh[h // (Hq // Hkv)])


def test_attention_gqa_head_mapping_contiguous_groups():
    # Query heads 0..2 read KV head 0, heads 3..5 read KV head 1 (not h % Hkv).
    Hq, Hkv, hd, n = 6, 2, 8, 5
    r = _rng(8)
    q = r.standard_normal(Hq * hd).astype(np.float32)
    K = r.standard_normal((n, Hkv * hd)).astype(np.float32)
    V = np.zeros((n, Hkv * hd), np.float32)
    V[:, :hd] = 1.0
    V[:, hd:] = 2.0
    out = oracle.attention(q, K, V, Hq, Hkv, hd).reshape(Hq, hd)
    assert np.allclose(out[:3], 1.0, atol=1e-6) and np.allclose(out[3:], 2.0, atol=1e-6)


def test_attention_identical_keys_give_mean_of_values():
    Hq, Hkv, hd, n = 4, 4, 16, 9
    r = _rng(9)
    q = r.standard_normal(Hq * hd).astype(np.float32)
    K = np.tile(r.standard_normal((1, Hkv * hd)).astype(np.float32), (n, 1))
    V = r.standard_normal((n, Hkv * hd)).astype(np.float32)
    out = oracle.attention(q, K, V, Hq, Hkv, hd)
    assert np.allclose(out, V.astype(np.float64).mean(0), atol=1e-6)


def test_attention_two_key_closed_form_with_sqrt_hd_scale():
    # q = a e0, K0 = e0, K1 = 0: weights e^{a/sqrt(hd)} : 1.  Catches a missing or
    # wrong score scale.
    hd, a = 16, 3.0
    q = np.zeros(hd, np.float32)
    q[0] = a
    K = np.zeros((2, hd), np.float32)
    K[0, 0] = 1.0
    V = np.zeros((2, hd), np.float32)
    V[0, :], V[1, :] = 1.0, -1.0
    out = oracle.attention(q, K, V, 1, 1, hd)
    w = math.exp(a / math.sqrt(hd))
    assert np.allclose(out, (w - 1) / (w + 1), atol=1e-6)


@pytest.mark.parametrize("shape", [(4, 2, 8, 7), (3, 1, 16, 13), (2, 2, 4, 1)])
def test_attention_matches_brute_force_f64(shape):
    Hq, Hkv, hd, n = shape
    r = _rng(sum(shape))
    q = r.standard_normal(Hq * hd).astype(np.float32)
    K = r.standard_normal((n, Hkv * hd)).astype(np.float32)
    V = r.standard_normal((n, Hkv * hd)).astype(np.float32)
    out = oracle.attention(q, K, V, Hq, Hkv, hd).reshape(Hq, hd)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        kh = K[:, g * hd:(g + 1) * hd].astype(np.float64)
        vh = V[:, g * hd:(g + 1) * hd].astype(np.float64)
        s = kh @ q[h * hd:(h + 1) * hd].astype(np.float64) / math.sqrt(hd)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(out[h], p @ vh, atol=2e-6)


def test_argmax_lowest_index_wins_ties():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([5.0, 5.0]) == 0
    assert oracle.argmax([-1.0, -0.5, -0.5]) == 1
