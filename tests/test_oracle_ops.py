"""Pins of the oracle's elementary operations against closed forms, invariants and brute force.

None of these re-types an oracle formula: each checks a property the definition
implies (a special case with a known answer, an algebraic identity, an
invariant) or compares with an independent brute-force evaluation."""
import math

import numpy as np
import pytest

from oracle import ops


rng = np.random.default_rng(1234)


def unit(x):
    return x / np.linalg.norm(x)


# ----------------------------------------------------------------------------- bf16 rounding
def test_round_bf16_known_values():
    one = 1.0
    half_ulp = 2.0 ** -8          # bf16 keeps 7 mantissa bits: ulp(1) = 2^-7
    assert ops.round_bf16(np.array([one]))[0] == 1.0
    assert ops.round_bf16(np.array([one + half_ulp]))[0] == 1.0                 # tie -> even (down)
    assert ops.round_bf16(np.array([one + 3 * half_ulp]))[0] == 1.0 + 2 ** -6   # tie -> even (up)
    assert ops.round_bf16(np.array([one + half_ulp * 1.5]))[0] == 1.0 + 2 ** -7  # above half -> up
    assert ops.round_bf16(np.array([-2.5]))[0] == -2.5
    # FP32 first: 1 + 2^-8 + 2^-30 becomes the exact tie 1 + 2^-8 in FP32, then ties to even.
    assert ops.round_bf16(np.array([one + half_ulp + 2.0 ** -30]))[0] == 1.0
    # bf16 values are fixed points
    v = ops.bf16_bits_to_f64(np.arange(0, 0x7F80, 97, dtype=np.uint16))
    assert np.array_equal(ops.round_bf16(v), v)


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    vals = ops.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.0
    assert math.copysign(1.0, vals[3]) == -1.0
    assert vals[4] == 3.140625
    assert vals[5] == (2 - 2 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------- pointwise
def test_gate_closed_forms():
    a = np.linspace(-30, 30, 121)
    alpha, beta = ops.gates(a, a)
    # exp(-softplus(a)) = 1 / (1 + e^a) = sigmoid(-a)
    np.testing.assert_allclose(alpha, 1.0 / (1.0 + np.exp(a)), rtol=1e-12)
    np.testing.assert_allclose(beta, 1.0 / (1.0 + np.exp(-a)), rtol=1e-12)
    assert ops.softplus(np.array([0.0]))[0] == pytest.approx(math.log(2.0), rel=1e-15)
    assert ops.softplus(np.array([800.0]))[0] == 800.0           # no overflow
    assert ops.sigmoid(np.array([-800.0]))[0] >= 0.0
    assert ops.silu(np.array([0.0]))[0] == 0.0
    assert ops.silu(np.array([50.0]))[0] == pytest.approx(50.0, rel=1e-15)
    assert ops.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def test_rmsnorm_and_l2norm_invariants():
    x = rng.standard_normal((5, 64)) * 3.0
    y = ops.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)
    y2 = ops.rmsnorm(7.5 * x, np.ones(64), 0.0)
    np.testing.assert_allclose(y, y2, rtol=1e-12)
    g = rng.standard_normal(64)
    np.testing.assert_allclose(ops.rmsnorm(x, g, 0.0), y * g, rtol=1e-12)
    # eps sits inside the square root: a zero vector stays zero, a constant row c maps to c/sqrt(c^2+eps)
    assert np.all(ops.rmsnorm(np.zeros((1, 8)), np.ones(8), 1e-6) == 0.0)
    c = 1e-3
    np.testing.assert_allclose(ops.rmsnorm(np.full((1, 4), c), np.ones(4), 1e-6), c / math.sqrt(c * c + 1e-6))
    u = ops.l2norm(x, 0.0)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, rtol=1e-12)


def test_gated_rmsnorm_scale_invariance_and_gate():
    o = rng.standard_normal((3, 4, 16))
    z = rng.standard_normal((3, 4, 16))
    g = rng.standard_normal(16)
    a = ops.gated_rmsnorm(o, z, g, 0.0)
    b = ops.gated_rmsnorm(o * 123.0, z, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # per head: normalised o times gain times z*sigmoid(z), brute force on one head
    oh, zh = o[1, 2], z[1, 2]
    want = [oh[i] / math.sqrt(sum(t * t for t in oh) / 16) * g[i] * zh[i] / (1 + math.exp(-zh[i]))
            for i in range(16)]
    np.testing.assert_allclose(a[1, 2], want, rtol=1e-12)


def test_swiglu_definition_brute_force():
    gv, uv = rng.standard_normal(10), rng.standard_normal(10)
    want = [gv[i] / (1 + math.exp(-gv[i])) * uv[i] for i in range(10)]
    np.testing.assert_allclose(ops.swiglu(gv, uv), want, rtol=1e-13)


def test_argmax_lowest_index_on_ties():
    assert ops.argmax_lowest(np.array([0.0, 3.0, 1.0, 3.0])) == 1
    assert ops.argmax_lowest(np.array([-1.0, -1.0])) == 0
    with pytest.raises(FloatingPointError):
        ops.argmax_lowest(np.array([0.0, np.nan]))


# ----------------------------------------------------------------------------- short conv
def test_conv_impulse_response_is_the_taps():
    C, K, T = 5, 4, 9
    taps = rng.standard_normal((C, K))
    x = np.zeros((T, C))
    x[0] = 1.0
    out, _ = ops.causal_conv(np.zeros((K - 1, C)), x, taps)
    for lag in range(K):     # the current token meets tap K-1, the token `lag` steps back meets tap K-1-lag
        np.testing.assert_array_equal(out[lag], taps[:, K - 1 - lag])
    assert np.all(out[K:] == 0.0)


def test_conv_split_equals_whole_and_brute_force():
    C, K, T = 6, 4, 11
    taps = rng.standard_normal((C, K))
    x = rng.standard_normal((T, C))
    whole, hist_whole = ops.causal_conv(np.zeros((K - 1, C)), x, taps)
    h = np.zeros((K - 1, C))
    parts = []
    for s in (slice(0, 1), slice(1, 2), slice(2, 7), slice(7, 11)):
        o, h = ops.causal_conv(h, x[s], taps)
        parts.append(o)
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=1e-14)
    np.testing.assert_array_equal(h, hist_whole)
    for t in range(T):
        for c in range(C):
            want = sum(taps[c, i] * x[t - (K - 1) + i, c] for i in range(K) if t - (K - 1) + i >= 0)
            assert whole[t, c] == pytest.approx(want, rel=1e-12, abs=1e-15)


# ----------------------------------------------------------------------------- delta rule
def test_delta_rule_identity_when_no_write_no_decay():
    S = rng.standard_normal((8, 6))
    k, v, q = unit(rng.standard_normal(6)), rng.standard_normal(8), rng.standard_normal(6)
    S1, o = ops.delta_rule_step(S, k, v, q, alpha=1.0, beta=0.0)
    np.testing.assert_array_equal(S1, S)
    np.testing.assert_allclose(o, S @ q, rtol=1e-14)


def test_delta_rule_full_decay_writes_outer_product():
    S = rng.standard_normal((8, 6))
    k, v, q = unit(rng.standard_normal(6)), rng.standard_normal(8), rng.standard_normal(6)
    beta = 0.37
    S1, o = ops.delta_rule_step(S, k, v, q, alpha=0.0, beta=beta)
    np.testing.assert_allclose(S1, beta * np.outer(v, k), rtol=1e-14)
    np.testing.assert_allclose(o, beta * v * (k @ q), rtol=1e-13)


def test_delta_rule_write_then_read_returns_value():
    S = rng.standard_normal((8, 6))
    k, v = unit(rng.standard_normal(6)), rng.standard_normal(8)
    S1, o = ops.delta_rule_step(S, k, v, k, alpha=1.0, beta=1.0)
    np.testing.assert_allclose(S1 @ k, v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_delta_rule_orthonormal_keys_store_every_pair():
    d_k, d_v, n = 6, 5, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    keys = Qm[:, :n].T
    vals = rng.standard_normal((n, d_v))
    S = np.zeros((d_v, d_k))
    for i in range(n):
        S, _ = ops.delta_rule_step(S, keys[i], vals[i], keys[i], 1.0, 1.0)
    np.testing.assert_allclose(S, sum(np.outer(vals[i], keys[i]) for i in range(n)), atol=1e-12)
    for i in range(n):
        np.testing.assert_allclose(S @ keys[i], vals[i], atol=1e-12)


def test_delta_rule_factored_equals_literal_form():
    for _ in range(5):
        S = rng.standard_normal((7, 5))
        k, v, q = unit(rng.standard_normal(5)), rng.standard_normal(7), rng.standard_normal(5)
        alpha, beta = rng.uniform(0, 1), rng.uniform(0, 1)
        S1, o = ops.delta_rule_step(S, k, v, q, alpha, beta)
        np.testing.assert_allclose(S1, ops.delta_rule_step_literal(S, k, v, alpha, beta), rtol=1e-12, atol=1e-14)


def test_delta_rule_brute_force_loops():
    d_v, d_k = 3, 4
    S = rng.standard_normal((d_v, d_k))
    k, v, q = unit(rng.standard_normal(d_k)), rng.standard_normal(d_v), rng.standard_normal(d_k)
    alpha, beta = 0.8, 0.3
    # S_new[r][c] = alpha*sum_m S[r][m]*(delta_mc - beta*k_m*k_c) + beta*v_r*k_c
    want = [[alpha * sum(S[r][m] * ((1.0 if m == c else 0.0) - beta * k[m] * k[c]) for m in range(d_k))
             + beta * v[r] * k[c] for c in range(d_k)] for r in range(d_v)]
    S1, o = ops.delta_rule_step(S, k, v, q, alpha, beta)
    np.testing.assert_allclose(S1, want, rtol=1e-12)
    np.testing.assert_allclose(o, [sum(want[r][c] * q[c] for c in range(d_k)) for r in range(d_v)], rtol=1e-12)


def test_delta_rule_spectral_contraction():
    S = rng.standard_normal((16, 16))
    for _ in range(20):
        k, v, q = unit(rng.standard_normal(16)), rng.standard_normal(16), rng.standard_normal(16)
        alpha, beta = rng.uniform(0, 1), rng.uniform(0, 1)
        S1, _ = ops.delta_rule_step(S, k, v, q, alpha, beta)
        assert np.linalg.norm(S1, 2) <= alpha * np.linalg.norm(S, 2) + beta * np.linalg.norm(v) + 1e-12
        S = S1


@pytest.mark.parametrize("chunk", [1, 7, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("gate_bias", [-5.0, 0.0, 4.0])
def test_chunked_equals_token_by_token(chunk, T, gate_bias):
    d_k, d_v = 16, 12
    r = np.random.default_rng(T * 100 + chunk)
    K = ops.l2norm(r.standard_normal((T, d_k)), 0.0)
    Q = ops.l2norm(r.standard_normal((T, d_k)), 0.0)
    V = r.standard_normal((T, d_v))
    a = r.standard_normal(T) + gate_bias    # bias -5: alpha near 1; bias +4: alpha near 0
    alpha, beta = ops.gates(a, r.standard_normal(T))
    S0 = r.standard_normal((d_v, d_k))
    S = S0.copy()
    O = np.zeros((T, d_v))
    for t in range(T):
        S, O[t] = ops.delta_rule_step(S, K[t], V[t], Q[t], alpha[t], beta[t])
    Oc, Sc = ops.delta_rule_chunked(S0, K, V, Q, -ops.softplus(a), beta, chunk)
    np.testing.assert_allclose(Oc, O, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(Sc, S, rtol=1e-9, atol=1e-11)


# ----------------------------------------------------------------------------- rope
def test_rope_closed_forms():
    theta = 10000.0
    x = rng.standard_normal((3, 2))
    for p in (0, 1, 5, 1234):
        got = ops.rope(x, p, theta)                  # d=2: one pair rotated by angle p
        want = np.stack([x[:, 0] * math.cos(p) - x[:, 1] * math.sin(p),
                         x[:, 1] * math.cos(p) + x[:, 0] * math.sin(p)], axis=1)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    x4 = rng.standard_normal(4)
    p = 7
    f1 = theta ** (-2.0 / 4)                         # second pair's inverse frequency
    want = [x4[0] * math.cos(p) - x4[2] * math.sin(p), x4[1] * math.cos(p * f1) - x4[3] * math.sin(p * f1),
            x4[2] * math.cos(p) + x4[0] * math.sin(p), x4[3] * math.cos(p * f1) + x4[1] * math.sin(p * f1)]
    np.testing.assert_allclose(ops.rope(x4, p, theta), want, rtol=1e-12)


def test_rope_invariants():
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    np.testing.assert_array_equal(ops.rope(q, 0, 10000.0), q)
    np.testing.assert_allclose(np.linalg.norm(ops.rope(q, 777, 10000.0)), np.linalg.norm(q), rtol=1e-12)
    d1 = ops.rope(q, 50, 10000.0) @ ops.rope(k, 20, 10000.0)
    d2 = ops.rope(q, 530, 10000.0) @ ops.rope(k, 500, 10000.0)
    assert d1 == pytest.approx(d2, rel=1e-9)


# ----------------------------------------------------------------------------- attention
def test_attention_single_key_returns_value():
    q = rng.standard_normal((4, 8))
    Kc, Vc = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8))
    o = ops.attention_one_query(q, Kc, Vc)
    for i in range(4):
        np.testing.assert_allclose(o[i], Vc[0, i * 2 // 4], rtol=1e-14)


def test_attention_zero_query_is_prefix_mean():
    Kc, Vc = rng.standard_normal((9, 2, 8)), rng.standard_normal((9, 2, 8))
    o = ops.attention_one_query(np.zeros((4, 8)), Kc, Vc)
    for i in range(4):
        np.testing.assert_allclose(o[i], Vc[:, i // 2].mean(axis=0), rtol=1e-13)


def test_attention_two_keys_closed_form_scale():
    d = 16
    q = np.zeros((1, d)); q[0, 0] = 2.0
    Kc = np.zeros((2, 1, d)); Kc[0, 0, 0] = 1.0; Kc[1, 0, 0] = -0.5
    Vc = rng.standard_normal((2, 1, d))
    s0, s1 = 2.0 / math.sqrt(d), -1.0 / math.sqrt(d)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(ops.attention_one_query(q, Kc, Vc)[0], w0 * Vc[0, 0] + (1 - w0) * Vc[1, 0], rtol=1e-13)


def test_attention_gqa_grouping_is_contiguous():
    n_q, n_kv, d, T = 8, 2, 4, 5
    q = rng.standard_normal((n_q, d))
    Kc = rng.standard_normal((T, n_kv, d))
    Vc = np.zeros((T, n_kv, d)); Vc[:, 1, :] = 1.0
    o = ops.attention_one_query(q, Kc, Vc)
    np.testing.assert_allclose(o[:4], 0.0, atol=1e-15)
    np.testing.assert_allclose(o[4:], 1.0, rtol=1e-13)


def test_attention_brute_force_and_incremental_agree():
    from oracle.model import attention_causal
    T, n_q, n_kv, d = 37, 4, 2, 8
    Q, K, V = (rng.standard_normal((T, n, d)) for n in (n_q, n_kv, n_kv))
    dense = ops.attention_masked_dense(Q, K, V)
    incr = np.stack([ops.attention_one_query(Q[t], K[:t + 1], V[:t + 1]) for t in range(T)])
    blocked = attention_causal(Q, K, V, np.arange(T), round_p=False, block=8)
    np.testing.assert_allclose(incr, dense, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(blocked, dense, rtol=1e-12, atol=1e-13)
    # MHA special case (n_kv = n_q) equals independent single-head attention, brute-force loops
    Kf, Vf = rng.standard_normal((T, n_q, d)), rng.standard_normal((T, n_q, d))
    mha = ops.attention_masked_dense(Q, Kf, Vf)
    t, i = 11, 3
    s = [sum(Q[t, i, c] * Kf[u, i, c] for c in range(d)) / math.sqrt(d) for u in range(t + 1)]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    want = [sum(e[u] * Vf[u, i, c] for u in range(t + 1)) / sum(e) for c in range(d)]
    np.testing.assert_allclose(mha[t, i], want, rtol=1e-12)


def test_attention_rounded_probabilities_stay_close():
    T, d = 50, 16
    Q, K, V = rng.standard_normal((T, 2, d)), rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, d))
    from oracle.model import attention_causal
    a = attention_causal(Q, K, V, np.arange(T), round_p=False)
    b = attention_causal(Q, K, V, np.arange(T), round_p=True)
    assert np.max(np.abs(a - b)) < 2.0 ** -7 * np.max(np.abs(V))     # within bf16 precision of P


def test_numpy_matmul_matches_python_loops():
    A, B = rng.standard_normal((3, 5)), rng.standard_normal((5, 4))
    want = [[sum(A[i, k] * B[k, j] for k in range(5)) for j in range(4)] for i in range(3)]
    np.testing.assert_allclose(A @ B, want, rtol=1e-13)
