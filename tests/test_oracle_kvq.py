"""Pins of the oracle's 8-bit K/V-cache quantiser (oracle.ops.kv_q8_rows).

The reading (the pages name an 8-bit KV cache without a format): per cached row, in float32,
a = max |x|, e = the smallest integer with a <= 127 * 2^e, codes = round-half-even(x * 2^-e),
stored value = code * 2^e.  Each pin follows from that definition, not from the code.
"""
import numpy as np
import pytest

from oracle import kv_q8_rows, round_bf16
from workloads import TINY, TINY_Q8, HYBRID_24L_Q8, make_weights
from oracle import OracleModel, C2


def test_exact_rows_round_trip():
    rng = np.random.default_rng(1)
    for e in (-20, -7, 0, 3):
        q = rng.integers(-127, 128, size=(5, 64))
        q[:, 0] = 127                       # the row maximum sets the exponent
        x = np.ldexp(q.astype(np.float64), e)
        codes, ex, val = kv_q8_rows(x)
        assert np.all(ex == e)
        assert np.array_equal(codes.astype(np.int64), q)
        assert np.array_equal(val, x)


def test_error_bound_and_minimal_exponent():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-8, 8, size=(200, 1)))
    codes, e, val = kv_q8_rows(x)
    x32 = x.astype(np.float32).astype(np.float64)
    a = np.max(np.abs(x32), axis=1)
    assert np.all(a <= 127 * np.ldexp(1.0, e))          # fits: no code beyond 127
    assert np.all(a > 127 * np.ldexp(1.0, e - 1))       # minimal: one exponent less would not fit
    assert np.all(np.abs(x32 - val) <= np.ldexp(0.5, e)[:, None])
    assert np.max(np.abs(codes.astype(np.int64))) <= 127


def test_ties_go_to_even():
    x = np.ldexp(np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5]]), -3)
    codes, e, _ = kv_q8_rows(x)
    assert e[0] == -3
    assert codes[0].tolist() == [127, 2, 4, -2, -4, 0, 2]


def test_exponent_boundary():
    base = np.ldexp(127.0, -5)
    up = np.nextafter(np.float32(base), np.float32(np.inf)).astype(np.float64)
    assert kv_q8_rows(np.array([[base, 1e-3]]))[1][0] == -5
    assert kv_q8_rows(np.array([[up, 1e-3]]))[1][0] == -4


def test_zero_row_and_sign_symmetry():
    codes, e, val = kv_q8_rows(np.zeros((2, 16)))
    assert not np.any(codes) and not np.any(val) and np.all(e == -126)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 64))
    c1, e1, v1 = kv_q8_rows(x)
    c2, e2, v2 = kv_q8_rows(-x)
    assert np.array_equal(e1, e2) and np.array_equal(c2.astype(np.int64), -c1.astype(np.int64))
    assert np.array_equal(v2, -v1)


def test_lowest_exponent():
    """Rows below 127 * 2^-126 keep e = -126: codes are x * 2^126 rounded (a normal-number floor)."""
    x = np.array([[np.ldexp(3.0, -127), np.ldexp(-1.0, -130), np.ldexp(5.0, -126)]])
    codes, e, val = kv_q8_rows(x)
    assert e[0] == -126
    assert codes[0].tolist() == [2, 0, 5]            # 1.5 rounds to even 2; 2^-4 rounds to 0
    assert np.array_equal(val[0], np.ldexp(np.array([2.0, 0.0, 5.0]), -126))
    big = np.array([[np.ldexp(127.0, -126), 0.0]])
    assert kv_q8_rows(big)[1][0] == -126
    assert kv_q8_rows(np.array([[np.ldexp(128.0, -126)]]))[1][0] == -125


def test_stored_values_are_bfloat16_numbers():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((100, 128)) * 3.0
    _, _, val = kv_q8_rows(x)
    assert np.array_equal(round_bf16(val), val)


def test_model_with_quantised_cache_stores_the_quantised_rows():
    """The oracle model with kv_quant = 1 holds exactly kv_q8_rows of the K/V it computes, and its
    logits stay close to the bf16-cache model's (the quantiser changes the cached values only)."""
    w = make_weights(TINY, seed=0)
    prompt = np.arange(12) * 37 % TINY.vocab
    m8 = OracleModel(TINY_Q8, w, C2)
    mb = OracleModel(TINY, w, C2)
    l8, lb = m8.prefill(prompt), mb.prefill(prompt)
    li = TINY.layer_kinds.index("A")
    K = m8.Kc[li][:len(prompt)]
    _, _, requant = kv_q8_rows(K)
    assert np.array_equal(requant, K)                   # a stored row is a fixed point of the quantiser
    assert np.max(np.abs(l8 - lb)) < 0.05 * np.max(np.abs(lb))
    assert HYBRID_24L_Q8.kv_quant == 1 and TINY_Q8.kv_quant == 1
