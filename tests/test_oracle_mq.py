"""Pins of the oracle's multi-query (causal) attention, oracle.attention.multi_query_attention:
closed forms, a scalar brute force, and the causal invariants."""

import math

import numpy as np

from oracle import attention, records


def rand_kv(rng, T, hkv=2, d=256):
    return rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hkv, d))


def test_one_visible_token_gives_its_value_exactly():
    """A query that sees one token returns that token's value (softmax of one score = 1);
    with n_q = T, query 0 sees token 0 only."""
    rng = np.random.default_rng(1)
    k, v = rand_kv(rng, 5)
    q = rng.standard_normal((5, 4, 256)).astype(np.float16)
    out = attention.multi_query_attention(q, k, v, records.FMT_INT8)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def test_queries_without_context_are_zero():
    rng = np.random.default_rng(2)
    k, v = rand_kv(rng, 2)
    q = rng.standard_normal((4, 4, 256)).astype(np.float16)
    out = attention.multi_query_attention(q, k, v, records.FMT_INT8)
    assert not out[:2].any() and out[2:].any()


def test_scalar_brute_force():
    """Every output element from plain loops: causal prefix, max-subtracted softmax."""
    rng = np.random.default_rng(3)
    T, n_q, hq, hkv, d = 7, 3, 4, 2, 8
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    q = rng.standard_normal((n_q, hq, d)).astype(np.float16)
    scale = 0.37
    got = attention.multi_query_attention(q, k, v, records.FMT_INT8, scale)
    for j in range(n_q):
        last = T - n_q + j
        for h in range(hq):
            g = h // (hq // hkv)
            s = [scale * sum(float(q[j, h, e]) * k[t, g, e] for e in range(d)) for t in range(last + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            for e in range(d):
                want = sum(w[t] * v[t, g, e] for t in range(last + 1)) / sum(w)
                assert abs(got[j, h, e] - want) <= 1e-12 * (1 + abs(want))


def test_causality_and_the_last_query():
    """Tokens after a query's position do not change it; the newest query is the decode
    attention over the whole context, for a rotated format too."""
    rng = np.random.default_rng(4)
    T, n_q = 40, 4
    k, v = rand_kv(rng, T, hkv=4)
    q = rng.standard_normal((n_q, 24, 256)).astype(np.float16)
    for fmt in (records.FMT_INT8, records.FMT_Q4_0, records.FMT_K8V4):
        out = attention.multi_query_attention(q, k, v, fmt)
        assert np.array_equal(out[-1], attention.decode_attention(q[-1], k, v, fmt))
        k2, v2 = k.copy(), v.copy()
        k2[T - 2:] += 5.0                          # the two newest tokens change
        v2[T - 2:] -= 3.0
        out2 = attention.multi_query_attention(q, k2, v2, fmt)
        assert np.array_equal(out2[:2], out[:2])   # queries 0, 1 see tokens <= T - 3
        assert not np.array_equal(out2[2:], out[2:])
