"""Pins of the oracle's page selection (oracle/selection.py) against independent
computations: exact rationals, hand-built pages, and float rankings."""

from fractions import Fraction

import numpy as np

from oracle import selection as sel


def test_fp16_times_2_24_is_exact_for_every_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    ints = sel.fp16_to_int(x)
    for v, i in zip(x[::97], ints[::97]):
        assert Fraction(float(v)) * (1 << 24) == i
    assert ints.max() == 65504 * (1 << 24) and ints.min() == -65504 * (1 << 24)


def test_scores_equal_exact_rational_products_per_head():
    """Scores from the grouped integer sums equal the products summed head by head in
    exact rationals (checks the head -> KV-head grouping and the page ranges)."""
    rng = np.random.default_rng(1)
    hq, hkv, d, T = 6, 2, 8, 600
    k = (rng.standard_normal((T, hkv, d)) * 3).astype(np.float16)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    S = sel.key_sums(k)
    assert S.shape == (3, hkv, d)
    got = sel.page_scores(q, S)
    G = hq // hkv
    for p in range(3):
        ref = Fraction(0)
        for h in range(hq):
            g = h // G
            for e in range(d):
                ks = sum(Fraction(float(k[t, g, e])) for t in range(256 * p, min(T, 256 * p + 256)))
                ref += Fraction(float(q[h, e])) * ks
        assert got[p] == ref * (1 << 48), p


def test_hand_built_pages():
    """Keys constant per page along element 0: the score is proportional to c_p."""
    hq, hkv, d = 2, 1, 4
    c = [1.0, 4.0, -2.0, 4.0, 3.0, 0.5]          # pages 1 and 3 tie
    k = np.zeros((256 * len(c), hkv, d), np.float16)
    for p, v in enumerate(c):
        k[256 * p:256 * p + 256, 0, 0] = v
    q = np.zeros((hq, d), np.float16)
    q[:, 0] = 1.0
    S = sel.key_sums(k)
    sc = sel.page_scores(q, S)
    assert sc == [int(2 * 256 * v * (1 << 48)) for v in c]
    assert sel.select_pages(sc, 3) == [1, 3, 5]       # last page + the tie (1, 3) of the best
    assert sel.select_pages(sc, 2) == [1, 5]          # tie broken to the lower index
    assert sel.select_pages(sc, 4) == [1, 3, 4, 5]
    q[:, 0] = -1.0                                      # reversed ranking
    assert sel.select_pages(sel.page_scores(q, S), 3) == [0, 2, 5]
    assert sel.select_pages(sc, 6) == [0, 1, 2, 3, 4, 5] and sel.select_pages(sc, 9) == list(range(6))


def test_last_page_forced_even_when_worst():
    c = [5.0, 4.0, 3.0, 2.0, -9.0]
    k = np.zeros((256 * 4 + 10, 1, 2), np.float16)     # a partial last page of 10 tokens
    for p, v in enumerate(c):
        k[256 * p:256 * p + 256, 0, 0] = v
    q = np.ones((1, 2), np.float16)
    assert sel.select(q, k, 2) == [0, 4]


def test_selection_agrees_with_float_ranking_when_gaps_are_clear():
    rng = np.random.default_rng(2)
    for trial in range(5):
        T, k_sel = 256 * 40 + 77, 8
        k = rng.standard_normal((T, 4, 256)).astype(np.float16)
        q = rng.standard_normal((24, 256)).astype(np.float16)
        exact = sel.select(q, k, k_sel)
        kf, qf = k.astype(np.float64), q.astype(np.float64)
        n = -(-T // 256)
        fs = np.array([sum(qf[h] @ kf[256 * p:256 * p + 256, h // 6].sum(axis=0) for h in range(24))
                       for p in range(n)])
        order = sorted(range(n - 1), key=lambda p: -fs[p])
        gap = abs(fs[order[k_sel - 2]] - fs[order[k_sel - 1]])
        if gap > 1e-6 * abs(fs[order[k_sel - 2]]):
            assert exact == sorted(order[:k_sel - 1] + [n - 1]), trial


def test_scaling_the_query_by_a_power_of_two_keeps_the_selection():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((256 * 12, 4, 256)).astype(np.float16)
    q = rng.standard_normal((24, 256)).astype(np.float16)
    assert sel.select(q, k, 5) == sel.select((q.astype(np.float32) * 4).astype(np.float16), k, 5)
