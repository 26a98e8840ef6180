"""Pins of the oracle's page selection (oracle/selection.py) against independent
computations: exact rationals, a brute-force nearest-fp16 search, hand-built pages,
and float rankings."""

import bisect
from fractions import Fraction

import numpy as np

from oracle import selection as sel

# every finite non-negative fp16 value, as (exact value, bit pattern), ascending
_F16_POS = sorted((Fraction(float(v)), int(b)) for b, v in
                  zip(np.arange(0x7C00, dtype=np.uint16), np.arange(0x7C00, dtype=np.uint16).view(np.float16)))
_F16_VALS = [v for v, _ in _F16_POS]


def nearest_f16_bits(x: Fraction) -> int:
    """Brute-force round to nearest fp16 (ties to the even bit pattern) by search over
    the sorted list of every finite fp16 value; the sign is taken from x."""
    a = abs(x)
    i = bisect.bisect_left(_F16_VALS, a)
    if i < len(_F16_VALS) and _F16_VALS[i] == a:
        bits = _F16_POS[i][1]
    else:
        lo, hi = _F16_POS[i - 1], _F16_POS[i]
        dl, dh = a - lo[0], hi[0] - a
        bits = lo[1] if dl < dh or (dl == dh and lo[1] % 2 == 0) else hi[1]
    return bits | (0x8000 if x < 0 else 0)


def test_representatives_round_once_to_nearest_even():
    """Step 2 against the brute force: exact fp16 values, midpoints between neighbours
    (ties to even), points just off them, subnormal and top-of-range sums."""
    rng = np.random.default_rng(7)
    S = [0, 1, -1, 1 << 7, (1 << 7) + 1, 3 << 7, 1 << 8, 65504 << 32, -(65504 << 32), (65504 << 32) - 1]
    for i in rng.integers(1, 0x7BFF, 400):
        a, b = _F16_POS[i][0], _F16_POS[i + 1][0]
        mid = (a + b) / 2 * (1 << 32)
        assert mid.denominator == 1
        m = int(mid.numerator)
        S += [m, m - 1, m + 1, -m, int(a * (1 << 32))]
    S += [int(x) for x in rng.integers(-(1 << 47), 1 << 47, 2000)]
    S += [int(x) for x in rng.integers(-(1 << 20), 1 << 20, 2000)]       # subnormal results
    got = sel.key_reps(np.array(S, np.int64)).view(np.uint16)
    for v, g in zip(S, got.tolist()):
        assert g == nearest_f16_bits(Fraction(v, 1 << 32)), v


def test_key_sums_equal_exact_rational_sums():
    rng = np.random.default_rng(4)
    T = 600
    k = (rng.standard_normal((T, 2, 8)) * 3).astype(np.float16)
    S = sel.key_sums(k)
    assert S.shape == (3, 2, 8)
    for p in range(3):
        for g in range(2):
            for e in range(8):
                ks = sum(Fraction(float(k[t, g, e])) for t in range(256 * p, min(T, 256 * p + 256)))
                assert S[p, g, e] == ks * (1 << 24)


def test_fp16_times_2_24_is_exact_for_every_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    ints = sel.fp16_to_int(x)
    for v, i in zip(x[::97], ints[::97]):
        assert Fraction(float(v)) * (1 << 24) == i
    assert ints.max() == 65504 * (1 << 24) and ints.min() == -65504 * (1 << 24)


def test_scores_equal_exact_rational_products_per_head():
    """Scores from the grouped integer query sums equal the products with the page
    representatives summed head by head in exact rationals, the representatives taken
    from the brute-force rounding of the exact page sums (checks the head -> KV-head
    grouping, the page ranges and the 2^-32 scale)."""
    rng = np.random.default_rng(1)
    hq, hkv, d, T = 6, 2, 8, 600
    k = (rng.standard_normal((T, hkv, d)) * 3).astype(np.float16)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    R = sel.key_reps(sel.key_sums(k))
    assert R.shape == (3, hkv, d) and R.dtype == np.float16
    got = sel.page_scores(q, R)
    G = hq // hkv
    for p in range(3):
        ref = Fraction(0)
        for h in range(hq):
            g = h // G
            for e in range(d):
                ks = sum(Fraction(float(k[t, g, e])) for t in range(256 * p, min(T, 256 * p + 256)))
                bits = nearest_f16_bits(ks / 256)
                rep = Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))
                ref += Fraction(float(q[h, e])) * rep
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
    R = sel.key_reps(sel.key_sums(k))
    assert R[:, 0, 0].tolist() == c                  # a constant page's mean is exact
    sc = sel.page_scores(q, R)
    assert sc == [int(2 * v * (1 << 48)) for v in c]
    assert sel.select_pages(sc, 3) == [1, 3, 5]       # last page + the tie (1, 3) of the best
    assert sel.select_pages(sc, 2) == [1, 5]          # tie broken to the lower index
    assert sel.select_pages(sc, 4) == [1, 3, 4, 5]
    q[:, 0] = -1.0                                      # reversed ranking
    assert sel.select_pages(sel.page_scores(q, R), 3) == [0, 2, 5]
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
        # page means of the keys (float64 sums of fp16 values are exact), cast to fp16
        mean = np.stack([kf[256 * p:256 * p + 256].sum(axis=0) / 256 for p in range(n)])
        rf = mean.astype(np.float16).astype(np.float64)
        fs = np.array([sum(qf[h] @ rf[p, h // 6] for h in range(24)) for p in range(n)])
        order = sorted(range(n - 1), key=lambda p: -fs[p])
        gap = abs(fs[order[k_sel - 2]] - fs[order[k_sel - 1]])
        if gap > 1e-6 * abs(fs[order[k_sel - 2]]):
            assert exact == sorted(order[:k_sel - 1] + [n - 1]), trial


def test_scaling_the_query_by_a_power_of_two_keeps_the_selection():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((256 * 12, 4, 256)).astype(np.float16)
    q = rng.standard_normal((24, 256)).astype(np.float16)
    assert sel.select(q, k, 5) == sel.select((q.astype(np.float32) * 4).astype(np.float16), k, 5)
