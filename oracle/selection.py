"""Page selection for streaming mode (oracle; test infrastructure only).

KV-offload news page (rebasdaily.com topic page on Qwen3.8-Flash-Next KV
offload), section "新招不是全搬，而是分层放": with most of the KV cache in system
memory, attention runs over a fixed budget of 2,048 selected tokens (QSA), and
the page's account of the rule breaks off. A plain rule is declared instead,
written out step by step:

1. Key sums. For page p (tokens 256p .. 256p+255 of the sequence), KV head g and
   element e: S[p][g][e] = sum over the page's tokens of k[t][g][e] * 2^24. fp16
   values are integer multiples of 2^-24 below 2^16, so every term and the sum
   (at most 256 terms, below 2^48) are exact integers.
2. Page representatives. R[p][g][e] = S[p][g][e] / 2^32 (the exact key sum
   divided by 256, the mean key of a full page) rounded once to fp16, nearest
   with ties to even. Scores read these 2-byte values instead of the 8-byte sums.
3. Query sums. Q[g][e] = sum over the query heads h of KV head g's group of
   q[h][e] * 2^24 (exact integers below 2^43).
4. Score. score[p] = sum over g and e of Q[g][e] * R[p][g][e] * 2^24: the summed
   query-key products of the group's heads with the page's representative keys,
   up to the positive factor 2^48; an exact integer (Python int).
5. Selection of k pages out of n: if n <= k, every page; otherwise the last
   page (the one holding the newest tokens) and the k - 1 other pages of
   largest score, ties to the lower page index. Returned in ascending order.

Steps 1, 3 and 4 are integer arithmetic and step 2 one rounding of an exact
value, so the selection is exact and does not depend on any summation order.
"""

from __future__ import annotations

import numpy as np

SCALE = 1 << 24  # fp16 values are integer multiples of 2^-24


def fp16_to_int(x) -> np.ndarray:
    """fp16 values as exact integers of 2^-24 (int64)."""
    v = np.asarray(x, np.float16).astype(np.float64) * SCALE
    out = v.astype(np.int64)
    assert np.array_equal(out.astype(np.float64), v), "fp16 times 2^24 must be an integer"
    return out


def key_sums(k, n_pages: int | None = None) -> np.ndarray:
    """k: fp16 [T, Hkv, D] (tokens 0..T-1) -> S int64 [n_pages, Hkv, D] (step 1)."""
    k = np.asarray(k, np.float16)
    T, hkv, d = k.shape
    n = -(-T // 256) if n_pages is None else n_pages
    ki = fp16_to_int(k)
    S = np.zeros((n, hkv, d), np.int64)
    for p in range(min(n, -(-T // 256))):
        S[p] = ki[256 * p:256 * p + 256].sum(axis=0)
    return S


def key_reps(S) -> np.ndarray:
    """S int64 [..., D] -> R fp16 (step 2): S / 2^32 rounded once to fp16, nearest-even.
    |S| < 2^48, so S / 2^32 is exact in float64 and the cast rounds it once."""
    S = np.asarray(S, np.int64)
    x = S.astype(np.float64)
    assert np.array_equal(x.astype(np.int64), S), "key sums must be exact in float64"
    return (x / 4294967296.0).astype(np.float16)


def query_sums(q, n_kv_heads: int) -> np.ndarray:
    """q: fp16 [Hq, D] -> Q int64 [Hkv, D] (step 3; groups of Hq / Hkv consecutive heads)."""
    qi = fp16_to_int(q)
    hq, d = qi.shape
    G = hq // n_kv_heads
    return qi.reshape(n_kv_heads, G, d).sum(axis=1)


def page_scores(q, R) -> list:
    """Exact scores (Python ints) of every page from its representatives R fp16
    [n_pages, Hkv, D] (step 4)."""
    Q = query_sums(q, R.shape[1]).astype(object)
    Ri = fp16_to_int(R)
    return [int((Q * Ri[p].astype(object)).sum()) for p in range(R.shape[0])]


def select_pages(scores, k_sel: int) -> list:
    """Step 5: the last page plus the k_sel - 1 best others (ties: lower index), ascending."""
    n = len(scores)
    if n <= k_sel:
        return list(range(n))
    last = n - 1
    others = sorted(range(last), key=lambda p: (-scores[p], p))[:k_sel - 1]
    return sorted(others + [last])


def select(q, k, k_sel: int) -> list:
    """Selection for query q [Hq, D] over keys k [T, Hkv, D] (all steps)."""
    return select_pages(page_scores(q, key_reps(key_sums(k))), k_sel)
