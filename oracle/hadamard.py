"""The normalized 256-point Walsh-Hadamard rotation (oracle).

Strata page, section "4-bit KV 缓存：先旋转，再压到 4-bit": before 4-bit storage
K and V, and the query with them, go through a 256-point Walsh-Hadamard
orthogonal rotation; because the same rotation is applied to Q and K the
scores are unchanged, the output is mixed from rotated V and restored by a
second product with H, which is its own inverse.

Readings (the page is silent on these):

* natural (Sylvester) ordering, H[i][j] = (-1)^popcount(i & j) / 16;
* normalization 1/16 = 1/sqrt(256), the only scaling for which H is both
  orthogonal and self-inverse, as the page states it is;
* no random sign flips (none are mentioned).
"""

from __future__ import annotations

import numpy as np

N = 256


def _popcount(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a >>= 1
    return c


def hadamard_matrix(n: int = N) -> np.ndarray:
    """H[i][j] = (-1)^popcount(i & j) / sqrt(n), float64, for n a power of two."""
    if n <= 0 or n & (n - 1):
        raise ValueError("n must be a power of two")
    i = np.arange(n)
    sign = np.where(_popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)
    return sign / np.sqrt(float(n))


_H = hadamard_matrix(N)


def rotate(x: np.ndarray) -> np.ndarray:
    """y = H x along the last axis (length 256), float64.

    For fp16-valued x the result is exact whatever the summation order: every
    product is +-x_j/16 (exact), every x_j is a multiple of 2^-24 below 2^16,
    so every partial sum is a multiple of 2^-28 below 2^20 and fits in the 53
    bits of a double. A library matrix product is therefore a faithful
    implementation of the definition here.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != N:
        raise ValueError("last axis must be 256")
    return x @ _H  # H is symmetric
