"""Pins of the oracle's fp4 record (oracle/records.py): the e2m1 rounding against a brute
force, the exponent rule, exact fp16 dequantized values, error bounds, signs, the byte
size against the page's NVFP4 figure, and the page layout round trip."""

import json
import os

import numpy as np

from oracle import attention, hadamard, layout, records as R

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def brute_index(v):
    """Nearest e2m1 value by scanning the grid; ties to the even index; above 6 -> 6."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    if v >= 6.0:
        return 7
    best = None
    for i, g in enumerate(grid):
        dist = abs(v - g)
        if best is None or dist < best[0] or (dist == best[0] and i % 2 == 0):
            best = (dist, i)
    return best[1]


def test_e2m1_rounding_matches_brute_force():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.0, 6.0, 7.9, 100.0] + mids + [m + s for m in mids for s in (-2.0 ** -40, 2.0 ** -40)]
    vals += list(np.random.default_rng(1).uniform(0, 8, 5000))
    got = R.fp4_index(np.array(vals))
    for v, g in zip(vals, got):
        assert g == brute_index(v), v
    # ties: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0
    assert [R.FP4_GRID[i] for i in R.fp4_index(np.array(mids))] == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_exponent_rule_and_clamp():
    rng = np.random.default_rng(2)
    for scale in (1e-9, 1e-6, 3e-3, 1.0, 7.0, 300.0, 30000.0):
        y = rng.standard_normal((20, 256)) * scale
        c, d = R.quantize_fp4_rotated(y)
        a = np.abs(y.reshape(20, 8, 32)).max(axis=-1)
        dd = d.astype(np.float64)
        e = np.log2(dd)
        assert np.array_equal(e, np.round(e))                   # powers of two
        assert e.min() >= -23 and e.max() <= 13
        free = (e > -23) & (e < 13)
        ratio = a[free] / dd[free]
        assert np.all((ratio >= 4) & (ratio < 8))              # floor(log2 a) - 2
        if scale == 30000.0:
            assert e.max() == 13                                # large blocks clamp at 2^13
        if scale == 1e-9:
            assert e.min() == -23                               # tiny blocks clamp at 2^-23


def test_dequantized_values_are_fp16_numbers_and_bounded():
    rng = np.random.default_rng(3)
    for scale in (1e-7, 0.01, 1.0, 50.0, 2000.0):
        y = rng.standard_normal((30, 256)) * scale
        c, d = R.quantize_fp4_rotated(y)
        yh = R.dequantize_fp4(c, d)
        assert np.array_equal(yh.astype(np.float16).astype(np.float64), yh)
        dd = np.repeat(d.astype(np.float64), 32, axis=-1)
        v = np.abs(y) / np.where(dd > 0, dd, 1)
        # half the local grid spacing below 6, the excess above it
        step = np.select([v <= 2, v <= 4], [0.5, 1.0], 2.0)
        bound = np.where(v <= 6, step / 2, v - 6) * dd
        assert np.all(np.abs(y - yh) <= bound + 1e-300)


def test_signs_zero_blocks_and_codes():
    y = np.zeros((2, 256))
    y[1, 0], y[1, 1], y[1, 2] = -3.0, 3.0, -0.1   # -0.1 rounds to magnitude 0
    c, d = R.quantize_fp4_rotated(y)
    assert d[0].tolist() == [0.0] * 8 and not c[0].any()
    assert c[1, 0] == 8 + 7 and c[1, 1] == 7 and c[1, 2] == 0       # a = 3: d = 0.5, 3/0.5 = 6
    assert float(d[1, 0]) == 0.5 and not (c == 8).any()


def test_record_size_is_the_pages_nvfp4_figure():
    g = GOLDEN["smzdm_per_position_nvfp4"]
    assert 2 * R.record_bytes(R.KIND_FP4) == g["bytes_per_position"]    # K + V of one head
    assert layout.page_bytes(R.FMT_FP4, 4) == 4 * 2 * 256 * 144


def test_layout_round_trip():
    rng = np.random.default_rng(4)
    T = 300
    k = rng.standard_normal((T, 4, 256))
    v = rng.standard_normal((T, 4, 256))
    kc, ks = R.encode(k, R.KIND_FP4)
    vc, vs = R.encode(v, R.KIND_FP4)
    pages = layout.pack_pages(kc, ks, vc, vs, R.FMT_FP4)
    kc2, ks2, vc2, vs2 = layout.unpack_pages(pages, R.FMT_FP4, 4)
    assert np.array_equal(kc2[:T], kc) and np.array_equal(vc2[:T], vc)
    assert np.array_equal(ks2[:T], ks) and np.array_equal(vs2[:T], vs)


def test_attention_rotates_both_sides():
    """With fp4 K and V, attention over dequantized records equals the plain attention of
    the unrotated dequantized vectors (H is orthogonal and symmetric)."""
    rng = np.random.default_rng(5)
    T = 40
    k = rng.standard_normal((T, 4, 256))
    v = rng.standard_normal((T, 4, 256))
    q = rng.standard_normal((24, 256)).astype(np.float16)
    kc, ks = R.encode(k, R.KIND_FP4)
    vc, vs = R.encode(v, R.KIND_FP4)
    kh, vh = R.decode(kc, ks, R.KIND_FP4), R.decode(vc, vs, R.KIND_FP4)
    got = attention.decode_attention(q, kh, vh, R.FMT_FP4)
    # unrotate the records, then plain attention (the int8 format applies no rotation)
    want = attention.decode_attention(q, hadamard.rotate(kh), hadamard.rotate(vh), R.FMT_INT8)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)
