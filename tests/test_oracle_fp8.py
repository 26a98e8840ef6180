"""Pins of the oracle's fp8 record (oracle/records.py): the E4M3 value table against the
encoding's definition and torch's float8_e4m3fn, the rounding against a brute force and
against torch's conversion, the scale rule, error bounds, signs and saturation, the byte
size against the page's FP8 figure, and the page layout round trip."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention, layout, records as R

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_e4m3_table():
    # known points of the encoding: smallest subnormal, largest subnormal, smallest
    # normal, one, largest finite
    assert R.E4M3[1] == 2.0 ** -9 and R.E4M3[7] == 7 * 2.0 ** -9
    assert R.E4M3[8] == 2.0 ** -6 and R.E4M3[0x38] == 1.0 and R.E4M3[126] == 448.0
    assert np.all(np.diff(R.E4M3) > 0)
    # torch's float8_e4m3fn decodes the same bytes to the same values
    codes = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn)
    assert np.array_equal(codes.to(torch.float64).numpy(), R.E4M3)


def brute_code(v):
    """Nearest E4M3 magnitude by scanning all 127 values; ties to the even code; >448 -> 448."""
    best = None
    for c in range(127):
        dist = abs(v - R.E4M3[c])
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1]


def test_rounding_matches_brute_force():
    mids = list((R.E4M3[1:] + R.E4M3[:-1]) / 2)          # every tie
    vals = [0.0, 448.0, 460.0, 464.0, 1000.0, 2.0 ** -11, 2.0 ** -10] + mids
    vals += [m * (1 + s * 2.0 ** -30) for m in mids[::7] for s in (-1, 1)]
    vals += list(np.exp(np.random.default_rng(1).uniform(np.log(2.0 ** -12), np.log(500.0), 3000)))
    got = R.e4m3_code(np.array(vals))
    for v, g in zip(vals, got):
        assert g == brute_code(v), v


def test_rounding_matches_torch_conversion():
    """Inside the finite range torch's cast to float8_e4m3fn (round to nearest even) gives
    the same codes (inputs exactly representable in fp32, so the cast rounds once)."""
    rng = np.random.default_rng(2)
    v = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(440.0), 20000)).astype(np.float32)
    v = np.concatenate([v, ((R.E4M3[1:] + R.E4M3[:-1]) / 2).astype(np.float32)])
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(R.e4m3_code(v.astype(np.float64)), t)


def test_scale_rule_and_bounds():
    rng = np.random.default_rng(3)
    for scale in (1e-6, 1e-4, 3e-3, 1.0, 40.0, 2000.0):
        x = (rng.standard_normal((40, 256)) * scale).astype(np.float16).astype(np.float64)
        c, d = R.quantize_fp8(x)
        a = np.abs(x).max(axis=-1, keepdims=True)
        assert d.shape == (40, 1)
        assert np.array_equal(d, (a / 448.0).astype(np.float16))
        xh = R.dequantize_fp8(c, d)
        zero = d[:, 0] == 0                                   # a / 448 below fp16's half-subnormal
        assert np.all(a[zero] / 448.0 <= 2.0 ** -25) and not c[zero].any()
        x, xh, c, d = x[~zero], xh[~zero], c[~zero], d[~zero]
        dd = d.astype(np.float64)
        v = np.abs(x) / dd
        # half the local E4M3 spacing (2^-10 below 2^-6, else 2^(floor(log2 v) - 4)), or the
        # excess beyond 448
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        half = np.exp2(e - 4)
        bound = np.where(v <= 448.0, half, v - 448.0) * dd
        assert np.all(np.abs(x - xh) <= bound * (1 + 1e-12))
        assert c.size == 0 or (c & 0x7F).max() <= 126          # never a NaN code


def test_signs_zero_and_saturation():
    x = np.zeros((3, 256))
    x[1, 0], x[1, 1], x[1, 2] = -448.0, 448.0, -2.0 ** -12     # d = 1; -2^-12 rounds to 0
    x[2, 0], x[2, 1] = 65504.0, -65504.0                       # d = fp16(146.21) = 146.25
    c, d = R.quantize_fp8(x)
    assert float(d[0, 0]) == 0.0 and not c[0].any()
    assert float(d[1, 0]) == 1.0
    assert c[1, 0] == 0xFE and c[1, 1] == 0x7E and c[1, 2] == 0
    assert float(d[2, 0]) == 146.25
    assert c[2, 0] == 0x7E and c[2, 1] == 0xFE                 # 65504 / 146.25 = 447.9 -> 448
    tiny = np.zeros((1, 256))
    tiny[0, 0] = 627 * 2.0 ** -24                              # a / 448 = 1.3996 * 2^-24
    c, d = R.quantize_fp8(tiny)
    assert float(d[0, 0]) == 2.0 ** -24 and c[0, 0] == 0x7E   # the subnormal d: 627 saturates


def test_record_size_is_the_pages_fp8_figure():
    g = GOLDEN["smzdm_per_position_fp8"]
    assert 2 * R.record_bytes(R.KIND_FP8) == g["bytes_per_position"]     # K + V of one head
    assert layout.page_bytes(R.FMT_FP8, 4) == 4 * 2 * 256 * 258


def test_layout_round_trip():
    rng = np.random.default_rng(4)
    T = 300
    k = rng.standard_normal((T, 4, 256)) * 3
    v = rng.standard_normal((T, 4, 256))
    kc, ks = R.encode(k, R.KIND_FP8)
    vc, vs = R.encode(v, R.KIND_FP8)
    pages = layout.pack_pages(kc, ks, vc, vs, R.FMT_FP8)
    kc2, ks2, vc2, vs2 = layout.unpack_pages(pages, R.FMT_FP8, 4)
    assert np.array_equal(kc2[:T], kc) and np.array_equal(vc2[:T], vc)
    assert np.array_equal(ks2[:T], ks) and np.array_equal(vs2[:T], vs)
    # K code bytes sit where the int8 layout puts int8 codes
    i8 = layout.pack_pages(kc.view(np.int8), np.zeros((T, 4, 4), np.float16), vc.view(np.int8),
                           np.zeros((T, 4, 4), np.float16), R.FMT_INT8)
    assert np.array_equal(pages[:, :256 * 256], i8[:, :256 * 256])


def test_not_rotated():
    assert not R.rotates_query(R.FMT_FP8) and not R.rotates_output(R.FMT_FP8)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 256))
    c, d = R.quantize_fp8(x)
    # codes of representable values reproduce them exactly (no rotation in between)
    xr = R.dequantize_fp8(c, d)
    c2, d2 = R.quantize_fp8(xr)
    assert np.array_equal(R.dequantize_fp8(c2, d2), xr)
    q = rng.standard_normal((24, 256)).astype(np.float16)
    kv = rng.standard_normal((10, 4, 256))
    kc, ks = R.encode(kv, R.KIND_FP8)
    kh = R.decode(kc, ks, R.KIND_FP8)
    got = attention.decode_attention(q, kh, kh, R.FMT_FP8)
    want = attention.decode_attention(q, kh, kh, R.FMT_INT8)
    assert np.array_equal(got, want)


def test_nan_codes_are_refused():
    c = np.zeros((1, 256), np.uint8)
    c[0, 5] = 0xFF
    with pytest.raises(ValueError):
        R.dequantize_fp8(c, np.ones((1, 1), np.float16))


def test_scale_rounding_exhaustive_against_rationals():
    """d = fp16 round-to-nearest-even of the exact rational a / 448, for every positive
    finite fp16 amax a (31,743 values, subnormals included): the oracle's scale is pinned
    against an exact rounding written from IEEE 754 binary16, not against its own formula.
    A scale formed by an fp32 reciprocal multiply, a * (1/448), differs on 39 of these
    values and fails here. A plain fp32 division a / 448 happens to round to the same
    fp16 for every value, so a GPU encoder may use either fp32 or fp64 division."""
    from fractions import Fraction

    from test_oracle_pins import fp16_values_positive, fraction_to_fp16_rne

    a = fp16_values_positive().astype(np.float64)
    x = np.zeros((a.size, 256))
    x[:, 7] = a                       # one nonzero element: amax = a
    x[::2, 7] *= -1                   # the sign of the largest element does not matter
    _, d = R.quantize_fp8(x)
    want = np.array([fraction_to_fp16_rne(Fraction(float(v)) / 448) for v in a], np.float64)
    assert np.array_equal(d[:, 0].astype(np.float64), want)
    # subnormal fp16 scales are part of the sweep
    assert np.count_nonzero((want > 0) & (want < 2.0 ** -14)) > 100
