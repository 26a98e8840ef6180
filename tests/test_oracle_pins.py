"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: an
independent construction (Sylvester recursion, exact rationals, scalar
loops), a closed form, an invariant, or a number printed on the pages
(``tests/golden/page_numbers.json``, every entry with its source).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import accounting, attention, hadamard, layout, records

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


# ---------------------------------------------------------------- helpers

def sylvester(n):
    """H_1 = [1], H_2n = [[H, H], [H, -H]] (unnormalized), built without popcount."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def exact_sign(i, j):
    return -1 if bin(i & j).count("1") % 2 else 1


def exact_rotate(x):
    """H x in exact rationals, from the sign definition, element by element."""
    xs = [Fraction(float(v)) for v in x]
    return [sum(exact_sign(i, j) * xs[j] for j in range(256)) / 16 for i in range(256)]


def fraction_to_fp16_rne(v: Fraction) -> float:
    """Exact round-to-nearest-even of a rational to fp16, written from IEEE 754 binary16."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a))
    # fix log2 rounding at powers of two
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                      # subnormal range shares exponent -14
    ulp = Fraction(2) ** (e - 10)
    q = a / ulp
    n = math.floor(q)
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val > 65504:
        return sign * math.inf
    return sign * float(val)


def fp16_values_positive():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)   # all positive finite, incl. subnormals
    return bits.view(np.float16)


# ---------------------------------------------------------------- Hadamard

def test_hadamard_matches_sylvester_recursion():
    H = hadamard.hadamard_matrix(256)
    assert np.array_equal(H * 16, sylvester(256))


def test_hadamard_orthogonal_symmetric_self_inverse_exact():
    H = hadamard.hadamard_matrix(256)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, np.eye(256))      # exact in fp64: sums of +-1/256


def test_hadamard_special_vectors():
    ones = np.ones(256)
    e0 = np.zeros(256); e0[0] = 16
    assert np.array_equal(hadamard.rotate(ones), e0)
    for c in (0, 1, 77, 255):
        ec = np.zeros(256); ec[c] = 1
        assert np.all(np.abs(hadamard.rotate(ec)) == 1 / 16)


def test_rotation_exact_against_rationals():
    rng = np.random.default_rng(1)
    cases = [rng.standard_normal(256).astype(np.float16),
             np.clip(rng.standard_normal(256) * 3e4, -65504, 65504).astype(np.float16)]
    sub = np.zeros(256, np.float16)
    sub[::3] = np.float16(2.0 ** -24)               # smallest subnormal
    sub[1::7] = np.float16(-65504.0)
    cases.append(sub)
    for x in cases:
        got = hadamard.rotate(x.astype(np.float64))
        want = exact_rotate(x)
        assert all(Fraction(float(g)) == w for g, w in zip(got, want))
        # any other summation order gives the same doubles
        H = hadamard.hadamard_matrix()
        rev = np.array([sum(H[i, j] * float(x[j]) for j in reversed(range(256))) for i in range(256)])
        assert np.array_equal(got, rev)


def test_rotation_preserves_inner_products():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(256).astype(np.float16).astype(np.float64)
    k = (rng.standard_normal(256) * 20).astype(np.float16).astype(np.float64)
    exact = sum(Fraction(a) * Fraction(b) for a, b in zip(q, k))
    hq, hk = hadamard.rotate(q), hadamard.rotate(k)
    rot = sum(Fraction(a) * Fraction(b) for a, b in zip(hq, hk))
    assert rot == exact                            # rotated values are exact, so equal exactly
    assert abs(float(hq @ hk) - float(exact)) < 1e-12 * float(np.abs(q) @ np.abs(k))


# ---------------------------------------------------------------- fp16 rounding

def test_fp16_rounding_is_single_rounding():
    v = 1 + 2.0 ** -11 + 2.0 ** -30
    assert float(records.fp16_rne(v)) == 1.0009765625
    assert float(np.float32(v).astype(np.float16)) == 1.0  # the double-rounding trap


def test_int8_scale_rounding_exhaustive():
    """d = fp16_rne(a/127) from an fp64 quotient equals the exact-rational rounding
    for every positive finite fp16 amax a."""
    a = fp16_values_positive()
    got = records.fp16_rne(a.astype(np.float64) / 127.0)
    want = np.array([fraction_to_fp16_rne(Fraction(float(x)) / 127) for x in a], np.float64)
    assert np.array_equal(got.astype(np.float64), want)


def test_fp16_rne_matches_exact_on_random_doubles():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 5, 2000),
                        rng.uniform(65000, 66000, 50)])
    got = records.fp16_rne(v).astype(np.float64)
    want = np.array([fraction_to_fp16_rne(Fraction(float(x))) for x in v])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- int8 record

def exact_int8_codes(x, d):
    """Exact-rational reference of the int8 code rule for one group."""
    out = []
    for v in x:
        if d == 0:
            out.append(0)
            continue
        qv = Fraction(float(v)) / Fraction(float(d))
        n = math.floor(abs(qv))
        if abs(qv) - n >= Fraction(1, 2):
            n += 1
        out.append(max(-127, min(127, n if qv >= 0 else -n)))
    return out


def test_int8_record_bounds_and_extremes():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, 256)) * np.where(rng.random(256) < 0.02, 20, 1)).astype(np.float16)
    c, d = records.quantize_int8(x.astype(np.float64))
    assert c.dtype == np.int8 and d.dtype == np.float16 and d.shape == (500, 4)
    xh = records.dequantize_int8(c, d)
    dd = np.repeat(d.astype(np.float64), 64, axis=-1)
    assert np.all(np.abs(x - xh) <= dd / 2)
    g = x.astype(np.float64).reshape(500, 4, 64)
    cg = c.reshape(500, 4, 64)
    arg = np.argmax(np.abs(g), axis=-1)
    top = np.take_along_axis(cg, arg[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.abs(c) <= 127)


def test_int8_record_decisions_exact():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 256)) * 7).astype(np.float16)
    c, d = records.quantize_int8(x.astype(np.float64))
    for r in range(40):
        for g in range(4):
            want = exact_int8_codes(x[r, 64 * g:64 * g + 64], d[r, g])
            assert list(c[r, 64 * g:64 * g + 64]) == want


def test_int8_ties_round_away_from_zero_and_zero_group():
    d = 2.0 ** -4
    grp = np.zeros(64)
    grp[0] = 127 * d                                 # amax -> d exactly 2^-4
    grp[1], grp[2], grp[3], grp[4] = 2.5 * d, -2.5 * d, 0.5 * d, -0.5 * d
    x = np.zeros(256)
    x[:64] = grp
    c, s = records.quantize_int8(x)
    assert float(s[0]) == d and float(s[1]) == 0.0
    assert list(c[:5]) == [127, 3, -3, 1, -1]
    assert np.all(c[64:] == 0)


def test_int8_record_size():
    assert records.record_bytes(records.KIND_INT8) == 264


# ---------------------------------------------------------------- q4_0 record

def exact_q4_codes(y, d):
    out = []
    for v in y:
        if d == 0:
            out.append(8)
            continue
        qv = Fraction(v) / Fraction(float(d))
        n = math.floor(qv)
        if qv - n >= Fraction(1, 2):
            n += 1
        out.append(max(0, min(15, n + 8)))
    return out


def test_q4_record_bounds_and_max_code():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((400, 256)) * np.where(rng.random(256) < 0.02, 20, 1)).astype(np.float16)
    c, d = records.quantize_q4(x.astype(np.float64))
    assert c.dtype == np.uint8 and d.shape == (400, 8) and c.max() <= 15
    y = hadamard.rotate(x.astype(np.float64)).reshape(400, 8, 32)
    yh = records.dequantize_q4(c, d).reshape(400, 8, 32)
    dd = np.abs(d.astype(np.float64))[..., None]
    err = np.abs(y - yh)
    clamped = c.reshape(400, 8, 32) == 15
    assert np.all(err[~clamped] <= dd.repeat(32, -1)[~clamped] / 2)
    assert np.all(err <= dd)
    arg = np.argmax(np.abs(y), axis=-1)
    top = np.take_along_axis(c.reshape(400, 8, 32), arg[..., None], -1)[..., 0]
    assert np.all(top == 0)


def test_q4_record_decisions_exact():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((12, 256)) * 5).astype(np.float16)
    y = hadamard.rotate(x.astype(np.float64))
    c, d = records.quantize_q4_rotated(y)
    for r in range(12):
        for b in range(8):
            blk = y[r, 32 * b:32 * b + 32]
            m = blk[np.argmax(np.abs(blk))]
            assert float(d[r, b]) == fraction_to_fp16_rne(-Fraction(m) / 8)
            assert list(c[r, 32 * b:32 * b + 32]) == exact_q4_codes(blk, d[r, b])


def test_q4_integer_block_roundtrips_exactly():
    rng = np.random.default_rng(8)
    for e in (-20, -3, 0, 5):
        k = rng.integers(-7, 8, 32).astype(np.float64)
        k[rng.integers(0, 32)] = -8
        y = np.zeros(256)
        y[:32] = k * 2.0 ** e
        c, d = records.quantize_q4_rotated(y)
        assert float(d[0]) == 2.0 ** e
        assert np.array_equal(records.dequantize_q4(c, d)[:32], y[:32])


def test_q4_ties_sign_ties_and_zero_block():
    y = np.zeros(256)
    # block 0: max -8, so d = 1; ties at +-0.5 and 2.5 round half up
    y[0], y[1], y[2], y[3], y[4] = -8.0, 0.5, -0.5, 2.5, -2.5
    # block 1: +a and -a share the largest magnitude; the first one sets m
    y[32], y[33] = 4.0, -4.0
    c, d = records.quantize_q4_rotated(y)
    assert float(d[0]) == 1.0
    assert list(c[:5]) == [0, 9, 8, 11, 6]
    assert float(d[1]) == -0.5
    assert c[32] == 0 and c[33] == 15               # -4 / -0.5 = 8 -> 16 -> clamped
    assert float(d[2]) == 0.0 and np.all(c[64:96] == 8)


def test_q4_scale_is_rounded_once_and_subnormal_scales():
    y = np.zeros(256)
    y[0] = -8 * (1 + 2.0 ** -11 + 2.0 ** -30)       # -m/8 is the double-rounding trap
    y[32] = 3 * 2.0 ** -18 + 2.0 ** -27              # -m/8 in the fp16 subnormal range
    y[33] = -2 * 2.0 ** -18
    c, d = records.quantize_q4_rotated(y)
    assert float(d[0]) == 1.0009765625
    assert float(d[1]) == fraction_to_fp16_rne(-Fraction(y[32]) / 8) == -3 * 2.0 ** -21
    assert float(d[1]) != 0.0 and abs(float(d[1])) < 2.0 ** -14


def test_q4_record_size():
    assert records.record_bytes(records.KIND_Q4) == 144


# ---------------------------------------------------------------- layout and byte accounting

def test_page_bytes():
    assert layout.page_bytes(records.FMT_INT8, 4) == 540672 == 132 * 4096
    assert layout.page_bytes(records.FMT_Q4_0, 4) == 294912 == 72 * 4096
    assert layout.page_bytes(records.FMT_K8V4, 4) == 417792 == 102 * 4096


def test_strata_bytes_per_token_layer():
    g = GOLDEN["strata_bytes_per_token_layer_two_heads"]
    assert accounting.bytes_per_token_layer(records.FMT_INT8, 2) == g["int8"]
    assert accounting.bytes_per_token_layer(records.FMT_Q4_0, 2) == g["q4_0"]
    k8v4 = accounting.bytes_per_token_layer(records.FMT_K8V4, 2)
    assert k8v4 == 816
    saving = 100 * (1 - k8v4 / g["int8"])
    assert abs(saving - g["k8v4_saving_vs_int8_percent"]["value"]) <= g["k8v4_saving_vs_int8_percent"]["approx"]
    for fmt in (0, 1, 2):
        assert accounting.bytes_per_token_layer_from_pages(fmt, 2) == accounting.bytes_per_token_layer(fmt, 2)


def test_strata_host_kv_size():
    g = GOLDEN["strata_host_kv"]
    per_token = 13 * accounting.bytes_per_token_layer(records.FMT_INT8, 2)
    assert abs(per_token / 1000 - g["bytes_per_token_kb"]["value"]) <= g["bytes_per_token_kb"]["approx"]
    assert abs(131072 * per_token / 2 ** 30 - g["context_128k_gb"]["value"]) <= g["context_128k_gb"]["approx"]


def test_vram_wiki_kv_formula():
    g = GOLDEN["vram_wiki_kv_formula_256k"]
    L, H, D, T = g["layers"], g["kv_heads"], g["head_dim"], g["context"]
    fp16 = accounting.kv_cache_bytes(L, H, D, 2, T)
    assert fp16 == 17_179_869_184
    for key, fmt in (("fp16_gb", "f16"), ("q8_0_gb", "q8_0"), ("q4_0_gb", "q4_0")):
        b = accounting.kv_cache_bytes(L, H, D, accounting.GGML_BITS_PER_ELEM[fmt] / 8, T)
        assert abs(b / 1e9 - g[key]["value"]) <= g[key]["approx"]
    b64 = accounting.kv_cache_bytes(64, H, D, 2, T)
    assert abs(b64 / 1e9 - g["pure_full_attention_64_layers_fp16_gb"]["value"]) <= 0.05
    m = GOLDEN["vram_wiki_1m"]
    assert abs(4 * accounting.kv_cache_bytes(L, H, D, 4.5 / 8, T) / 1e9 - m["q4_0_gb"]["value"]) <= m["q4_0_gb"]["approx"]
    assert 4 * fp16 / 1e9 >= m["fp16_gb_at_least"]


def test_news_pcie_bound():
    g = GOLDEN["news_pcie_bound"]
    per_tok_layer = 2 * 256 * 2 * 2                   # 2 KV heads x 256 x {K,V} x fp16
    assert per_tok_layer == g["bytes_per_token_layer"]
    assert per_tok_layer * g["context"] == g["per_layer_mib"] * 2 ** 20
    total = g["layers"] * per_tok_layer * g["context"]
    assert total == g["total_gib"] * 2 ** 30
    tps = accounting.pcie_tokens_per_second(total, g["link_gib_per_s"] * 2 ** 30)
    assert abs(tps - g["tokens_per_s"]["value"]) <= g["tokens_per_s"]["approx"]


def test_smzdm_per_position_method():
    g = GOLDEN["smzdm_per_position_nvfp4"]
    for ctx, key in ((163840, "gib_at_163840"), (262144, "gib_at_262144")):
        gib = ctx * g["positions_per_token"] * g["bytes_per_position"] / 2 ** 30
        assert abs(gib - g[key]["value"]) <= g[key]["approx"]


# ---------------------------------------------------------------- attention

def brute_attention(q, kh, vh, fmt, scale=1 / 16):
    """Scalar-loop softmax attention with math.exp and an explicit WHT."""
    def wht(v):
        return [sum(exact_sign(i, j) * v[j] for j in range(256)) / 16 for i in range(256)]
    Hq, T, Hkv = len(q), len(kh), len(kh[0])
    G = Hq // Hkv
    kk, vk = records.kinds(fmt)
    out = []
    for h in range(Hq):
        g = h // G
        qq = wht(list(q[h])) if kk == records.KIND_Q4 else list(q[h])
        s = [scale * sum(qq[i] * kh[t][g][i] for i in range(256)) for t in range(T)]
        mx = max(s)
        w = [math.exp(v - mx) for v in s]
        z = sum(w)
        o = [sum(w[t] * vh[t][g][i] for t in range(T)) / z for i in range(256)]
        out.append(wht(o) if vk == records.KIND_Q4 else o)
    return np.array(out)


def quantized_kv(x_k, x_v, fmt):
    kk, vk = records.kinds(fmt)
    kc, ks = records.encode(x_k.astype(np.float64), kk)
    vc, vs = records.encode(x_v.astype(np.float64), vk)
    return records.decode(kc, ks, kk), records.decode(vc, vs, vk)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_attention_matches_brute_force(fmt, T):
    rng = np.random.default_rng(10 + T + 100 * fmt)
    q = rng.standard_normal((4, 256)).astype(np.float16)
    xk = (rng.standard_normal((T, 2, 256)) * 2).astype(np.float16)
    xv = rng.standard_normal((T, 2, 256)).astype(np.float16)
    kh, vh = quantized_kv(xk, xv, fmt)
    got = attention.decode_attention(q, kh, vh, fmt)
    want = brute_attention(q.astype(np.float64), kh, vh, fmt)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_attention_special_cases(fmt):
    rng = np.random.default_rng(20 + fmt)
    H = hadamard.hadamard_matrix()
    kk, vk = records.kinds(fmt)
    q = rng.standard_normal((6, 256)).astype(np.float16)
    xk = rng.standard_normal((5, 1, 256)).astype(np.float16)
    xv = rng.standard_normal((5, 1, 256)).astype(np.float16)
    kh, vh = quantized_kv(xk, xv, fmt)
    back = (lambda o: o @ H) if vk == records.KIND_Q4 else (lambda o: o)
    # T = 1: output is the single value vector (rotated back if stored rotated)
    o1 = attention.decode_attention(q, kh[:1], vh[:1], fmt)
    assert np.allclose(o1, np.broadcast_to(back(vh[0, 0]), o1.shape), atol=1e-12)
    # identical keys, or q = 0: output is the mean value
    same = np.repeat(kh[:1], 5, axis=0)
    mean = back(vh[:, 0].mean(axis=0))
    assert np.allclose(attention.decode_attention(q, same, vh, fmt), mean, atol=1e-12)
    assert np.allclose(attention.decode_attention(np.zeros_like(q), kh, vh, fmt), mean, atol=1e-12)
    # T = 0 gives zeros
    assert np.array_equal(attention.decode_attention(q, kh[:0], vh[:0], fmt), np.zeros((6, 256)))
    # equal queries within a group give equal outputs
    qq = np.repeat(q[:1], 6, axis=0)
    o = attention.decode_attention(qq, kh, vh, fmt)
    assert np.array_equal(o, np.repeat(o[:1], 6, axis=0))


def test_attention_shift_and_order_invariance():
    rng = np.random.default_rng(30)
    q = rng.standard_normal((6, 256))
    kh = rng.standard_normal((50, 1, 256)) * 3
    vh = rng.standard_normal((50, 1, 256))
    base = attention.decode_attention(q, kh, vh, records.FMT_INT8)
    u = rng.standard_normal(256) * 4                # adds <q_h, u> to every score of head h
    shifted = attention.decode_attention(q, kh + u, vh, records.FMT_INT8)
    assert np.allclose(base, shifted, atol=1e-10)
    perm = rng.permutation(50)
    assert np.allclose(base, attention.decode_attention(q, kh[perm], vh[perm], records.FMT_INT8), atol=1e-12)
    big = attention.decode_attention(q * 1e3, kh, vh, records.FMT_INT8)
    assert np.all(np.isfinite(big))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_attention_chunked_equals_direct(fmt):
    rng = np.random.default_rng(40 + fmt)
    q = rng.standard_normal((24, 256)).astype(np.float16)
    kh = rng.standard_normal((1000, 4, 256))
    vh = rng.standard_normal((1000, 4, 256))
    a = attention.decode_attention(q, kh, vh, fmt)
    b = attention.decode_attention_chunked(q, lambda t0, t1: (kh[t0:t1], vh[t0:t1]), 1000, 4, fmt, chunk=128)
    assert np.allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------- layout round trip

@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_layout_roundtrip_and_zero_tail(fmt):
    rng = np.random.default_rng(50 + fmt)
    T = 300
    x = rng.standard_normal((T, 4, 256)).astype(np.float16)
    kk, vk = records.kinds(fmt)
    kc, ks = records.encode(x.astype(np.float64), kk)
    vc, vs = records.encode(-x.astype(np.float64), vk)
    pages = layout.pack_pages(kc, ks, vc, vs, fmt)
    assert pages.shape == (2, layout.page_bytes(fmt, 4))
    a, b, c, d = layout.unpack_pages(pages, fmt, 4)
    assert np.array_equal(a[:T], kc) and np.array_equal(b[:T], ks)
    assert np.array_equal(c[:T], vc) and np.array_equal(d[:T], vs)
    assert not np.any(a[T:]) and not np.any(c[T:])


def test_layout_worked_example_q4():
    """A page whose K token 0 has code[e] = e % 16 and V element 5 has code = token % 16."""
    kc = np.full((256, 1, 256), 8, np.uint8)
    kc[0, 0] = np.arange(256) % 16
    vc = np.full((256, 1, 256), 8, np.uint8)
    vc[:, 0, 5] = np.arange(256) % 16
    ks = np.ones((256, 1, 8), np.float16)
    vs = np.full((256, 1, 8), 2.0, np.float16)
    page = layout.pack_pages(kc, ks, vc, vs, records.FMT_Q4_0)[0]
    # K row 0, slice s, block j, byte w holds elements 32j+4s+w (low) and 32j+16+4s+w (high):
    # both are congruent to 4s+w mod 16, so the byte is (4s+w) * 0x11.
    assert list(page[0:4]) == [0x00, 0x11, 0x22, 0x33]          # s=0, j=0
    assert list(page[32:36]) == [0x44, 0x55, 0x66, 0x77]        # s=1, j=0
    assert page[128] == 0x88                                    # K row 1 is all code 8
    # V plane starts after the K plane (36,864 B); row of element 5 starts 5*128 B in.
    vrow = page[36864 + 5 * 128:36864 + 6 * 128]
    # byte 16G+i holds tokens 32G+i (low) and 32G+16+i (high): (i, i) mod 16
    assert list(vrow[:3]) == [0x00, 0x11, 0x22]
    # V scales: 8 rows of 256 fp16 after 256 code rows
    vsc = page[36864 + 256 * 128:36864 + 256 * 128 + 16].view(np.float16)
    assert np.all(vsc == 2.0)
