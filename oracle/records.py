"""The int8, q4_0, fp4 and fp8 vector records (oracle).

Strata page, section "三种 KV 格式横向对比": int8 (the default, 1,056 B per
token per layer for the K and V of two KV heads, i.e. 264 B per 256-element
vector), q4_0 (576 B, i.e. 144 B per vector, after the Walsh-Hadamard
rotation of section "4-bit KV 缓存：先旋转，再压到 4-bit") and k8v4 (K kept in
8 bits, V rotated and stored in 4 bits, 23% less than int8, i.e. 816 B).

The pages give the sizes and the rotation, not the rounding rules. Readings
taken here (each is a plain choice consistent with the sizes):

int8 record, per group of 64 elements (4 groups, 4 fp16 scales + 256 codes):
  a = max |x_j|;  d = fp16 round-to-nearest-even of the exact quotient a/127;
  d == 0 -> all codes 0; else c_j = clamp(round_half_away_from_zero(x_j / d),
  -127, 127), computed from the stored d. Dequantized value c_j * d.

q4_0 record, on y = H x, per block of 32 elements (8 blocks, 8 fp16 scales +
128 bytes of 4-bit codes), following the ggml q4_0 convention that the name
points to:
  m = the y_j of largest |y_j| (first index on ties);
  d = fp16 round-to-nearest-even of the exact value -m/8;
  d == 0 -> all codes 8; else c_j = clamp(floor(y_j / d + 1/2) + 8, 0, 15)
  (round half up, then offset 8), computed from the stored d.
  Dequantized (rotated-domain) value (c_j - 8) * d.

Every decision is taken on exact values: the quotient x/d (or y/d) is formed
in fp64, and it cannot land within fp64 rounding of a half-integer unless it
is one exactly (x, y, d are multiples of 2^-28 below 2^20, so a non-tie
quotient stays at least 2^-44 away from a tie, far above the 2^-49 error of
an fp64 quotient below 16). The halves are detected as ``frac >= 0.5`` on
the exact remainder, never by adding 0.5 in floating point.

A d that overflows fp16 (|a| or |m| beyond what fp16 can scale) is out of the
method's domain; the rules above still give codes (0 for int8, 8 for q4_0),
and the dequantized values are then not finite.

fp4 record (a block-scaled 4-bit floating-point format; the smzdm roundup,
post.smzdm.com/p/ad79lwwz, section "一、先修正一笔老账", lists NVFP4 KV among the
formats of other engines at 288 B per position, i.e. 144 B per vector, and
the builder declares its own layout). Declared here: on y = H x like q4_0,
per block of 32 elements (8 blocks, 8 fp16 scales + 128 bytes of 4-bit
codes, in q4_0's byte layout):
  a = max |y_j|; a == 0 -> d = 0 and all codes 0. Otherwise the block
  exponent e = floor(log2 a) - 2 (the shared-exponent rule of the OCP
  microscaling formats, 2 being the largest exponent of the e2m1 element),
  clamped to [-23, 13] so that every dequantized value is an fp16 number;
  d = 2^e, stored as an fp16 (exactly).
  Each |y_j| / d (exact: d is a power of two) is rounded to the nearest value
  of the e2m1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even grid index,
  values above 6 to 6 (saturation). The code is the grid index (0..7), plus
  8 (the sign bit) when y_j < 0 and the index is not 0.
  Dequantized (rotated-domain) value: +-grid[code & 7] * d.

fp8 record (the same roundup section lists an FP8 KV format at 516 B per
position, i.e. 258 B per vector: 256 one-byte codes and one 2-byte scale).
Declared here: not rotated (like int8), one scale for the whole vector, codes
in the OCP FP8 E4M3 encoding (1 sign, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F and 0xFF are NaN, so
the largest value is 448 = 1.75 * 2^8; no infinities):
  a = max |x_j|; d = fp16 round-to-nearest-even of the exact quotient a/448
  (the quotient in fp64 is never within its rounding error of an fp16 tie
  unless it is one: 448 = 7 * 64, and a/7 either terminates or repeats 001);
  d == 0 -> all codes 0. Otherwise |x_j| / d (exact decision in fp64, as for
  int8) goes to the nearest E4M3 magnitude, ties to the even code (even
  mantissa), magnitudes beyond 448 to 448 (saturation); the sign bit 0x80 is
  set when x_j < 0 and the magnitude code is not 0. Dequantized value
  +-E4M3(code & 0x7F) * d.
"""

from __future__ import annotations

import numpy as np

from .hadamard import rotate

FMT_INT8, FMT_Q4_0, FMT_K8V4, FMT_FP4, FMT_FP8 = 0, 1, 2, 3, 4
FORMATS = {"int8": FMT_INT8, "q4_0": FMT_Q4_0, "k8v4": FMT_K8V4, "fp4": FMT_FP4, "fp8": FMT_FP8}

KIND_INT8, KIND_Q4, KIND_FP4, KIND_FP8 = "int8", "q4", "fp4", "fp8"
ROTATED_KINDS = (KIND_Q4, KIND_FP4)
FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FP4_EMIN, FP4_EMAX = -23, 13

HEAD_DIM = 256
INT8_GROUP = 64
Q4_BLOCK = 32


def kinds(fmt: int):
    """(K record kind, V record kind) of a cache format."""
    if fmt == FMT_INT8:
        return KIND_INT8, KIND_INT8
    if fmt == FMT_Q4_0:
        return KIND_Q4, KIND_Q4
    if fmt == FMT_K8V4:
        return KIND_INT8, KIND_Q4
    if fmt == FMT_FP4:
        return KIND_FP4, KIND_FP4
    if fmt == FMT_FP8:
        return KIND_FP8, KIND_FP8
    raise ValueError(f"unknown format {fmt}")


def rotates_query(fmt: int) -> bool:
    """The query is rotated exactly when K is stored rotated (q4_0, fp4)."""
    return kinds(fmt)[0] in ROTATED_KINDS


def rotates_output(fmt: int) -> bool:
    """The output is rotated back exactly when V is stored rotated."""
    return kinds(fmt)[1] in ROTATED_KINDS


def fp16_rne(v) -> np.ndarray:
    """Round float64 values to fp16 once, to nearest, ties to even.

    numpy converts a double to a half directly from its bits (one rounding,
    overflow to +-inf), which is what is needed when the double holds the
    exact value being rounded.
    """
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def _round_half_away(q: np.ndarray) -> np.ndarray:
    a = np.abs(q)
    r = np.floor(a)
    r = r + ((a - r) >= 0.5)
    return np.copysign(r, q)


def _round_half_up(q: np.ndarray) -> np.ndarray:
    r = np.floor(q)
    return r + ((q - r) >= 0.5)


def quantize_int8(x) -> tuple[np.ndarray, np.ndarray]:
    """int8 record of vectors x [..., 256] -> (codes int8 [..., 256], scales fp16 [..., 4])."""
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(x.shape[:-1] + (HEAD_DIM // INT8_GROUP, INT8_GROUP))
    a = np.max(np.abs(g), axis=-1)
    d16 = fp16_rne(a / 127.0)  # a/127 in fp64 then one rounding: see test pin
    d = d16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d != 0, g / np.where(d != 0, d, 1.0), 0.0)
    c = np.clip(_round_half_away(q), -127, 127)
    return c.reshape(x.shape).astype(np.int8), d16


def dequantize_int8(codes, scales) -> np.ndarray:
    c = np.asarray(codes, dtype=np.float64)
    d = np.asarray(scales, dtype=np.float64)
    g = c.reshape(c.shape[:-1] + (HEAD_DIM // INT8_GROUP, INT8_GROUP))
    return (g * d[..., None]).reshape(c.shape)


def quantize_q4_rotated(y) -> tuple[np.ndarray, np.ndarray]:
    """q4_0 record of already-rotated vectors y [..., 256] -> (codes uint8 0..15, scales fp16 [..., 8])."""
    y = np.asarray(y, dtype=np.float64)
    b = y.reshape(y.shape[:-1] + (HEAD_DIM // Q4_BLOCK, Q4_BLOCK))
    idx = np.argmax(np.abs(b), axis=-1)  # first index on ties
    m = np.take_along_axis(b, idx[..., None], axis=-1)[..., 0]
    d16 = fp16_rne(-m / 8.0)  # -m/8 is exact in fp64
    d = d16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d != 0, b / np.where(d != 0, d, 1.0), 0.0)
    c = np.clip(_round_half_up(q) + 8, 0, 15)
    return c.reshape(y.shape).astype(np.uint8), d16


def quantize_q4(x) -> tuple[np.ndarray, np.ndarray]:
    """q4_0 record of vectors x [..., 256]: rotate by H, then quantize."""
    return quantize_q4_rotated(rotate(x))


def dequantize_q4(codes, scales) -> np.ndarray:
    """Rotated-domain values (c - 8) * d of a q4_0 record."""
    c = np.asarray(codes, dtype=np.float64) - 8.0
    d = np.asarray(scales, dtype=np.float64)
    b = c.reshape(c.shape[:-1] + (HEAD_DIM // Q4_BLOCK, Q4_BLOCK))
    return (b * d[..., None]).reshape(c.shape)


def fp4_index(v) -> np.ndarray:
    """e2m1 grid index of magnitudes v >= 0 (exact values): nearest, ties to the even
    index, saturating at 6. The midpoints between grid values are 0.25, 0.75, 1.25,
    1.75, 2.5, 3.5 and 5; at a midpoint the even index wins, so the boundary belongs
    to the lower value when that one has an even index."""
    v = np.asarray(v, dtype=np.float64)
    return ((v > 0.25).astype(np.int64) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) + (v > 2.5)
            + (v >= 3.5) + (v > 5.0))


def quantize_fp4_rotated(y) -> tuple[np.ndarray, np.ndarray]:
    """fp4 record of already-rotated vectors y [..., 256] -> (codes uint8 0..15, scales fp16 [..., 8])."""
    y = np.asarray(y, dtype=np.float64)
    b = y.reshape(y.shape[:-1] + (HEAD_DIM // Q4_BLOCK, Q4_BLOCK))
    a = np.max(np.abs(b), axis=-1)
    _, ex = np.frexp(a)                        # a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.clip(ex - 1 - 2, FP4_EMIN, FP4_EMAX)
    d = np.where(a > 0, np.ldexp(1.0, e), 0.0)
    v = np.abs(b) / np.where(d > 0, d, 1.0)[..., None]  # exact: d is a power of two
    idx = np.where(d[..., None] > 0, fp4_index(v), 0)
    c = idx + 8 * ((b < 0) & (idx > 0))
    return c.reshape(y.shape).astype(np.uint8), fp16_rne(d)


def quantize_fp4(x) -> tuple[np.ndarray, np.ndarray]:
    """fp4 record of vectors x [..., 256]: rotate by H, then quantize."""
    return quantize_fp4_rotated(rotate(x))


def dequantize_fp4(codes, scales) -> np.ndarray:
    """Rotated-domain values +-grid[c & 7] * d of an fp4 record."""
    c = np.asarray(codes, dtype=np.int64)
    mag = FP4_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    d = np.asarray(scales, dtype=np.float64)
    b = mag.reshape(c.shape[:-1] + (HEAD_DIM // Q4_BLOCK, Q4_BLOCK))
    return (b * d[..., None]).reshape(c.shape)


def e4m3_magnitudes() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E, in code order
    (which is increasing order): exponent field e = code >> 3, mantissa m = code & 7;
    e == 0: m * 2^-9, else (1 + m/8) * 2^(e - 7)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


E4M3 = e4m3_magnitudes()
FP8_MAX = float(E4M3[-1])  # 448


def e4m3_code(v) -> np.ndarray:
    """Magnitude code (0..126) of exact values v >= 0: the nearest E4M3 magnitude, ties
    to the even code, beyond 448 -> 448."""
    v = np.asarray(v, dtype=np.float64)
    hi = np.clip(np.searchsorted(E4M3, v), 1, 126)   # E4M3[hi - 1] < v <= E4M3[hi] inside the range
    lo = hi - 1
    dl, dh = v - E4M3[lo], E4M3[hi] - v
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    c = np.where(pick_hi, hi, lo)
    return np.where(v >= FP8_MAX, 126, np.where(v <= 0, 0, c))


def quantize_fp8(x) -> tuple[np.ndarray, np.ndarray]:
    """fp8 record of vectors x [..., 256] -> (codes uint8 [..., 256], scales fp16 [..., 1])."""
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1, keepdims=True)
    d16 = fp16_rne(a / FP8_MAX)
    d = d16.astype(np.float64)
    mag = np.where(d != 0, e4m3_code(np.abs(x) / np.where(d != 0, d, 1.0)), 0)
    c = mag + 0x80 * ((x < 0) & (mag > 0))
    return c.astype(np.uint8), d16


def dequantize_fp8(codes, scales) -> np.ndarray:
    """Values +-E4M3(c & 0x7F) * d of an fp8 record (codes 0x7F / 0xFF, NaN, never occur)."""
    c = np.asarray(codes, dtype=np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN code (0x7F / 0xFF) in an fp8 record")
    mag = E4M3[c & 0x7F] * np.where(c & 0x80, -1.0, 1.0)
    return mag * np.asarray(scales, dtype=np.float64)


def encode(x, kind: str):
    return {KIND_INT8: quantize_int8, KIND_Q4: quantize_q4, KIND_FP4: quantize_fp4,
            KIND_FP8: quantize_fp8}[kind](x)


def decode(codes, scales, kind: str):
    return {KIND_INT8: dequantize_int8, KIND_Q4: dequantize_q4, KIND_FP4: dequantize_fp4,
            KIND_FP8: dequantize_fp8}[kind](codes, scales)


def record_bytes(kind: str) -> int:
    """Bytes of one 256-element vector record: codes plus fp16 scales."""
    if kind == KIND_INT8:
        return HEAD_DIM + 2 * (HEAD_DIM // INT8_GROUP)
    if kind == KIND_FP8:
        return HEAD_DIM + 2
    return HEAD_DIM // 2 + 2 * (HEAD_DIM // Q4_BLOCK)
