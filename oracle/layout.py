"""Byte layout of the paged KV pool (oracle packer and unpacker).

The Strata page (section "KV 从显存搬进内存之后发生了什么") speaks of pages,
blocks and slots looked up in a table but fixes no byte layout, so the layout
is a design choice. This module writes it out from its specification, without
any reference to how the GPU library computes offsets:

* A page holds 256 consecutive tokens of one sequence and one layer, for all
  KV heads: for h = 0 .. Hkv-1, the K plane of head h, then its V plane.
  Logical token p of a sequence lives in page ``block_table[p // 256]``,
  row ``p % 256``.
* Plane sizes: int8 67,584 B (256 x 256 codes + 256 x 4 fp16 scales);
  q4 and fp4 36,864 B (256 x 128 code bytes + 256 x 8 fp16 scales). So a page
  is 540,672 B (int8), 294,912 B (q4_0, fp4) or 417,792 B (k8v4) for 4 KV
  heads. The fp4 record uses the q4 byte layout below (4-bit codes, 8 scales).
  fp8: 66,048 B (256 x 256 codes + 256 x 1 fp16 scale), 528,384 B a page; its
  code bytes are placed exactly like int8 codes, with one scale per token.
* K plane, token-major. Codes: 256 rows (one per token) of 256 B (int8) or
  128 B (q4), then scales: 256 rows of 4 (int8) or 8 (q4) little-endian fp16.
  Inside a code row the bytes of each 32-element block are spread over four
  slices s = 0..3 so that slice s of all eight blocks is contiguous:
    q4:   byte 32*s + 4*j + w (j = block 0..7, w = 0..3) =
          code[32j + 4s + w] | code[32j + 16 + 4s + w] << 4
    int8: byte 64*s + 8*j + w (w = 0..7) = code[32j + 8s + w]
* V plane, element-major (transposed). Codes: 256 rows (one per head
  element) holding that element for all 256 tokens, then scales: 8 (q4) or
  4 (int8) rows of 256 fp16, one row per block / group, one entry per token
  (fp8: one row).
    int8, fp8: byte t of row e = code of token t, element e
    q4:   byte 16*G + i of row e (G = 0..7, i = 0..15) =
          code[token 32G + i] | code[token 32G + 16 + i] << 4 (element e)

Each vector still occupies exactly its record size (264 B or 144 B); only
the arrangement differs from a record-after-record layout.
"""

from __future__ import annotations

import numpy as np

from .records import HEAD_DIM, KIND_FP4, KIND_FP8, KIND_INT8, KIND_Q4, kinds

PAGE_TOKENS = 256
BYTE_KINDS = (KIND_INT8, KIND_FP8)  # one byte per code


def n_scales(kind: str) -> int:
    return {KIND_INT8: 4, KIND_FP8: 1}.get(kind, 8)


def code_row_bytes(kind: str) -> int:
    return 256 if kind in BYTE_KINDS else 128


def plane_bytes(kind: str) -> int:
    return PAGE_TOKENS * code_row_bytes(kind) + PAGE_TOKENS * n_scales(kind) * 2


def page_bytes(fmt: int, n_kv_heads: int) -> int:
    kk, vk = kinds(fmt)
    return n_kv_heads * (plane_bytes(kk) + plane_bytes(vk))


def _k_row_maps(kind: str):
    """For each byte of a K code row: the element(s) it holds (built from the loops of the spec)."""
    if kind in BYTE_KINDS:
        elem = np.zeros(256, np.int64)
        for s in range(4):
            for j in range(8):
                for w in range(8):
                    elem[64 * s + 8 * j + w] = 32 * j + 8 * s + w
        return elem, None
    lo = np.zeros(128, np.int64)
    hi = np.zeros(128, np.int64)
    for s in range(4):
        for j in range(8):
            for w in range(4):
                lo[32 * s + 4 * j + w] = 32 * j + 4 * s + w
                hi[32 * s + 4 * j + w] = 32 * j + 16 + 4 * s + w
    return lo, hi


_KMAP = {k: _k_row_maps(k) for k in (KIND_INT8, KIND_Q4, KIND_FP4, KIND_FP8)}


def _k_row_bytes(codes: np.ndarray, kind: str) -> np.ndarray:
    """codes [..., 256] (int8, or 0..15) -> K code rows [..., R] uint8."""
    a, b = _KMAP[kind]
    if kind == KIND_INT8:
        return codes.astype(np.int8).view(np.uint8)[..., a]
    if kind == KIND_FP8:
        return codes.astype(np.uint8)[..., a]
    c = codes.astype(np.uint8)
    return c[..., a] | (c[..., b] << 4)


def _k_row_codes(rows: np.ndarray, kind: str) -> np.ndarray:
    """Inverse of ``_k_row_bytes``."""
    a, b = _KMAP[kind]
    if kind == KIND_INT8:
        out = np.zeros(rows.shape[:-1] + (HEAD_DIM,), np.int8)
        out[..., a] = rows.view(np.int8)
        return out
    out = np.zeros(rows.shape[:-1] + (HEAD_DIM,), np.uint8)
    if kind == KIND_FP8:
        out[..., a] = rows
        return out
    out[..., a] = rows & 0xF
    out[..., b] = rows >> 4
    return out


def _v_rows(codes_page: np.ndarray, kind: str) -> np.ndarray:
    """codes of one page and head [256 tok, 256 elem] -> V code rows [256 elem, R] uint8."""
    t = codes_page.T  # [elem, tok]
    if kind == KIND_INT8:
        return np.ascontiguousarray(t.astype(np.int8).view(np.uint8))
    if kind == KIND_FP8:
        return np.ascontiguousarray(t.astype(np.uint8))
    c = t.astype(np.uint8)
    out = np.zeros((HEAD_DIM, 128), np.uint8)
    for g in range(8):
        for i in range(16):
            out[:, 16 * g + i] = c[:, 32 * g + i] | (c[:, 32 * g + 16 + i] << 4)
    return out


def _v_codes(rows: np.ndarray, kind: str) -> np.ndarray:
    """Inverse of ``_v_rows``: [256 elem, R] -> [256 tok, 256 elem]."""
    if kind == KIND_INT8:
        return np.ascontiguousarray(rows.view(np.int8).T)
    if kind == KIND_FP8:
        return np.ascontiguousarray(rows.T)
    c = np.zeros((HEAD_DIM, PAGE_TOKENS), np.uint8)
    for g in range(8):
        for i in range(16):
            b = rows[:, 16 * g + i]
            c[:, 32 * g + i] = b & 0xF
            c[:, 32 * g + 16 + i] = b >> 4
    return np.ascontiguousarray(c.T)


def _pad_pages(a: np.ndarray, n_pages: int) -> np.ndarray:
    out = np.zeros((n_pages * PAGE_TOKENS,) + a.shape[1:], a.dtype)
    out[: a.shape[0]] = a
    return out


def pack_pages(k_codes, k_scales, v_codes, v_scales, fmt: int) -> np.ndarray:
    """Pack one sequence's records (tokens in logical order) into pages.

    k_codes/v_codes [T, Hkv, 256]; k_scales/v_scales [T, Hkv, G] fp16.
    Returns uint8 [ceil(T/256), page_bytes]; rows past T are zero.
    """
    kk, vk = kinds(fmt)
    T, hkv = k_codes.shape[0], k_codes.shape[1]
    n_pages = -(-T // PAGE_TOKENS)
    pk, pv = plane_bytes(kk), plane_bytes(vk)
    out = np.zeros((n_pages, page_bytes(fmt, hkv)), np.uint8)
    kc, ks = _pad_pages(k_codes, n_pages), _pad_pages(k_scales.astype(np.float16), n_pages)
    vc, vs = _pad_pages(v_codes, n_pages), _pad_pages(v_scales.astype(np.float16), n_pages)
    for p in range(n_pages):
        sl = slice(p * PAGE_TOKENS, (p + 1) * PAGE_TOKENS)
        for h in range(hkv):
            base = h * (pk + pv)
            krow = _k_row_bytes(kc[sl, h], kk)  # [256, R]
            kcb = krow.size
            out[p, base:base + kcb] = krow.reshape(-1)
            out[p, base + kcb:base + pk] = np.ascontiguousarray(ks[sl, h]).reshape(-1).view(np.uint8)
            vbase = base + pk
            vrow = _v_rows(vc[sl, h], vk)  # [256, R]
            vcb = vrow.size
            out[p, vbase:vbase + vcb] = vrow.reshape(-1)
            out[p, vbase + vcb:vbase + pv] = np.ascontiguousarray(vs[sl, h].T).reshape(-1).view(np.uint8)
    return out


def unpack_pages(pages: np.ndarray, fmt: int, n_kv_heads: int):
    """Inverse of ``pack_pages``: uint8 [P, page_bytes] -> (k_codes, k_scales, v_codes, v_scales),
    each with P*256 token rows in page order."""
    kk, vk = kinds(fmt)
    pk, pv = plane_bytes(kk), plane_bytes(vk)
    P = pages.shape[0]
    T = P * PAGE_TOKENS
    kc = np.zeros((T, n_kv_heads, HEAD_DIM), np.int8 if kk == KIND_INT8 else np.uint8)
    vc = np.zeros((T, n_kv_heads, HEAD_DIM), np.int8 if vk == KIND_INT8 else np.uint8)
    ks = np.zeros((T, n_kv_heads, n_scales(kk)), np.float16)
    vs = np.zeros((T, n_kv_heads, n_scales(vk)), np.float16)
    for p in range(P):
        sl = slice(p * PAGE_TOKENS, (p + 1) * PAGE_TOKENS)
        for h in range(n_kv_heads):
            base = h * (pk + pv)
            R = code_row_bytes(kk)
            krows = pages[p, base:base + PAGE_TOKENS * R].reshape(PAGE_TOKENS, R)
            kc[sl, h] = _k_row_codes(krows, kk)
            ks[sl, h] = pages[p, base + PAGE_TOKENS * R:base + pk].copy().view(np.float16).reshape(PAGE_TOKENS, -1)
            vbase = base + pk
            Rv = code_row_bytes(vk)
            vrows = pages[p, vbase:vbase + HEAD_DIM * Rv].reshape(HEAD_DIM, Rv)
            vc[sl, h] = _v_codes(vrows, vk)
            vs[sl, h] = pages[p, vbase + HEAD_DIM * Rv:vbase + pv].copy().view(np.float16).reshape(-1, PAGE_TOKENS).T
    return kc, ks, vc, vs
