"""Helpers shared by the GPU tests: oracle-packed pools, tolerance checks."""

from __future__ import annotations

import numpy as np

import kvsynth
from oracle import attention, layout, records

ATOL = 2e-3   # max-abs error allowed against the fp64 oracle on dequantized values
RTOL_L2 = 1e-3  # relative L2 error allowed


def fmt_id(fmt: str) -> int:
    return records.FORMATS[fmt]


def oracle_records(k, v, fmt):
    """Records of K and V [T, Hkv, 256] (fp16) -> (kc, ks, vc, vs)."""
    kk, vk = records.kinds(fmt_id(fmt))
    kc, ks = records.encode(k.astype(np.float64), kk)
    vc, vs = records.encode(v.astype(np.float64), vk)
    return kc, ks, vc, vs


def dequantized(kc, ks, vc, vs, fmt):
    kk, vk = records.kinds(fmt_id(fmt))
    return records.decode(kc, ks, kk), records.decode(vc, vs, vk)


class Sequence:
    """One sequence's inputs, its oracle records and its logical pages."""

    def __init__(self, cfg, layer, seq, T, fmt, n_kv_heads=4, k=None, v=None):
        self.T, self.fmt = T, fmt
        if k is None:
            k, v = kvsynth.kv_tokens_np(cfg, layer, seq, 0, T, n_kv_heads)
        self.k, self.v = k, v
        self.rec = oracle_records(k, v, fmt)
        self.pages = layout.pack_pages(*self.rec, fmt_id(fmt)) if T > 0 else np.zeros((0, 0), np.uint8)
        self.n_pages = self.pages.shape[0]

    def hat(self):
        return dequantized(*self.rec, self.fmt)


def place_pages(seqs, n_pool_pages, seed, page_bytes):
    """Scatter the sequences' logical pages over a pool with a seeded permutation.

    Returns (pool bytes uint8 [n_pool_pages * page_bytes], block tables int32 [B, max_pages]).
    Unused pool pages hold seeded garbage bytes.
    """
    total = sum(s.n_pages for s in seqs)
    assert total <= n_pool_pages
    perm = kvsynth.permutation_np(seed, n_pool_pages)
    rng = np.random.default_rng(seed + 1)
    pool = rng.integers(0, 256, n_pool_pages * page_bytes, dtype=np.uint8)
    max_pages = max(1, max(s.n_pages for s in seqs))
    bt = np.zeros((len(seqs), max_pages), np.int32)
    nxt = 0
    for b, s in enumerate(seqs):
        for p in range(s.n_pages):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, p] = phys
            pool[phys * page_bytes:(phys + 1) * page_bytes] = s.pages[p]
    return pool, bt


def oracle_out(q, seqs, fmt):
    outs = []
    for b, s in enumerate(seqs):
        if s.T == 0:
            outs.append(np.zeros((q.shape[1], 256)))
            continue
        kh, vh = s.hat()
        outs.append(attention.decode_attention(q[b], kh, vh, fmt_id(fmt)))
    return np.stack(outs)


def errors(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / den) if den > 0 else float(np.linalg.norm(got - want))
    return max_abs, rel


def assert_close(got, want, atol=ATOL, rtol_l2=RTOL_L2, what=""):
    max_abs, rel = errors(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= atol and rel <= rtol_l2, f"{what}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}"
    return max_abs, rel
