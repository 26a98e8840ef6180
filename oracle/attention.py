"""fp64 GQA decode attention over dequantized KV (oracle).

What is computed, per sequence and query head h (KV-offload news page,
section "缓存为何不能直接搬走？": each decoded token reads the whole KV of
every full-attention layer; VRAM wiki page, section "一、为什么 256K 上下文的
显存这么吓人": 24 query heads share 4 KV heads, head_dim 256; Strata page,
section "4-bit KV 缓存：先旋转，再压到 4-bit": Q is rotated like K, the output
is mixed from rotated V and multiplied by H):

    g   = h // (Hq / Hkv)                   contiguous GQA groups
    q'  = H q  if K is stored rotated, else q
    s_t = <q', k^_t> * scale                t < T (context length)
    p   = softmax(s)                         max-subtracted, fp64
    o'  = sum_t p_t v^_t
    o   = H o' if V is stored rotated, else o'

k^ and v^ are the dequantized record values (rotated domain for q4 records).
The quantization is the only lossy step, so on dequantized values this is
the exact mathematics, rounded once per fp64 operation.

Readings: scale = 1/sqrt(256) = 1/16 by default (the pages give none);
q and k arrive after any positional encoding; T = 0 gives a zero output.

Several new tokens per sequence (speculative drafts checked in one pass, or a
chunk of a prompt; smzdm roundup post.smzdm.com/p/ad79lwwz, section
"二、一周跨卡实测": MTP drafts and prefill rates): the n_q newest tokens of a
sequence of T tokens are its queries, query j at position T - n_q + j, and
each attends causally, to tokens 0 .. T - n_q + j (reading: the usual causal
mask of a decoder; the pages give no other rule). Each query is therefore
the decode attention above over its own prefix.
"""

from __future__ import annotations

import numpy as np

from .hadamard import rotate
from .records import rotates_output, rotates_query

DEFAULT_SCALE = 1.0 / 16.0


def decode_attention(q, k_hat, v_hat, fmt: int, scale: float = DEFAULT_SCALE) -> np.ndarray:
    """One sequence. q [Hq, 256] (fp16 values); k_hat, v_hat [T, Hkv, 256] float64.

    Returns o [Hq, 256] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    T, hkv = k_hat.shape[0], k_hat.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    if T == 0:
        return out
    qr = rotate(q) if rotates_query(fmt) else q
    for g in range(hkv):
        qs = qr[g * G:(g + 1) * G]                      # [G, D]
        s = (qs @ k_hat[:, g, :].T) * scale             # [G, T]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        o = (p @ v_hat[:, g, :]) / p.sum(axis=1, keepdims=True)
        out[g * G:(g + 1) * G] = o
    return rotate(out) if rotates_output(fmt) else out


def decode_attention_chunked(q, get_kv, T: int, hkv: int, fmt: int,
                             scale: float = DEFAULT_SCALE, chunk: int = 32768) -> np.ndarray:
    """Same result as ``decode_attention`` for contexts too large to dequantize at once.

    ``get_kv(t0, t1)`` returns (k_hat, v_hat) float64 [t1-t0, Hkv, 256]. Scores
    of all T tokens are kept (fp64, Hq x T), then the softmax and the weighted
    sum are taken chunk by chunk in token order.
    """
    q = np.asarray(q, dtype=np.float64)
    hq, D = q.shape
    G = hq // hkv
    out = np.zeros((hq, D))
    if T == 0:
        return out
    qr = rotate(q) if rotates_query(fmt) else q
    s = np.empty((hq, T))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        kh, _ = get_kv(t0, t1)
        for g in range(hkv):
            s[g * G:(g + 1) * G, t0:t1] = (qr[g * G:(g + 1) * G] @ kh[:, g, :].T) * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    acc = np.zeros((hq, D))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        _, vh = get_kv(t0, t1)
        for g in range(hkv):
            acc[g * G:(g + 1) * G] += p[g * G:(g + 1) * G, t0:t1] @ vh[:, g, :]
    out = acc / p.sum(axis=1, keepdims=True)
    return rotate(out) if rotates_output(fmt) else out


def multi_query_attention(q, k_hat, v_hat, fmt: int, scale: float = DEFAULT_SCALE) -> np.ndarray:
    """The n_q newest tokens of one sequence as queries. q [n_q, Hq, 256] (fp16 values);
    k_hat, v_hat [T, Hkv, 256] float64 (T >= 0 tokens, the queries' own tokens included).

    Query j sees tokens 0 .. T - n_q + j (none if that is negative). Returns [n_q, Hq, 256].
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, T = q.shape[0], k_hat.shape[0]
    out = np.zeros(q.shape)
    for j in range(n_q):
        seen = max(0, T - n_q + j + 1)
        out[j] = decode_attention(q[j], k_hat[:seen], v_hat[:seen], fmt, scale)
    return out
