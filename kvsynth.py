"""Seeded synthetic inputs for the quantized paged KV decode path.

This module only draws numbers. It holds none of the method's arithmetic
(no rotation, no quantizer, no attention), so both the fp64 oracle and the
HIP path can take their inputs from it without sharing any computation.

Value distribution (the workloads the KV-offload pages describe are real
Qwen3.8 activations; these stand in for them):

* K and V entries are N(0, 1). For every (layer, KV head, K|V) four fixed
  head channels are multiplied by 20, the outlier channels that the Strata
  page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文",
  section "4-bit KV 缓存：先旋转，再压到 4-bit") says the rotation spreads
  across the head. Values are cast to fp16 with round-to-nearest-even.
* Q entries are N(0, 1), cast to fp16.
* The outlier channel sets of a (config, layer) come from
  ``numpy.random.default_rng(1000 * cfg + layer).choice(256, 4, replace=False)``,
  drawn per KV head, first for K then for V.

Two sources of bulk normals exist:

* ``*_np``: numpy PCG64 streams keyed by (cfg, layer, seq, page, kind), so a
  token range can be drawn page by page and any sub-range is reproducible.
  Tests use these, at sizes the oracle finishes in seconds.
* ``*_torch``: a ``torch.Generator`` on the target device, seeded with
  ``1000 * cfg + 100 * seq + layer``; used to fill the large benchmark pools
  in device memory quickly. A check at full size copies the drawn fp16
  tensors back to the host and hands the same values to the oracle.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 256
PAGE_TOKENS = 256
OUTLIER_GAIN = 20.0
N_OUTLIERS = 4

_KIND_K, _KIND_V, _KIND_Q = 1, 2, 3


def outlier_channels(cfg: int, layer: int, n_kv_heads: int = 4,
                     head_dim: int = HEAD_DIM, n_out: int = N_OUTLIERS):
    """Outlier channel indices, shape [2, n_kv_heads, n_out] (K first, then V)."""
    rng = np.random.default_rng(1000 * cfg + layer)
    k = np.stack([rng.choice(head_dim, n_out, replace=False) for _ in range(n_kv_heads)])
    v = np.stack([rng.choice(head_dim, n_out, replace=False) for _ in range(n_kv_heads)])
    return np.stack([k, v])


def _gain(cfg, layer, n_kv_heads, head_dim, outlier):
    ch = outlier_channels(cfg, layer, n_kv_heads, head_dim)
    g = np.ones((2, n_kv_heads, head_dim))
    if outlier != 1.0:
        for kind in range(2):
            for h in range(n_kv_heads):
                g[kind, h, ch[kind, h]] = outlier
    return g


def kv_tokens_np(cfg: int, layer: int, seq: int, start: int, n: int,
                 n_kv_heads: int = 4, head_dim: int = HEAD_DIM,
                 outlier: float = OUTLIER_GAIN):
    """K, V for logical tokens [start, start+n) of one sequence.

    Returns two float16 arrays of shape [n, n_kv_heads, head_dim]. Each
    256-token page has its own stream, so the result does not depend on how
    a range is chunked.
    """
    k = np.empty((n, n_kv_heads, head_dim), np.float16)
    v = np.empty((n, n_kv_heads, head_dim), np.float16)
    if n == 0:
        return k, v
    gain = _gain(cfg, layer, n_kv_heads, head_dim, outlier)
    first, last = start // PAGE_TOKENS, (start + n - 1) // PAGE_TOKENS
    for page in range(first, last + 1):
        p0 = page * PAGE_TOKENS
        lo, hi = max(start, p0), min(start + n, p0 + PAGE_TOKENS)
        for kind, dst in ((_KIND_K, k), (_KIND_V, v)):
            rng = np.random.default_rng([cfg, layer, seq, page, kind])
            z = rng.standard_normal((PAGE_TOKENS, n_kv_heads, head_dim))
            z *= gain[kind - 1][None]
            dst[lo - start:hi - start] = z[lo - p0:hi - p0].astype(np.float16)
    return k, v


def q_np(cfg: int, layer: int, batch: int, n_q_heads: int = 24,
         head_dim: int = HEAD_DIM, step: int = 0):
    """Decode queries, float16 [batch, n_q_heads, head_dim]."""
    rng = np.random.default_rng([cfg, layer, step, _KIND_Q])
    return rng.standard_normal((batch, n_q_heads, head_dim)).astype(np.float16)


def torch_seed(cfg: int, layer: int, seq: int = 0) -> int:
    return 1000 * cfg + 100 * seq + layer


def kv_tokens_torch(gen, n: int, gain, device):
    """Draw K, V (fp16 [n, Hkv, D]) on ``device`` from torch generator ``gen``.

    ``gain`` is a float32 tensor [2, Hkv, D] on ``device`` (see ``gain_torch``).
    """
    import torch
    hkv, d = gain.shape[1], gain.shape[2]
    k = torch.randn((n, hkv, d), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((n, hkv, d), generator=gen, device=device, dtype=torch.float32)
    return (k * gain[0]).to(torch.float16), (v * gain[1]).to(torch.float16)


def gain_torch(cfg: int, layer: int, n_kv_heads: int, device,
               head_dim: int = HEAD_DIM, outlier: float = OUTLIER_GAIN):
    import torch
    return torch.tensor(_gain(cfg, layer, n_kv_heads, head_dim, outlier),
                        dtype=torch.float32, device=device)


def q_torch(gen, batch: int, n_q_heads: int, device, head_dim: int = HEAD_DIM):
    import torch
    return torch.randn((batch, n_q_heads, head_dim), generator=gen, device=device,
                       dtype=torch.float32).to(torch.float16)


def selection_np(seed: int, n_pages: int, n_sel: int):
    """A seeded ordered selection of ``n_sel`` distinct logical pages."""
    rng = np.random.default_rng(seed)
    return rng.choice(n_pages, n_sel, replace=False).astype(np.int32)


def permutation_np(seed: int, n: int):
    """A seeded permutation of range(n) (shuffled physical page ids)."""
    return np.random.default_rng(seed).permutation(n).astype(np.int32)
