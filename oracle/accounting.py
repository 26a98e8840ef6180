"""Byte accounting of the KV formats and the KV-size formula (oracle).

* Strata page, section "三种 KV 格式横向对比": per token per layer, for the K
  and V of two KV heads, int8 takes 1,056 B, q4_0 576 B, k8v4 23% less than
  int8 (816 B).
* VRAM wiki page, section "一、为什么 256K 上下文的显存这么吓人": KV bytes =
  2 x full-attention layers x KV heads x head_dim x bytes per element x
  context length; section "二、核心组合表": at 256K with 16 layers, 4 KV heads
  and head_dim 256, FP16 ~17.2 GB, Q8_0 ~9.1 GB, Q4_0 ~4.8 GB.
* KV-offload news page, section "缓存为何不能直接搬走？": 2,048 B per token per
  layer, ~512 MiB per layer at 262,144 tokens, ~6 GiB for 12 layers, ~5
  tokens/s if all of it crosses a ~32 GiB/s PCIe 4.0 x16 link each token.
"""

from __future__ import annotations

from .layout import PAGE_TOKENS, page_bytes
from .records import KIND_INT8, kinds, record_bytes


def bytes_per_token_layer(fmt: int, n_kv_heads: int) -> int:
    """K + V record bytes of one token in one layer."""
    kk, vk = kinds(fmt)
    return n_kv_heads * (record_bytes(kk) + record_bytes(vk))


def bytes_per_token_layer_from_pages(fmt: int, n_kv_heads: int) -> int:
    return page_bytes(fmt, n_kv_heads) // PAGE_TOKENS


def kv_cache_bytes(layers: int, n_kv_heads: int, head_dim: int,
                   bytes_per_elem: float, context: int) -> float:
    """The VRAM wiki page's formula: 2 x layers x KV heads x head_dim x bytes x context."""
    return 2 * layers * n_kv_heads * head_dim * bytes_per_elem * context


GGML_BITS_PER_ELEM = {"f16": 16.0, "q8_0": 8.5, "q4_0": 4.5}


def pcie_tokens_per_second(bytes_per_token: float, link_bytes_per_s: float) -> float:
    """Decode rate if every token re-reads ``bytes_per_token`` over a link."""
    return link_bytes_per_s / bytes_per_token


def is_int8(kind: str) -> bool:
    return kind == KIND_INT8
