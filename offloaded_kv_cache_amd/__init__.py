"""MI355X-native quantized, paged, host-offloadable GQA decode attention.

The hot path lives in the HIP library ``lib/libkvcache.so`` (C ABI in
``include/kvcache.h``): quantize-on-append (int8, Walsh-Hadamard-rotated
q4_0, k8v4), split-K decode attention with the rotation back, and a
CLOCK-managed zero-copy page gather from pinned host memory. This package is
the thin Python binding over it; it raises ImportError if the library has
not been built (``python offloaded_kv_cache_amd/build.py``).
"""

from ._native import (  # noqa: F401
    FORMATS, KV_FMT_FP4, KV_FMT_FP8, KV_FMT_INT8, KV_FMT_K8V4, KV_FMT_Q4_0, KV_STATUS_BAD_PAGE_ID,
    KV_STATUS_CONTEXT_CLAMPED, KVError, KVShape, Residency, append_decode, append_quantize,
    decode_attention, decode_attention_mq, decode_attention_noalloc, decode_mq_workspace_bytes, decode_split_pages, decode_workspace_bytes, gather_pages, gather_pages_layers,
    host_encode_vector,
    host_f64_to_f16, last_error, page_bytes, page_key_sums, select_pages, select_workspace_bytes, shape,
    version,
)
from . import paged, streaming  # noqa: F401
