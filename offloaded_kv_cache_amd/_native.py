"""ctypes binding of ``lib/libkvcache.so`` (the C ABI in ``include/kvcache.h``).

Argument marshalling only: every step of the hot path runs in the HIP
library. PyTorch supplies device memory, pinned host memory and the stream.
If the library is missing, importing this module raises: there is no CPU
fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkvcache.so")

KV_OK, KV_EINVAL, KV_EUNSUPPORTED, KV_EALIGN, KV_ENOSLOTS, KV_EHIP, KV_ESMALL = 0, -1, -2, -3, -4, -5, -6
KV_STATUS_BAD_PAGE_ID, KV_STATUS_CONTEXT_CLAMPED = 1, 2
KV_FMT_INT8, KV_FMT_Q4_0, KV_FMT_K8V4, KV_FMT_FP4, KV_FMT_FP8 = 0, 1, 2, 3, 4
FORMATS = {"int8": KV_FMT_INT8, "q4_0": KV_FMT_Q4_0, "k8v4": KV_FMT_K8V4, "fp4": KV_FMT_FP4,
           "fp8": KV_FMT_FP8}

EXPORTED_SYMBOLS = (
    "kv_last_error", "kv_version", "kv_page_bytes", "kv_append_quantize", "kv_append_quantize_timed",
    "kv_decode_workspace_bytes", "kv_decode_split_pages", "kv_decode_attention", "kv_decode_split",
    "kv_decode_split_timed", "kv_decode_attention_noalloc",
    "kv_decode_combine", "kv_decode_attention_mq", "kv_decode_mq_workspace_bytes", "kv_append_decode", "kv_gather_pages_layers",
    "kv_gather_pages_layers_timed", "kv_page_key_sums",
    "kv_select_workspace_bytes", "kv_select_pages",
    "kv_residency_reset",
    "kv_residency_select", "kv_gather_pages", "kv_host_f64_to_f16", "kv_host_encode_vector",
)


class KVShape(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_tokens", C.c_int32), ("format", C.c_int32)]


class KVResidency(C.Structure):
    _fields_ = [("n_slots", C.c_int32), ("n_pages", C.c_int32),
                ("slot_page", C.POINTER(C.c_int32)), ("page_slot", C.POINTER(C.c_int32)),
                ("ref", C.POINTER(C.c_uint8)), ("hand", C.c_int32)]


class KVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvcache error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(run `python offloaded_kv_cache_amd/build.py`)")
    # torch first: its wheel bundles a HIP runtime under the same soname as the one the
    # library links. Loaded first, the library would pull in a second runtime, and its
    # launches would not see the device torch's runtime holds.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    sig = {
        "kv_last_error": (C.c_char_p, []),
        "kv_version": (C.c_char_p, []),
        "kv_page_bytes": (I64, [C.POINTER(KVShape)]),
        "kv_append_quantize": (C.c_int, [C.POINTER(KVShape), P, P, I64, I64, P, I32, P, I64, P, P]),
        "kv_append_quantize_timed": (C.c_int, [C.POINTER(KVShape), P, P, I64, I64, P, I32, P, I64, P, P, P, P]),
        "kv_decode_workspace_bytes": (SZ, [C.POINTER(KVShape), I32, I64, I32]),
        "kv_decode_split_pages": (I32, [C.POINTER(KVShape), I32, I64, I64]),
        "kv_decode_attention": (C.c_int, [C.POINTER(KVShape), P, I32, P, I64, P, I32, P, I64, F32,
                                          P, P, SZ, I32, P]),
        "kv_decode_split": (C.c_int, [C.POINTER(KVShape), P, I32, P, I64, P, I32, P, I64, F32,
                                      P, P, SZ, I32, P]),
        "kv_decode_combine": (C.c_int, [C.POINTER(KVShape), P, I32, P, I64, P, I32, P, I64, F32,
                                        P, P, SZ, I32, P]),
        "kv_decode_split_timed": (C.c_int, [C.POINTER(KVShape), P, I32, P, I64, P, I32, P, I64, F32,
                                            P, P, SZ, I32, P, P, P]),
        "kv_decode_attention_noalloc": (C.c_int, [C.POINTER(KVShape), P, I32, P, I64, P, I32, P, I64, F32,
                                                  P, P, I32, P]),
        "kv_decode_mq_workspace_bytes": (SZ, [C.POINTER(KVShape), I32, I32, I64, I32]),
        "kv_decode_attention_mq": (C.c_int, [C.POINTER(KVShape), P, I32, I32, P, I64, P, I32, P, I64,
                                             F32, P, P, SZ, I32, P]),
        "kv_append_decode": (C.c_int, [C.POINTER(KVShape), P, P, P, I32, P, I64, P, I32, P, I64,
                                       F32, P, P, SZ, I32, P, P, P]),
        "kv_residency_reset": (C.c_int, [C.POINTER(KVResidency)]),
        "kv_residency_select": (C.c_int, [C.POINTER(KVResidency), P, I32, P, P, P, P]),
        "kv_gather_pages": (C.c_int, [C.POINTER(KVShape), C.POINTER(KVResidency), P, I32, P, P, P,
                                      P, P]),
        "kv_gather_pages_layers": (C.c_int, [C.POINTER(KVShape), I32, C.POINTER(KVResidency), P, I32,
                                             P, P, P, P, P]),
        "kv_gather_pages_layers_timed": (C.c_int, [C.POINTER(KVShape), I32, C.POINTER(KVResidency), P, I32,
                                                   P, P, P, P, P, P, P]),
        "kv_page_key_sums": (C.c_int, [C.POINTER(KVShape), P, I64, I64, P, P, I64, P]),
        "kv_select_workspace_bytes": (SZ, [I64, I32]),
        "kv_select_pages": (C.c_int, [C.POINTER(KVShape), P, P, I64, I64, I32, I32, P, P, SZ, P]),
        "kv_host_f64_to_f16": (C.c_uint16, [C.c_double]),
        "kv_host_encode_vector": (C.c_int, [I32, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.kv_last_error().decode()


def version() -> str:
    return lib.kv_version().decode()


def _check(code: int):
    if code != KV_OK:
        raise KVError(code, last_error())


def shape(fmt, n_q_heads: int = 24, n_kv_heads: int = 4, head_dim: int = 256,
          page_tokens: int = 256) -> KVShape:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return KVShape(n_q_heads, n_kv_heads, head_dim, page_tokens, f)


def page_bytes(s: KVShape) -> int:
    r = lib.kv_page_bytes(C.byref(s))
    if r < 0:
        raise KVError(int(r), last_error())
    return int(r)


# ------------------------------------------------------------------ torch glue

def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, device=True, name="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    return C.c_void_p(t.data_ptr())


def _buf(t, name, pinned_ok=False):
    """Address of a byte buffer (pool, workspace, slots): a contiguous uint8 tensor in
    device memory (or, where the C ABI accepts it, pinned host memory). Anything else is
    refused here, before a kernel could be handed a host address."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be torch.uint8, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not (t.is_cuda or (pinned_ok and t.is_pinned())):
        raise ValueError(f"{name} must be in device memory" + (" or pinned host memory" if pinned_ok else ""))
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _event_ptrs(events):
    if events is None:
        return ()
    ev = []
    for e in events:
        if not e.cuda_event:
            e.record()  # creates the underlying event
        ev.append(C.c_void_p(e.cuda_event))
    return tuple(ev)


def append_quantize(s: KVShape, k, v, start_pos: int, block_table, pool, status=None, stream=None,
                    events=None):
    """Quantize-on-append of tokens [start_pos, start_pos + k.shape[0]) of one sequence.
    ``events`` = (start, stop) torch.cuda.Event pair: recorded at the append kernel's own
    start and end (kv_append_quantize_timed)."""
    torch = _torch()
    n = k.shape[0]
    if k.shape != v.shape or k.dim() != 3 or k.shape[1] != s.n_kv_heads or k.shape[2] != s.head_dim:
        raise ValueError("k and v must be [n_tokens, n_kv_heads, head_dim]")
    pb = page_bytes(s)
    if pool.numel() % pb:
        raise ValueError("pool size is not a whole number of pages")
    fn, ev = lib.kv_append_quantize, _event_ptrs(events)
    if ev:
        fn = lib.kv_append_quantize_timed
    _check(fn(
        C.byref(s), _ptr(k, torch.float16, name="k"), _ptr(v, torch.float16, name="v"),
        n, start_pos, _ptr(block_table, torch.int32, name="block_table"), block_table.numel(),
        _buf(pool, "pool", pinned_ok=True), pool.numel() // pb,
        _ptr(status, torch.int32, name="status"), _stream(stream), *ev))


def decode_workspace_bytes(s: KVShape, batch: int, max_context: int, pages_per_split: int = 0) -> int:
    r = lib.kv_decode_workspace_bytes(C.byref(s), batch, max_context, pages_per_split)
    if r == 0:
        raise KVError(KV_EINVAL, last_error())
    return int(r)


def decode_mq_workspace_bytes(s: KVShape, batch: int, n_q: int, max_context: int,
                              pages_per_split: int = 0) -> int:
    r = lib.kv_decode_mq_workspace_bytes(C.byref(s), batch, n_q, max_context, pages_per_split)
    if r == 0:
        raise KVError(KV_EINVAL, last_error())
    return int(r)


def decode_split_pages(s: KVShape, batch: int, max_context: int, total_context: int = 0) -> int:
    """Pages per split the library selects (for a batch whose lengths add up to total_context)."""
    r = lib.kv_decode_split_pages(C.byref(s), batch, max_context, total_context)
    if r <= 0:
        raise KVError(KV_EINVAL, last_error())
    return int(r)


_PHASES = {"all": "kv_decode_attention", "split": "kv_decode_split", "combine": "kv_decode_combine"}


def decode_attention(s: KVShape, q, pool, block_tables, context_lens, max_context: int, out,
                     workspace, softmax_scale: float = 1.0 / 16.0, pages_per_split: int = 0,
                     stream=None, phase: str = "all", events=None):
    """GQA decode attention over the paged cache; writes fp32 ``out`` [B, Hq, 256].

    ``phase`` = "split" or "combine" enqueues only that kernel (see kvcache.h).
    ``events`` = (start, stop) torch.cuda.Event pair, with phase "split" only:
    recorded at the split kernel's own start and end (kv_decode_split_timed)."""
    torch = _torch()
    fn = getattr(lib, _PHASES[phase])
    extra = ()
    if events is not None:
        if phase != "split":
            raise ValueError("events are recorded around the split kernel only (phase='split')")
        ev = []
        for e in events:
            if not e.cuda_event:
                e.record()  # creates the underlying event
            ev.append(C.c_void_p(e.cuda_event))
        fn = lib.kv_decode_split_timed
        extra = tuple(ev)
    B = q.shape[0]
    if q.shape != (B, s.n_q_heads, s.head_dim) or out.shape != (B, s.n_q_heads, s.head_dim):
        raise ValueError("q and out must be [batch, n_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [batch, max_pages] and context_lens [batch]")
    pb = page_bytes(s)
    _check(fn(
        C.byref(s), _ptr(q, torch.float16, name="q"), B, _buf(pool, "pool"),
        pool.numel() // pb, _ptr(block_tables, torch.int32, name="block_tables"),
        block_tables.shape[1], _ptr(context_lens, torch.int32, name="context_lens"), max_context,
        softmax_scale, _ptr(out, torch.float32, name="out"), _buf(workspace, "workspace"),
        workspace.numel(), pages_per_split, _stream(stream), *extra))


NOALLOC_SCRATCH_BYTES = 16777216  # KV_NOALLOC_SCRATCH_BYTES


def decode_attention_noalloc(s: KVShape, q, pool, block_tables, context_lens, max_context: int, out,
                             status=None, softmax_scale: float = 1.0 / 16.0, pages_per_split: int = 0,
                             stream=None):
    """kv_decode_attention_noalloc: decode_attention without a workspace (the library's own
    device array holds the partials). ``status``: device int32 [1] or None."""
    torch = _torch()
    B = q.shape[0]
    if q.shape != (B, s.n_q_heads, s.head_dim) or out.shape != (B, s.n_q_heads, s.head_dim):
        raise ValueError("q and out must be [batch, n_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [batch, max_pages] and context_lens [batch]")
    pb = page_bytes(s)
    _check(lib.kv_decode_attention_noalloc(
        C.byref(s), _ptr(q, torch.float16, name="q"), B, _buf(pool, "pool"),
        pool.numel() // pb, _ptr(block_tables, torch.int32, name="block_tables"),
        block_tables.shape[1], _ptr(context_lens, torch.int32, name="context_lens"), max_context,
        softmax_scale, _ptr(out, torch.float32, name="out"), _ptr(status, torch.int32, name="status"),
        pages_per_split, _stream(stream)))


def decode_attention_mq(s: KVShape, q, pool, block_tables, context_lens, max_context: int, out,
                        workspace, softmax_scale: float = 1.0 / 16.0, pages_per_split: int = 0,
                        stream=None):
    """Causal attention of each sequence's n_q newest tokens (kv_decode_attention_mq):
    ``q`` fp16 [B, n_q, Hq, 256], query j of sequence b at position context_lens[b] - n_q + j;
    writes fp32 ``out`` [B, n_q, Hq, 256]. Workspace: decode_mq_workspace_bytes(s, B, n_q, ...)."""
    torch = _torch()
    if q.dim() != 4 or q.shape[2:] != (s.n_q_heads, s.head_dim) or out.shape != q.shape:
        raise ValueError("q and out must be [batch, n_q, n_q_heads, head_dim]")
    B, n_q = q.shape[0], q.shape[1]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [batch, max_pages] and context_lens [batch]")
    pb = page_bytes(s)
    _check(lib.kv_decode_attention_mq(
        C.byref(s), _ptr(q, torch.float16, name="q"), B, n_q, _buf(pool, "pool"),
        pool.numel() // pb, _ptr(block_tables, torch.int32, name="block_tables"),
        block_tables.shape[1], _ptr(context_lens, torch.int32, name="context_lens"), max_context,
        softmax_scale, _ptr(out, torch.float32, name="out"), _buf(workspace, "workspace"),
        workspace.numel(), pages_per_split, _stream(stream)))


def append_decode(s: KVShape, k_new, v_new, q, pool, block_tables, context_lens, max_context: int,
                  out, workspace, softmax_scale: float = 1.0 / 16.0, pages_per_split: int = 0,
                  stream=None, events=None):
    """One decode step of one layer (kv_append_decode): append token context_lens[b] - 1
    of every sequence (``k_new``, ``v_new`` fp16 [B, n_kv_heads, 256]) into ``pool``,
    then attend; writes fp32 ``out`` [B, Hq, 256]. ``events`` = (start, stop)
    torch.cuda.Event pair recorded at the split kernel's own start and end."""
    torch = _torch()
    B = q.shape[0]
    if q.shape != (B, s.n_q_heads, s.head_dim) or out.shape != (B, s.n_q_heads, s.head_dim):
        raise ValueError("q and out must be [batch, n_q_heads, head_dim]")
    if k_new.shape != (B, s.n_kv_heads, s.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [batch, n_kv_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [batch, max_pages] and context_lens [batch]")
    ev = [None, None]
    if events is not None:
        for i, e in enumerate(events):
            if not e.cuda_event:
                e.record()  # creates the underlying event
            ev[i] = e.cuda_event
    pb = page_bytes(s)
    _check(lib.kv_append_decode(
        C.byref(s), _ptr(k_new, torch.float16, name="k_new"), _ptr(v_new, torch.float16, name="v_new"),
        _ptr(q, torch.float16, name="q"), B, _buf(pool, "pool"), pool.numel() // pb,
        _ptr(block_tables, torch.int32, name="block_tables"), block_tables.shape[1],
        _ptr(context_lens, torch.int32, name="context_lens"), max_context, softmax_scale,
        _ptr(out, torch.float32, name="out"), _buf(workspace, "workspace"),
        workspace.numel(), pages_per_split, _stream(stream),
        C.c_void_p(ev[0]), C.c_void_p(ev[1])))


class Residency:
    """Host arrays of one layer's CLOCK residency table (kv_residency)."""

    def __init__(self, n_slots: int, n_pages: int):
        self.slot_page = np.full(n_slots, -1, np.int32)
        self.page_slot = np.full(max(n_pages, 1), -1, np.int32)
        self.ref = np.zeros(n_slots, np.uint8)
        self.c = KVResidency(n_slots, n_pages,
                             self.slot_page.ctypes.data_as(C.POINTER(C.c_int32)),
                             self.page_slot.ctypes.data_as(C.POINTER(C.c_int32)),
                             self.ref.ctypes.data_as(C.POINTER(C.c_uint8)), 0)
        _check(lib.kv_residency_reset(C.byref(self.c)))

    @property
    def hand(self) -> int:
        return self.c.hand

    def select(self, selection):
        sel = np.ascontiguousarray(selection, dtype=np.int32)
        n = sel.size
        slots = np.empty(max(n, 1), np.int32)
        mp = np.empty(max(n, 1), np.int32)
        ms = np.empty(max(n, 1), np.int32)
        nm = C.c_int32(0)
        _check(lib.kv_residency_select(C.byref(self.c), sel.ctypes.data_as(C.c_void_p), n,
                                       slots.ctypes.data_as(C.c_void_p), mp.ctypes.data_as(C.c_void_p),
                                       ms.ctypes.data_as(C.c_void_p), C.byref(nm)))
        k = nm.value
        return slots[:n].copy(), list(zip(mp[:k].tolist(), ms[:k].tolist()))


def gather_pages(s: KVShape, table: Residency, selection, host_pool, slot_pool, out_block_table,
                 stream=None) -> int:
    """CLOCK step + zero-copy page-in; returns the number of pages copied."""
    torch = _torch()
    sel = np.ascontiguousarray(selection, dtype=np.int32)
    if not host_pool.is_pinned():
        raise ValueError("host_pool must be pinned host memory")
    nm = C.c_int32(0)
    _check(lib.kv_gather_pages(C.byref(s), C.byref(table.c), sel.ctypes.data_as(C.c_void_p), sel.size,
                               _buf(host_pool, "host_pool", pinned_ok=True), _buf(slot_pool, "slot_pool"),
                               _ptr(out_block_table, torch.int32, name="out_block_table"),
                               C.byref(nm), _stream(stream)))
    return nm.value


def gather_pages_layers(s: KVShape, tables, selections, host_pools, slot_pools, out_block_tables,
                        stream=None, events=None):
    """kv_gather_pages_layers: CLOCK step of every layer, then one page-in launch for all
    of them. selections int32 [L, n_sel]; out_block_tables device int32 [L, n_sel].
    Returns the misses per layer (numpy int32 [L]). ``events`` = (start, stop)
    torch.cuda.Event pair: recorded at the copy kernel's own start and end
    (kv_gather_pages_layers_timed)."""
    torch = _torch()
    sel = np.ascontiguousarray(selections, dtype=np.int32)
    L = len(tables)
    if sel.ndim != 2 or sel.shape[0] != L or len(host_pools) != L or len(slot_pools) != L:
        raise ValueError("one selection row, host pool and slot pool per table")
    if out_block_tables.shape != sel.shape:
        raise ValueError("out_block_tables must be [n_layers, n_sel]")
    for h in host_pools:
        if not h.is_pinned():
            raise ValueError("host pools must be pinned host memory")
    arr = (KVResidency * L)(*[t.c for t in tables])
    hp = (C.c_void_p * L)(*[_buf(h, "host pool", pinned_ok=True).value for h in host_pools])
    sp = (C.c_void_p * L)(*[_buf(p, "slot pool").value for p in slot_pools])
    nm = np.zeros(L, np.int32)
    fn, ev = lib.kv_gather_pages_layers, _event_ptrs(events)
    if ev:
        fn = lib.kv_gather_pages_layers_timed
    _check(fn(C.byref(s), L, arr, sel.ctypes.data_as(C.c_void_p), sel.shape[1],
              C.cast(hp, C.c_void_p), C.cast(sp, C.c_void_p),
              _ptr(out_block_tables, torch.int32, name="out_block_tables"),
              nm.ctypes.data_as(C.c_void_p), _stream(stream), *ev))
    for t, a in zip(tables, arr):  # the tables' arrays are shared; the hand is copied back
        t.c.hand = a.hand
    return nm


def page_key_sums(s: KVShape, k, start_pos: int, sums, reps, stream=None):
    """kv_page_key_sums: add keys k (fp16 [n, n_kv_heads, 256]) of tokens start_pos.. to
    sums (device int64 [n_pages_cap, n_kv_heads, 256]) and round the touched pages'
    representatives into reps (device fp16, same shape)."""
    torch = _torch()
    if k.dim() != 3 or k.shape[1:] != (s.n_kv_heads, s.head_dim):
        raise ValueError("k must be [n_tokens, n_kv_heads, head_dim]")
    if sums.dim() != 3 or sums.shape[1:] != (s.n_kv_heads, s.head_dim):
        raise ValueError("sums must be [n_pages_cap, n_kv_heads, head_dim]")
    if reps.shape != sums.shape:
        raise ValueError("reps must have the shape of sums")
    _check(lib.kv_page_key_sums(C.byref(s), _ptr(k, torch.float16, name="k"), k.shape[0], start_pos,
                                _ptr(sums, torch.int64, name="sums"), _ptr(reps, torch.float16, name="reps"),
                                sums.shape[0], _stream(stream)))


def select_workspace_bytes(n_pages: int, n_sets: int = 1) -> int:
    nb = lib.kv_select_workspace_bytes(n_pages, n_sets)
    if nb == 0:
        raise KVError(-1, last_error())
    return nb


def select_pages(s: KVShape, q, reps, n_pages: int, k_sel: int, out_selection, workspace, stream=None):
    """kv_select_pages over the leading dimension of q ([n_sets, Hq, 256], or [Hq, 256] for
    one set), reps (fp16 [n_sets, reps_pages, Hkv, 256] or [reps_pages, Hkv, 256]) and
    out_selection ([n_sets, k_sel] or [k_sel]); each set's pages in ascending order."""
    torch = _torch()
    one = q.dim() == 2
    n_sets = 1 if one else q.shape[0]
    if q.shape[-2:] != (s.n_q_heads, s.head_dim) or reps.dim() != (3 if one else 4):
        raise ValueError("q must be [n_sets, n_q_heads, head_dim] and reps [n_sets, pages, n_kv_heads, head_dim]")
    if not one and (reps.shape[0] != n_sets or out_selection.dim() != 2 or out_selection.shape[0] != n_sets):
        raise ValueError("one reps block and one selection row per set")
    if out_selection.shape[-1] != k_sel:
        raise ValueError("out_selection rows must hold k_sel entries")
    _check(lib.kv_select_pages(C.byref(s), _ptr(q, torch.float16, name="q"), _ptr(reps, torch.float16, name="reps"),
                               reps.shape[-3], n_pages, k_sel, n_sets,
                               _ptr(out_selection, torch.int32, name="out_selection"),
                               _buf(workspace, "workspace"), workspace.numel(),
                               _stream(stream)))


def host_f64_to_f16(x: float) -> int:
    return int(lib.kv_host_f64_to_f16(float(x)))


def host_encode_vector(kind: int, x: np.ndarray):
    """Record of one fp16 vector by the library's host rules: (codes uint8[256], scales fp16)."""
    xb = np.ascontiguousarray(np.asarray(x, np.float16)).view(np.uint16)
    codes = np.zeros(256, np.uint8)
    scales = np.zeros(8, np.uint16)
    _check(lib.kv_host_encode_vector(kind, xb.ctypes.data_as(C.c_void_p),
                                     codes.ctypes.data_as(C.c_void_p), scales.ctypes.data_as(C.c_void_p)))
    n = {0: 4, 3: 1}.get(kind, 8)
    return codes, scales[:n].view(np.float16)
