"""Small owner objects for a layer's paged pool and a decode workspace.

Memory is allocated through PyTorch (device memory, pinned host memory); all
computation goes through the HIP library.
"""

from __future__ import annotations

from . import _native as N


class PagedPool:
    """A pool of ``n_pages`` pages of one layer, on the device or in pinned host memory."""

    def __init__(self, fmt, n_pages: int, n_q_heads: int = 24, n_kv_heads: int = 4,
                 device="cuda", pinned_host: bool = False):
        import torch
        self.shape = N.shape(fmt, n_q_heads, n_kv_heads)
        self.page_bytes = N.page_bytes(self.shape)
        self.n_pages = n_pages
        nbytes = n_pages * self.page_bytes
        if pinned_host:
            self.data = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        else:
            self.data = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def page(self, i: int):
        return self.data[i * self.page_bytes:(i + 1) * self.page_bytes]

    def append(self, k, v, start_pos: int, block_table, status=None, stream=None, events=None):
        N.append_quantize(self.shape, k, v, start_pos, block_table, self.data, status, stream, events)


class DecodeWorkspace:
    """A zero-filled decode workspace sized for (batch, max_context, pages_per_split); with
    n_q > 1, for kv_decode_attention_mq with n_q queries per sequence."""

    def __init__(self, shape, batch: int, max_context: int, pages_per_split: int = 0, device="cuda",
                 n_q: int = 1):
        import torch
        self.nbytes = (N.decode_workspace_bytes(shape, batch, max_context, pages_per_split) if n_q == 1
                       else N.decode_mq_workspace_bytes(shape, batch, n_q, max_context, pages_per_split))
        self.data = torch.zeros(self.nbytes, dtype=torch.uint8, device=device)
        self.pages_per_split = pages_per_split

    def status(self) -> int:
        return int(self.data[:4].view(__import__("torch").int32).item())

    def clear_status(self):
        self.data[:4].zero_()
