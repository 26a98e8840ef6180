"""Streaming-mode decode over several layers: schedules of the page-in.

Strata page ("KV 沉进内存、显存减半：Strata 让 12 GB 显卡跑满 262K 上下文"),
section "KV 从显存搬进内存之后发生了什么": the authoritative KV copy stays in
pinned host memory, and before each attention the selected pages are looked up
in the residency table and the missing ones are copied over PCIe into device
slots. Every layer has its own table and slots, so the page-in of one layer
does not depend on the attention of another. Three schedules:

* "layers" (batched): one kv_gather_pages_layers call pages in every layer's
  selection with one launch, then the layers attend;
* "serial": per layer, kv_gather_pages then attention, on one stream;
* "overlap": each layer's gather on a copy stream while earlier layers attend on
  the compute stream. Ordering by events: attention of layer l waits for the
  gather of layer l; the next gather into layer l's slots waits for layer l's
  previous attention (CLOCK may reuse a slot that attention is still reading).

This module only schedules calls of the C ABI (kv_gather_pages_layers,
kv_gather_pages, kv_decode_attention) on streams; all work runs in the
library's kernels.
"""

from __future__ import annotations

from . import _native as N


class StreamedLayers:
    """Per-layer residency tables, device slots and slot block tables for L layers."""

    def __init__(self, s: N.KVShape, n_layers: int, n_slots: int, n_pages: int, n_sel: int,
                 device, overlap: bool = False):
        torch = N._torch()
        self.s, self.n_sel, self.overlap = s, n_sel, overlap
        pb = N.page_bytes(s)
        self.tables = [N.Residency(n_slots, n_pages) for _ in range(n_layers)]
        self.slots = [torch.zeros(n_slots * pb, dtype=torch.uint8, device=device) for _ in range(n_layers)]
        self.block_table_all = torch.empty((n_layers, n_sel), dtype=torch.int32, device=device)
        self.block_tables = [self.block_table_all[layer] for layer in range(n_layers)]
        self.copy_stream = torch.cuda.Stream(device=device) if overlap else None  # default priority
        self.gathered = [torch.cuda.Event() for _ in range(n_layers)]
        self.attended = [torch.cuda.Event() for _ in range(n_layers)]
        cur = torch.cuda.current_stream(device)
        for e in self.gathered + self.attended:
            e.record(cur)  # every event starts out complete

    def gather_layers(self, selections, host_pools, stream, events=None):
        """Page in every layer's selection ([n_layers, n_sel]) with one launch on `stream`;
        returns the misses per layer. `events` = (start, stop): recorded at the copy
        kernel's own start and end."""
        return N.gather_pages_layers(self.s, self.tables, selections, host_pools, self.slots,
                                     self.block_table_all, stream=stream, events=events)

    def gather(self, layer: int, selection, host_pool, stream) -> int:
        """Page in layer `layer`'s selection (CLOCK on the host, copy kernel on the GPU);
        returns the number of misses. `stream` is the compute stream."""
        if not self.overlap:
            return N.gather_pages(self.s, self.tables[layer], selection, host_pool, self.slots[layer],
                                  self.block_tables[layer], stream=stream)
        cs = self.copy_stream
        cs.wait_event(self.attended[layer])
        m = N.gather_pages(self.s, self.tables[layer], selection, host_pool, self.slots[layer],
                           self.block_tables[layer], stream=cs)
        self.gathered[layer].record(cs)
        return m

    def attend(self, layer: int, q, context_lens, max_context: int, out, workspace, stream, **kw):
        """Decode attention of layer `layer` over its gathered slots, on `stream`."""
        if self.overlap:
            stream.wait_event(self.gathered[layer])
        N.decode_attention(self.s, q, self.slots[layer], self.block_tables[layer][None], context_lens,
                           max_context, out, workspace, stream=stream, **kw)
        if self.overlap:
            self.attended[layer].record(stream)
