"""GPU tests of the CLOCK-managed zero-copy page gather (through the C ABI).

Streaming must not change results: attention over pages gathered into slots
equals, bit for bit, attention over the same pages read from a fully
resident pool, whatever the miss rate and the slots chosen.
"""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K
from oracle.residency import ClockTable

from gpu_helpers import Sequence, assert_close, oracle_out, place_pages

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("fmt", ["int8", "k8v4", "fp4", "fp8"])
@pytest.mark.parametrize("miss_rate", [0.0, 0.3, 1.0])
def test_gather_then_attend_equals_resident(gpu, fmt, miss_rate):
    n_pages, n_slots, n_sel, steps = 40, 12, 8, 6
    T = n_pages * 256
    seq = Sequence(31, 0, 0, T, fmt)
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    # authoritative copy: pinned host memory, logical page p at p * page_bytes
    host = torch.from_numpy(seq.pages.reshape(-1).copy()).pin_memory()
    # fully resident reference pool (device), same pages at shuffled places
    res_np, res_bt = place_pages([seq], n_pages + 2, 7, pb)
    resident = to_dev(res_np, gpu)
    slots = torch.zeros(n_slots * pb, dtype=torch.uint8, device=gpu)
    table = K.Residency(n_slots, n_pages)
    shadow = ClockTable(n_slots, n_pages)
    rng = np.random.default_rng(int(miss_rate * 10))
    bt_dev = torch.empty(n_sel, dtype=torch.int32, device=gpu)
    ws = K.paged.DecodeWorkspace(s, 1, n_sel * 256, 2, device=gpu)
    out_a = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    out_b = torch.empty_like(out_a)
    lens = to_dev(np.array([n_sel * 256], np.int32), gpu)
    total_miss = 0
    for step in range(steps + 1):
        resident_now = [p for p in shadow.slot_page if p >= 0]
        if step == 0 or not resident_now:
            sel = rng.choice(n_pages, n_sel, replace=False)
        else:
            pick = []
            pool_res = list(rng.permutation(resident_now))
            pool_non = list(rng.permutation([p for p in range(n_pages) if p not in resident_now]))
            for _ in range(n_sel):
                want_miss = rng.random() < miss_rate
                src = pool_non if (want_miss and pool_non) or not pool_res else pool_res
                pick.append(src.pop())
            sel = np.array(pick)
        n_miss = K.gather_pages(s, table, sel, host, slots, bt_dev)
        _, copies = shadow.select(sel)
        assert n_miss == len(copies)
        if step > 0:
            total_miss += n_miss
        q = kvsynth.q_np(31, 0, 1, step=step)
        qd = to_dev(q, gpu)
        K.decode_attention(s, qd, slots, bt_dev[None].contiguous(), lens, n_sel * 256, out_a, ws.data,
                           pages_per_split=2)
        ref_bt = to_dev(res_bt[0, sel][None], gpu)
        K.decode_attention(s, qd, resident, ref_bt, lens, n_sel * 256, out_b, ws.data,
                           pages_per_split=2)
        torch.cuda.synchronize()
        assert np.array_equal(out_a.cpu().numpy(), out_b.cpu().numpy()), f"step {step}"
        # the slots hold the selected host pages byte for byte
        got_slots = slots.cpu().numpy().reshape(n_slots, pb)
        for i, p in enumerate(sel):
            assert np.array_equal(got_slots[bt_dev[i].item()], seq.pages[p])
        # and the result matches the oracle over the selected tokens
        if step == steps:
            kk = np.concatenate([seq.k[p * 256:(p + 1) * 256] for p in sel])
            vv = np.concatenate([seq.v[p * 256:(p + 1) * 256] for p in sel])
            ref = Sequence(31, 0, 0, n_sel * 256, fmt, k=kk, v=vv)
            assert_close(out_a.cpu().numpy(), oracle_out(q, [ref], fmt))
    if miss_rate == 0.0:
        assert total_miss == 0
    if miss_rate == 1.0:
        assert total_miss == steps * n_sel


def test_gather_refuses_unpinned_host_memory(gpu):
    s = K.shape("int8")
    table = K.Residency(4, 8)
    host = torch.zeros(8 * K.page_bytes(s), dtype=torch.uint8)
    slots = torch.zeros(4 * K.page_bytes(s), dtype=torch.uint8, device=gpu)
    bt = torch.empty(2, dtype=torch.int32, device=gpu)
    with pytest.raises(ValueError):
        K.gather_pages(s, table, [0, 1], host, slots, bt)


def draw_selections(L, n_pages, n_slots, n_sel, steps, seed):
    """One selection per (step, layer) with a mix of hits and misses, drawn from shadow
    CLOCK tables that make the same decisions as the library's."""
    rng = np.random.default_rng(seed)
    shadows = [ClockTable(n_slots, n_pages) for _ in range(L)]
    sels = []
    for st in range(steps):
        row = []
        for layer in range(L):
            res = [p for p in shadows[layer].slot_page if p >= 0]
            if res and st > 0:
                k = min(len(res), n_sel - 3)
                pick = list(rng.choice(res, k, replace=False))
                non = [p for p in range(n_pages) if p not in res]
                pick += list(rng.choice(non, n_sel - k, replace=False))
            else:
                pick = list(rng.choice(n_pages, n_sel, replace=False))
            sel = np.array(pick, np.int32)
            shadows[layer].select(sel)
            row.append(sel)
        sels.append(row)
    return sels


@pytest.mark.parametrize("fmt", ["int8", "k8v4", "fp8"])
def test_gather_layers_equals_per_layer_gathers(gpu, fmt):
    """kv_gather_pages_layers (one launch for every layer) leaves the same tables, slots
    and block tables as kv_gather_pages per layer, and attention over them is identical;
    so does kv_gather_pages_layers_timed, whose events span the copy kernel."""
    L, n_pages, n_slots, n_sel, steps = 4, 30, 10, 8, 4
    s = K.shape(fmt)
    seqs = [Sequence(35, layer, 0, n_pages * 256, fmt) for layer in range(L)]
    host = [torch.from_numpy(sq.pages.reshape(-1).copy()).pin_memory() for sq in seqs]
    sels = draw_selections(L, n_pages, n_slots, n_sel, steps, 6)
    q = to_dev(kvsynth.q_np(35, 0, steps * L).reshape(steps, L, 1, 24, 256), gpu)
    ctx = to_dev(np.array([n_sel * 256], np.int32), gpu)
    runs = []
    for mode in ("per_layer", "layers", "layers_timed"):
        sl = K.streaming.StreamedLayers(s, L, n_slots, n_pages, n_sel, gpu)
        stream = torch.cuda.current_stream()
        ws = K.paged.DecodeWorkspace(s, 1, n_sel * 256, 0, device=gpu)
        out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
        keep = torch.empty((steps, L, 24, 256), dtype=torch.float32, device=gpu)
        bts, miss, evs = [], [], []
        for st in range(steps):
            if mode != "per_layer":
                ev = None
                if mode == "layers_timed":
                    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    evs.append(ev)
                miss.append(list(sl.gather_layers(np.stack(sels[st]), host, stream, events=ev)))
            else:
                miss.append([sl.gather(layer, sels[st][layer], host[layer], stream) for layer in range(L)])
            bts.append(sl.block_table_all.cpu().numpy().copy())
            for layer in range(L):
                sl.attend(layer, q[st, layer], ctx, n_sel * 256, out, ws.data, stream)
                keep[st, layer].copy_(out[0])
        torch.cuda.synchronize()
        assert ws.status() == 0
        for (e0, e1), m in zip(evs, miss):  # a copy kernel ran between the events of each step
            assert e0.elapsed_time(e1) > 0.0 or sum(m) == 0
        runs.append((keep.cpu().numpy(), bts, miss, [t.slot_page.copy() for t in sl.tables],
                     [t.hand for t in sl.tables], [x.cpu().numpy() for x in sl.slots]))
    a = runs[0]
    for b in runs[1:]:
        assert a[2] == b[2], "misses per layer"
        assert all(np.array_equal(x, y) for x, y in zip(a[1], b[1])), "block tables"
        assert all(np.array_equal(x, y) for x, y in zip(a[3], b[3])) and a[4] == b[4], "residency tables"
        assert all(np.array_equal(x, y) for x, y in zip(a[5], b[5])), "slot contents"
        assert np.array_equal(a[0], b[0]), "attention outputs"
    assert sum(sum(m) for m in a[2]) > 0


@pytest.mark.parametrize("fmt", ["int8", "q4_0"])
def test_overlapped_streaming_equals_serial(gpu, fmt):
    """Each layer's gather on a copy stream, overlapped with the attention of earlier
    layers (and of the previous step), gives bit for bit the outputs of the same calls
    serialized on one stream."""
    L, n_pages, n_slots, n_sel, steps = 3, 40, 12, 8, 5
    s = K.shape(fmt)
    seqs = [Sequence(34, layer, 0, n_pages * 256, fmt) for layer in range(L)]
    host = [torch.from_numpy(sq.pages.reshape(-1).copy()).pin_memory() for sq in seqs]
    sels = draw_selections(L, n_pages, n_slots, n_sel, steps, 5)
    q = to_dev(kvsynth.q_np(34, 0, steps * L).reshape(steps, L, 1, 24, 256), gpu)
    ctx = to_dev(np.array([n_sel * 256], np.int32), gpu)
    results = []
    for overlap in (False, True):
        sl = K.streaming.StreamedLayers(s, L, n_slots, n_pages, n_sel, gpu, overlap=overlap)
        stream = torch.cuda.current_stream()
        ws = K.paged.DecodeWorkspace(s, 1, n_sel * 256, 0, device=gpu)
        out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
        keep = torch.empty((steps, L, 24, 256), dtype=torch.float32, device=gpu)
        for st in range(steps):
            for layer in range(L):
                sl.gather(layer, sels[st][layer], host[layer], stream)
                sl.attend(layer, q[st, layer], ctx, n_sel * 256, out, ws.data, stream)
                keep[st, layer].copy_(out[0])
        torch.cuda.synchronize()
        assert ws.status() == 0
        results.append(keep.cpu().numpy())
    assert np.array_equal(results[0], results[1])
    # and the outputs are those of attention over the selected pages
    for st in (0, steps - 1):
        for layer in range(L):
            sel = sels[st][layer]
            k = np.concatenate([seqs[layer].k[256 * p:256 * p + 256] for p in sel])
            v = np.concatenate([seqs[layer].v[256 * p:256 * p + 256] for p in sel])
            sub = Sequence(34, layer, 0, n_sel * 256, fmt, k=k, v=v)
            assert_close(results[1][st, layer][None], oracle_out(q[st, layer].cpu().numpy(), [sub], fmt),
                         what=f"step {st} layer {layer}")


def test_gather_layers_beyond_one_launch(gpu):
    """A kv_gather_pages_layers call with more copies (96) and block-table entries (256) than
    one launch carries is split into several launches; it leaves the same tables, slots and
    block tables as kv_gather_pages per layer, and the timed form's events span all of its
    launches. Pages are random bytes (the copy is verbatim)."""
    s = K.shape("int8")
    pb = K.page_bytes(s)
    L, n_pages, n_slots, n_sel = 5, 80, 64, 64  # 320 entries, 320 copies at the first step
    rng = np.random.default_rng(71)
    host = [torch.from_numpy(rng.integers(0, 256, n_pages * pb, dtype=np.uint8)).pin_memory() for _ in range(L)]
    sels = [np.stack([rng.permutation(n_pages)[:n_sel].astype(np.int32) for _ in range(L)]) for _ in range(3)]
    stream = torch.cuda.current_stream()
    runs = []
    for timed in (False, True):
        sl = K.streaming.StreamedLayers(s, L, n_slots, n_pages, n_sel, gpu)
        miss, bts = [], []
        for st in range(3):
            if timed:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                m = sl.gather_layers(sels[st], host, stream, events=ev)
                torch.cuda.synchronize()
                assert ev[0].elapsed_time(ev[1]) > 0.0
            else:
                m = np.array([sl.gather(layer, sels[st][layer], host[layer], stream) for layer in range(L)])
            miss.append(m.tolist())
            bts.append(sl.block_table_all.cpu().numpy().copy())
        torch.cuda.synchronize()
        runs.append((miss, bts, [t.slot_page.copy() for t in sl.tables], [x.cpu() for x in sl.slots]))
        # every selected page of the last step sits in its slot
        for layer in range(L):
            for i in range(0, n_sel, 7):
                slot, page = int(bts[-1][layer, i]), int(sels[-1][layer, i])
                assert torch.equal(runs[-1][3][layer][slot * pb:(slot + 1) * pb], host[layer][page * pb:(page + 1) * pb])
    a, b = runs
    assert a[0] == b[0] and sum(a[0][0]) == L * n_sel, "misses per layer"
    assert all(np.array_equal(x, y) for x, y in zip(a[1], b[1])), "block tables"
    assert all(np.array_equal(x, y) for x, y in zip(a[2], b[2])), "residency tables"
    assert all(torch.equal(x, y) for x, y in zip(a[3], b[3])), "slot contents"
