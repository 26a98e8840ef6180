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


@pytest.mark.parametrize("fmt", ["int8", "k8v4"])
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
