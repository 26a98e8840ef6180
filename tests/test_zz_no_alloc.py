"""kv_decode_attention_noalloc (the decode entry point that allocates nothing, for callers
that cannot allocate) against kv_decode_attention with a workspace: the same outputs, bit
for bit, on consecutive calls that share the library's device array, a later call smaller
than an earlier one; every output also within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K

from gpu_helpers import Sequence, assert_close, oracle_out, place_pages

pytestmark = pytest.mark.gpu


def case(gpu, fmt, lens, seed):
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    seqs = [Sequence(36, 0, b, T, fmt) for b, T in enumerate(lens)]
    pool, bt = place_pages(seqs, sum(sq.n_pages for sq in seqs) + 3, seed, pb)
    q = kvsynth.q_np(36, seed, len(lens))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    return s, seqs, q, dev(pool), dev(bt), dev(np.array(lens, np.int32)), dev(q)


# (format, context lengths, pages per split): the first call takes the counter-fed kernel
# form (129 splits x 4 KV heads at one page per split, more items than resident
# workgroups), the next ones are smaller (fewer splits, a batch of two), then the first
# again, so the counters that one call leaves in the array serve the next
CALLS = [("q4_0", [33000], 1), ("q4_0", [3000, 700], 0), ("int8", [600], 0), ("q4_0", [33000], 1)]


def test_noalloc_equals_workspace_entry_point(gpu):
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    built = {}
    for i, (fmt, lens, pps) in enumerate(CALLS):
        key = (fmt, tuple(lens))
        if key not in built:
            built[key] = case(gpu, fmt, lens, seed=50 + len(built))
        s, seqs, q, pool, bt, ctx, qd = built[key]
        max_ctx = max(lens)
        out_n = torch.full((len(lens), 24, 256), float("nan"), dtype=torch.float32, device=gpu)
        K.decode_attention_noalloc(s, qd, pool, bt, ctx, max_ctx, out_n, status=status, pages_per_split=pps)
        ws = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
        out_w = torch.empty_like(out_n)
        K.decode_attention(s, qd, pool, bt, ctx, max_ctx, out_w, ws.data, pages_per_split=pps)
        torch.cuda.synchronize()
        assert status.item() == 0 and ws.status() == 0, f"call {i}"
        got = out_n.cpu().numpy()
        assert np.array_equal(got, out_w.cpu().numpy()), f"call {i} ({fmt} {lens}): outputs differ"
        assert_close(got, oracle_out(q, seqs, fmt), what=f"call {i} ({fmt} {lens})")


def test_noalloc_reports_bad_pages_in_the_callers_status(gpu):
    s, seqs, q, pool, bt, ctx, qd = case(gpu, "q4_0", [900], seed=60)
    bad = bt.clone()
    bad[0, 1] = 10 ** 6
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    K.decode_attention_noalloc(s, qd, pool, bad, ctx, 900, out, status=status)
    torch.cuda.synchronize()
    assert status.item() & K.KV_STATUS_BAD_PAGE_ID
    # the next call, with a good table and no status word, is unaffected
    K.decode_attention_noalloc(s, qd, pool, bt, ctx, 900, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle_out(q, seqs, "q4_0"), what="after a flagged call")
