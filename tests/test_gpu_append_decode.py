"""kv_append_decode: the decode step with the new token's append fused into the
split-K kernel, against the two separate calls (kv_append_quantize of the token,
then kv_decode_attention) and the fp64 oracle.

The fused step must leave the pool byte for byte as the separate append does and
give bit-identical outputs, for every position of the new token in its page (first
row of a page that is the first of its split, the upper and lower token of a
4-bit V byte pair, the last row), for several split sizes and for mixed batches.
"""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K

from oracle import layout

from gpu_helpers import Sequence, assert_close, fmt_id, oracle_out

pytestmark = pytest.mark.gpu

FMTS = ["int8", "q4_0", "k8v4", "fp4", "fp8"]


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def build_step(fmt, lens, seed, cfg=31):
    """Pool holding tokens 0..T-2 of every sequence (oracle records, shuffled pages,
    garbage elsewhere, including the row the new token goes to), block tables with
    room for token T-1, the tokens' K, V [T, 4, 256], and each sequence's oracle
    records of all T tokens (the pool's pages are packed from their first T-1)."""
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    kv = [kvsynth.kv_tokens_np(cfg, 0, b, 0, T) for b, T in enumerate(lens)]
    full = [Sequence(cfg, 0, b, T, fmt, k=kv[b][0], v=kv[b][1]) for b, T in enumerate(lens)]
    need = [-(-T // 256) for T in lens]
    n_pool = sum(need) + 2
    perm = kvsynth.permutation_np(seed, n_pool)
    rng = np.random.default_rng(seed + 1)
    pool = rng.integers(0, 256, n_pool * pb, dtype=np.uint8).reshape(n_pool, pb)
    bt = np.zeros((len(lens), max(1, max(need))), np.int32)
    nxt = 0
    for b, sq in enumerate(full):
        pre = (layout.pack_pages(*(r[:sq.T - 1] for r in sq.rec), fmt_id(fmt)) if sq.T > 1
               else np.zeros((0, pb), np.uint8))
        for p in range(need[b]):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, p] = phys
            if p < pre.shape[0]:
                pool[phys] = pre[p]
    return s, pool.reshape(-1), bt, kv, full


def new_tokens(kv, lens):
    kn = np.zeros((len(lens), 4, 256), np.float16)
    vn = np.zeros_like(kn)
    for b, T in enumerate(lens):
        if T > 0:
            kn[b], vn[b] = kv[b][0][T - 1], kv[b][1][T - 1]
    return kn, vn


def run_both(gpu, fmt, lens, pps, seed, q):
    s, pool_np, bt, kv, full = build_step(fmt, lens, seed)
    kn, vn = new_tokens(kv, lens)
    ctx = np.array(lens, np.int32)
    max_ctx = int(max(1, max(lens)))
    btd, ctxd, qd = to_dev(bt, gpu), to_dev(ctx, gpu), to_dev(q, gpu)
    # separate calls
    pool_a = to_dev(pool_np, gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    for b, T in enumerate(lens):
        if T > 0:
            K.append_quantize(s, to_dev(kn[b:b + 1], gpu), to_dev(vn[b:b + 1], gpu), T - 1,
                              btd[b].contiguous(), pool_a, status)
    ws_a = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
    out_a = torch.empty((len(lens), 24, 256), dtype=torch.float32, device=gpu)
    K.decode_attention(s, qd, pool_a, btd, ctxd, max_ctx, out_a, ws_a.data, pages_per_split=pps)
    # fused step
    pool_b = to_dev(pool_np, gpu)
    ws_b = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
    out_b = torch.empty_like(out_a)
    K.append_decode(s, to_dev(kn, gpu), to_dev(vn, gpu), qd, pool_b, btd, ctxd, max_ctx, out_b,
                    ws_b.data, pages_per_split=pps)
    torch.cuda.synchronize()
    assert status.item() == 0 and ws_a.status() == 0 and ws_b.status() == 0
    # the work counters (workspace bytes 4..11) are left at zero by both calls
    for ws in (ws_a, ws_b):
        assert not ws.data[4:12].cpu().numpy().any(), "work counters not reset"
    return full, pool_a.cpu().numpy(), pool_b.cpu().numpy(), out_a.cpu().numpy(), out_b.cpu().numpy(), bt


def check_new_rows(pool_bytes, seqs, fmt, bt):
    """The page holding each sequence's newest token, unpacked by the oracle's layout
    code: its rows up to and including that token equal the oracle's records (codes
    exactly, scales bit for bit)."""
    pb = K.page_bytes(K.shape(fmt))
    for b, sq in enumerate(seqs):
        if sq.T == 0:
            continue
        p = (sq.T - 1) // 256
        phys = int(bt[b, p])
        got = layout.unpack_pages(pool_bytes[phys * pb:(phys + 1) * pb][None], fmt_id(fmt), 4)
        n = sq.T - 256 * p
        for g, w, what in zip(got, sq.rec, ("K codes", "K scales", "V codes", "V scales")):
            g, w = np.ascontiguousarray(g[:n]), np.ascontiguousarray(w[256 * p:sq.T])
            if g.dtype == np.float16:
                g, w = g.view(np.uint16), w.astype(np.float16).view(np.uint16)
            assert np.array_equal(g, w.astype(g.dtype)), f"sequence {b}: {what} of page {p} differ"


# (name, context lengths after the append, pages per split)
CASES = [
    ("T1", [1], 0),                  # row 0 of page 0, the split's first page
    ("T17", [17], 0),                # row 16: upper token of a 4-bit V byte pair
    ("T33", [33], 0),                # row 32: lower token
    ("T256", [256], 0),              # last row of a page
    ("T257_pps1", [257], 1),         # first row of a page that starts a split
    ("T700_pps2", [700], 2),
    ("T4096_pps3", [4096], 3),       # last row of the page that starts the last split
    ("T3000", [3000], 0),
    ("batch", [1000, 4096, 17, 0, 513, 2], 2),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name, lens, pps", CASES, ids=[c[0] for c in CASES])
def test_fused_step_equals_separate_calls(gpu, fmt, name, lens, pps):
    q = kvsynth.q_np(31, 0, len(lens))
    seqs, pa, pb_, oa, ob, _ = run_both(gpu, fmt, lens, pps, seed=len(lens) * 5 + pps + 1, q=q)
    assert np.array_equal(pa, pb_), f"{fmt} {name}: pool bytes differ"
    assert np.array_equal(oa, ob), f"{fmt} {name}: outputs differ"
    assert_close(ob, oracle_out(q, seqs, fmt), what=f"{fmt} {name}")


def resident_workgroups(gpu, fmt):
    """Workgroups of the split kernel resident at once: two 4-wave workgroups per CU for
    4-bit K, one 8-wave workgroup for 8-bit K."""
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    return cus * (2 if fmt in ("q4_0", "fp4") else 1)


# More work items (split, sequence, KV head) than resident workgroups: the kernel form
# whose workgroups take further items from the workspace counter, with the append fused.
# (name, context lengths after the append, pages per split; None = the split size the
# library picks for the batch's total length, as the benchmark does for several sequences)
DYN_CASES = [
    ("mixed_total", [40000, 9000, 2000, 300], None),
    ("mixed_total_b", [12289, 1, 5000, 257, 700], None),  # rows 0, 0, 136, 0 and 187 of a page
    ("T40000_pps1", [40000], 1),
    ("T39937_pps1", [39937], 1),   # the token in row 0 of a page that starts a split
    ("T66000_pps2", [66000], 2),   # 129 splits x 4 KV heads
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name, lens, pps", DYN_CASES, ids=[c[0] for c in DYN_CASES])
def test_fused_counter_fed_equals_separate_calls(gpu, fmt, name, lens, pps):
    s = K.shape(fmt)
    if pps is None:
        pps = K.decode_split_pages(s, len(lens), max(lens), sum(lens))
    n_splits = -(-(-(-max(lens) // 256)) // pps)
    items = n_splits * s.n_kv_heads * len(lens)
    assert items > resident_workgroups(gpu, fmt), "case does not reach the counter-fed form"
    q = kvsynth.q_np(34, 0, len(lens))
    seqs, pa, pb_, oa, ob, bt = run_both(gpu, fmt, lens, pps, seed=len(lens) * 7 + pps, q=q)
    assert np.array_equal(pa, pb_), f"{fmt} {name}: pool bytes differ"
    assert np.array_equal(oa, ob), f"{fmt} {name}: outputs differ"
    # the pool after the step holds every sequence's records byte for byte (valid rows)
    check_new_rows(pb_, seqs, fmt, bt)
    assert_close(ob, oracle_out(q, seqs, fmt), what=f"{fmt} {name}")


@pytest.mark.parametrize("fmt", ["q4_0", "int8", "k8v4"])
def test_fused_counter_fed_steps_share_a_workspace(gpu, fmt):
    """Decode steps at one page per split (more items than resident workgroups) on one
    workspace, each appending its token inside the counter-fed kernel: every step matches
    the oracle, so the counters left by one call serve the next."""
    T0, steps = 33000, 3
    k, v = kvsynth.kv_tokens_np(35, 0, 0, 0, T0 + steps)
    s = K.shape(fmt)
    n_pages = -(-(T0 + steps) // 256)
    pool = K.paged.PagedPool(fmt, n_pages + 3, device=gpu)
    perm = kvsynth.permutation_np(77, n_pages + 3)[:n_pages].astype(np.int32)
    bt = to_dev(perm[None], gpu)
    kd, vd = to_dev(k, gpu), to_dev(v, gpu)
    pool.append(kd[:T0].contiguous(), vd[:T0].contiguous(), 0, bt[0].contiguous())
    ws = K.paged.DecodeWorkspace(s, 1, T0 + steps, 1, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    for st in range(steps):
        T = T0 + st + 1
        q = kvsynth.q_np(35, 0, 1, step=st)
        K.append_decode(s, kd[T - 1:T].contiguous(), vd[T - 1:T].contiguous(), to_dev(q, gpu), pool.data,
                        bt, to_dev(np.array([T], np.int32), gpu), T0 + steps, out, ws.data, pages_per_split=1)
        torch.cuda.synchronize()
        assert ws.status() == 0 and not ws.data[4:12].cpu().numpy().any()
        seq = Sequence(35, 0, 0, T, fmt, k=k[:T], v=v[:T])
        assert_close(out.cpu().numpy(), oracle_out(q, [seq], fmt), what=f"{fmt} step {st}")


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_steps_end_to_end(gpu, fmt):
    """Prefill by chunks, then decode steps that each append their token in the kernel."""
    T0, steps = 1500, 6
    k, v = kvsynth.kv_tokens_np(32, 0, 0, 0, T0 + steps)
    s = K.shape(fmt)
    pool = K.paged.PagedPool(fmt, 8, device=gpu)
    bt = to_dev(np.array([[5, 2, 7, 0, 3, 6, 1, 4]], np.int32), gpu)
    kd, vd = to_dev(k, gpu), to_dev(v, gpu)
    pool.append(kd[:T0].contiguous(), vd[:T0].contiguous(), 0, bt[0].contiguous())
    ws = K.paged.DecodeWorkspace(s, 1, T0 + steps, 0, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    for st in range(steps):
        T = T0 + st + 1
        q = kvsynth.q_np(32, 0, 1, step=st)
        K.append_decode(s, kd[T - 1:T].contiguous(), vd[T - 1:T].contiguous(), to_dev(q, gpu), pool.data,
                        bt, to_dev(np.array([T], np.int32), gpu), T0 + steps, out, ws.data)
        torch.cuda.synchronize()
        assert ws.status() == 0
        seq = Sequence(32, 0, 0, T, fmt, k=k[:T], v=v[:T])
        assert_close(out.cpu().numpy(), oracle_out(q, [seq], fmt), what=f"step {st}")


def test_fused_step_bad_page_and_clamped_context(gpu):
    fmt = "q4_0"
    lens = [600]
    s, pool_np, bt, kv, _ = build_step(fmt, lens, seed=3)
    kn, vn = new_tokens(kv, lens)
    q = to_dev(kvsynth.q_np(33, 0, 1), gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    # the new token's page id outside the pool: nothing written, flagged
    bad = bt.copy()
    bad[0, 2] = 10 ** 6
    pool = to_dev(pool_np, gpu)
    ws = K.paged.DecodeWorkspace(s, 1, 600, 0, device=gpu)
    K.append_decode(s, to_dev(kn, gpu), to_dev(vn, gpu), q, pool, to_dev(bad, gpu),
                    to_dev(np.array(lens, np.int32), gpu), 600, out, ws.data)
    torch.cuda.synchronize()
    assert ws.status() & K.KV_STATUS_BAD_PAGE_ID
    assert np.array_equal(pool.cpu().numpy(), pool_np)
    # a context length above the bound: clamped, flagged, and no token appended
    pool = to_dev(pool_np, gpu)
    ws = K.paged.DecodeWorkspace(s, 1, 600, 0, device=gpu)
    K.append_decode(s, to_dev(kn, gpu), to_dev(vn, gpu), q, pool, to_dev(bt, gpu),
                    to_dev(np.array([601], np.int32), gpu), 600, out, ws.data)
    torch.cuda.synchronize()
    assert ws.status() & K.KV_STATUS_CONTEXT_CLAMPED
    assert np.array_equal(pool.cpu().numpy(), pool_np)
