"""GPU parity of the HIP path against the fp64 oracle (through the C ABI).

* quantize-on-append: pool bytes bit-exact to the oracle's records and layout;
* decode attention on oracle-packed pools: max-abs <= 2e-3, rel-L2 <= 1e-3;
* split-count independence, placement independence (bitwise), masking of
  stale rows, T = 0, status flags for bad page ids and clamped contexts.
"""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K
from oracle import layout, records

from gpu_helpers import Sequence, assert_close, fmt_id, oracle_out, oracle_records, place_pages

pytestmark = pytest.mark.gpu

FMTS = ["int8", "q4_0", "k8v4", "fp4", "fp8"]


def to_dev(a, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


def special_vectors(n_kv_heads=4):
    """fp16 token vectors that hit the rounding edge cases."""
    vs = []
    z = np.zeros((n_kv_heads, 256), np.float16)
    vs.append(z)                                               # all zero: d = 0
    t = np.zeros((n_kv_heads, 256), np.float16)
    t[:, 0] = 127 / 16
    t[:, 1:5] = np.array([2.5, -2.5, 0.5, -0.5], np.float16) / 16   # int8 ties
    vs.append(t)
    s = np.full((n_kv_heads, 256), np.float16(2.0 ** -24))     # subnormal inputs
    s[:, ::2] *= -3
    vs.append(s)
    big = np.zeros((n_kv_heads, 256), np.float16)
    big[:, 7] = 2048.0
    big[:, 100] = -2048.0                                        # sign tie in a block
    vs.append(big)
    e = np.zeros((n_kv_heads, 256), np.float16)
    e[:, :32] = np.arange(-8, 24)[:32].astype(np.float16) * 0.25   # integer multiples
    vs.append(e)
    return np.stack(vs)


@pytest.mark.parametrize("fmt", FMTS)
def test_append_bitexact(gpu, fmt):
    T = 700
    k, v = kvsynth.kv_tokens_np(11, 0, 0, 0, T)
    sp = special_vectors()
    k[40:40 + len(sp)] = sp
    v[300:300 + len(sp)] = sp
    v[41:41 + len(sp)] = sp[::-1]
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    n_pool = 6
    bt = np.array([4, 1, 3], np.int32)
    rng = np.random.default_rng(5)
    pool = to_dev(rng.integers(0, 256, n_pool * pb, dtype=np.uint8), gpu)
    kd, vd = to_dev(k, gpu), to_dev(v, gpu)
    btd = to_dev(bt, gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    for a, b in ((0, 1), (1, 18), (18, 300), (300, 301), (301, 512), (512, 700)):
        K.append_quantize(s, kd[a:b].contiguous(), vd[a:b].contiguous(), a, btd, pool, status)
    torch.cuda.synchronize()
    assert status.item() == 0
    got_pages = pool.cpu().numpy().reshape(n_pool, pb)[bt]
    kc, ks, vc, vs = oracle_records(k, v, fmt)
    a, b_, c, d = layout.unpack_pages(got_pages, fmt_id(fmt), 4)
    assert np.array_equal(a[:T], kc), "K codes"
    assert np.array_equal(b_[:T].view(np.uint16), ks.view(np.uint16)), "K scales"
    assert np.array_equal(c[:T], vc), "V codes"
    assert np.array_equal(d[:T].view(np.uint16), vs.view(np.uint16)), "V scales"
    # whole pages are byte-identical to the oracle's packing
    want = layout.pack_pages(kc, ks, vc, vs, fmt_id(fmt))
    assert np.array_equal(got_pages[:2], want[:2])


def rounding_edge_vectors(n_kv_heads=4):
    """Vectors a e_0 + b e_1: after the rotation every element is (a +- b) / 16, so the
    q4 scale is fp16(-(a + b) / 128) and the other elements sit at -8 (a - b) / (a + b)
    in units of it. Chosen to hit fp16 ties of the scale (2049, 2051: ties to even),
    a value just past a tie, code ties (-0.5, -3.5: half up) and a subnormal scale."""
    pairs = [(2048, 1), (2048, 3), (2048, 1 + 2 ** -10), (17, 15), (23, 9), (-23, -9),
             (2 ** -14, 2 ** -20), (2048, -1), (65504, 65504)]
    vs = []
    for a, b in pairs:
        x = np.zeros((n_kv_heads, 256), np.float16)
        x[:, 0], x[:, 1] = a, b
        vs.append(x)
        y = x.copy()
        y[:, 0], y[:, 1] = b, a  # the larger magnitude second
        vs.append(y)
    return np.stack(vs)


def fp4_edge_vectors(n_kv_heads=4):
    """fp4 block-scale and grid edge cases. With a + b = 1024 the block maximum is
    64 = 4 d (d = 16) and the other element sits at (a - b) / 256 in units of d: the
    grid midpoints 0.25, 0.75, 1.25, 1.75, 2.5 and 3.5 (ties to the even index). With
    a + b = 1920 the maximum 7.5 d saturates and (a - b) = 1280 is the tie 5.0. A tiny
    pair puts the block exponent below its floor (-23); a Sylvester row of 4096s gives
    y = 65,536 in one slot, above the exponent's ceiling (13), so the codes saturate."""
    pairs = [(544, 480), (608, 416), (672, 352), (736, 288), (832, 192), (960, 64),
             (1600, 320), (2.0 ** -18, 2.0 ** -19), (2.0 ** -17, -(2.0 ** -20))]
    vs = []
    for a, b in pairs:
        x = np.zeros((n_kv_heads, 256), np.float16)
        x[:, 0], x[:, 1] = a, b
        vs.append(x)
    j = np.arange(256)
    x = np.zeros((n_kv_heads, 256), np.float16)
    for h in range(n_kv_heads):
        kk = 3 + 41 * h
        x[h] = 4096.0 * (1.0 - 2.0 * (np.array([bin(t & kk).count("1") for t in j]) & 1))
    vs.append(x)
    return np.stack(vs)


def fp8_edge_vectors(n_kv_heads=4):
    """E4M3 edge cases. With the largest element 448 (d = 1) or 896 (d = 2), the other
    elements sit on every midpoint between neighbouring E4M3 magnitudes (ties to the
    even code), with both signs; a vector of 627 * 2^-24 has the subnormal scale 2^-24
    and saturates; one just below fp16's largest value has d = 146.25."""
    e = np.arange(127)
    ex, m = e >> 3, e & 7
    mag = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ex - 7.0))
    mids = (mag[1:] + mag[:-1]) / 2                                   # 126 ties
    vs = []
    for top in (448.0, 896.0):
        x = np.zeros((n_kv_heads, 256))
        x[:, 0] = top
        x[:, 1:127] = mids * (top / 448.0)
        x[:, 127:253] = -mids * (top / 448.0)
        x[:, 253] = -top
        vs.append(x.astype(np.float16))
    x = np.zeros((n_kv_heads, 256))
    x[:, 0], x[:, 1], x[:, 2] = 627 * 2.0 ** -24, -300 * 2.0 ** -24, 2.0 ** -24
    vs.append(x.astype(np.float16))
    x = np.zeros((n_kv_heads, 256))
    x[:, 0], x[:, 1], x[:, 2] = 65504.0, -65504.0, 146.0
    vs.append(x.astype(np.float16))
    return np.stack(vs)


@pytest.mark.parametrize("fmt", FMTS)
def test_append_rounding_edges_bitexact(gpu, fmt):
    """Scale and code rounding edge cases appended one token at a time and as a chunk,
    bit for bit against the oracle's records."""
    sp = np.concatenate([rounding_edge_vectors(), special_vectors(), fp4_edge_vectors(),
                         fp8_edge_vectors()])
    T = len(sp)
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    for chunk in (1, T):
        pool = torch.zeros(2 * pb, dtype=torch.uint8, device=gpu)
        btd = to_dev(np.array([1], np.int32), gpu)
        status = torch.zeros(1, dtype=torch.int32, device=gpu)
        kd, vd = to_dev(sp, gpu), to_dev(sp[::-1].copy(), gpu)
        for a in range(0, T, chunk):
            K.append_quantize(s, kd[a:a + chunk].contiguous(), vd[a:a + chunk].contiguous(), a, btd, pool, status)
        torch.cuda.synchronize()
        assert status.item() == 0
        got = pool.cpu().numpy().reshape(2, pb)[[1]]
        kc, ks, vc, vs = oracle_records(sp, sp[::-1].copy(), fmt)
        a_, b_, c_, d_ = layout.unpack_pages(got, fmt_id(fmt), 4)
        assert np.array_equal(a_[:T], kc), f"K codes (chunk {chunk})"
        assert np.array_equal(b_[:T].view(np.uint16), ks.view(np.uint16)), f"K scales (chunk {chunk})"
        assert np.array_equal(c_[:T], vc), f"V codes (chunk {chunk})"
        assert np.array_equal(d_[:T].view(np.uint16), vs.view(np.uint16)), f"V scales (chunk {chunk})"


@pytest.mark.parametrize("fmt", FMTS)
def test_append_bad_page_id_is_skipped_and_flagged(gpu, fmt):
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    k, v = kvsynth.kv_tokens_np(12, 0, 0, 0, 10)
    pool = torch.zeros(2 * pb, dtype=torch.uint8, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    K.append_quantize(s, to_dev(k, gpu), to_dev(v, gpu), 0, to_dev(np.array([7], np.int32), gpu), pool, status)
    torch.cuda.synchronize()
    assert status.item() & K.KV_STATUS_BAD_PAGE_ID
    assert int(pool.sum().item()) == 0


def run_decode(gpu, fmt, seqs, q, pps=0, seed=0, n_pool_extra=3):
    s = K.shape(fmt, q.shape[1], seqs[0].k.shape[1])
    pb = K.page_bytes(s)
    n_pool = sum(x.n_pages for x in seqs) + n_pool_extra
    pool_np, bt = place_pages(seqs, n_pool, seed, pb)
    pool = to_dev(pool_np, gpu)
    lens = np.array([x.T for x in seqs], np.int32)
    max_ctx = int(max(lens.max(), 1))
    ws = K.paged.DecodeWorkspace(s, len(seqs), max_ctx, pps, device=gpu)
    out = torch.empty((len(seqs), q.shape[1], 256), dtype=torch.float32, device=gpu)
    K.decode_attention(s, to_dev(q, gpu), pool, to_dev(bt, gpu), to_dev(lens, gpu), max_ctx, out,
                       ws.data, pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws.status()


CASES = [
    ("T1", [1], 0), ("T2", [2], 0), ("T7", [7], 0), ("T8", [8], 0),
    ("T255", [255], 0), ("T256", [256], 0), ("T257", [257], 0),
    ("T1000_pps1", [1000], 1), ("T4096", [4096], 0), ("T4096_pps3", [4096], 3),
    ("batch_mixed", [1000, 4096, 17, 0, 513], 2),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name, lens, pps", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(gpu, fmt, name, lens, pps):
    seqs = [Sequence(21, 0, b, T, fmt) for b, T in enumerate(lens)]
    q = kvsynth.q_np(21, 0, len(lens))
    got, status = run_decode(gpu, fmt, seqs, q, pps, seed=len(lens) * 7 + pps)
    assert status == 0
    want = oracle_out(q, seqs, fmt)
    assert_close(got, want, what=f"{fmt} {name}")
    for b, T in enumerate(lens):
        if T == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b]))


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_split_and_placement_independence(gpu, fmt):
    seqs = [Sequence(22, 1, 0, 3000, fmt)]
    q = kvsynth.q_np(22, 1, 1)
    want = oracle_out(q, seqs, fmt)
    outs = {}
    for pps in (1, 2, 4, 12):
        got, _ = run_decode(gpu, fmt, seqs, q, pps, seed=1)
        assert_close(got, want, what=f"pps {pps}")
        outs[pps] = got
    # same split, different physical placement: bitwise identical
    again, _ = run_decode(gpu, fmt, seqs, q, 4, seed=99, n_pool_extra=9)
    assert np.array_equal(again, outs[4])


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_group_sizes(gpu, fmt):
    """Other GQA groupings: 8, 1 and 3 query heads per KV head."""
    for hq, hkv in ((16, 2), (4, 4), (6, 2)):
        k, v = kvsynth.kv_tokens_np(23, hq, 0, 0, 600, hkv)
        seqs = [Sequence(23, hq, 0, 600, fmt, hkv, k, v)]
        q = kvsynth.q_np(23, hq, 1, hq)
        got, _ = run_decode(gpu, fmt, seqs, q, 0, seed=hq)
        assert_close(got, oracle_out(q, seqs, fmt), what=f"{hq}/{hkv}")


def test_decode_flags_bad_page_and_clamped_context(gpu):
    fmt = "q4_0"
    seqs = [Sequence(24, 0, 0, 600, fmt)]
    q = kvsynth.q_np(24, 0, 1)
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    pool_np, bt = place_pages(seqs, 5, 3, pb)
    pool = to_dev(pool_np, gpu)
    ws = K.paged.DecodeWorkspace(s, 1, 600, 1, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    bad = bt.copy()
    bad[0, 1] = 1000
    K.decode_attention(s, to_dev(q, gpu), pool, to_dev(bad, gpu), to_dev(np.array([600], np.int32), gpu),
                       600, out, ws.data, pages_per_split=1)
    torch.cuda.synchronize()
    assert ws.status() & K.KV_STATUS_BAD_PAGE_ID
    assert np.all(np.isfinite(out.cpu().numpy()))
    ws.clear_status()
    # a context length above the declared bound is clamped to it and flagged
    K.decode_attention(s, to_dev(q, gpu), pool, to_dev(bt, gpu), to_dev(np.array([650], np.int32), gpu),
                       600, out, ws.data, pages_per_split=1)
    torch.cuda.synchronize()
    assert ws.status() & K.KV_STATUS_CONTEXT_CLAMPED
    assert_close(out.cpu().numpy(), oracle_out(q, seqs, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_append_then_decode_end_to_end(gpu, fmt):
    """Pool written by the append kernel (prefill chunk + decode steps), read by decode."""
    T0, steps = 2000, 5
    k, v = kvsynth.kv_tokens_np(25, 0, 0, 0, T0 + steps)
    s = K.shape(fmt)
    pool = K.paged.PagedPool(fmt, 12, device=gpu)
    bt = to_dev(np.array([9, 2, 7, 0, 11, 5, 3, 1, 4, 6, 8, 10], np.int32), gpu)
    kd, vd = to_dev(k, gpu), to_dev(v, gpu)
    pool.append(kd[:T0].contiguous(), vd[:T0].contiguous(), 0, bt)
    ws = K.paged.DecodeWorkspace(s, 1, T0 + steps, 0, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    for st in range(steps):
        T = T0 + st + 1
        pool.append(kd[T - 1:T].contiguous(), vd[T - 1:T].contiguous(), T - 1, bt)
        q = kvsynth.q_np(25, 0, 1, step=st)
        K.decode_attention(s, to_dev(q, gpu), pool.data, bt[None].contiguous(),
                           to_dev(np.array([T], np.int32), gpu), T0 + steps, out, ws.data)
        torch.cuda.synchronize()
        seq = Sequence(25, 0, 0, T, fmt, k=k[:T], v=v[:T])
        assert_close(out.cpu().numpy(), oracle_out(q, [seq], fmt), what=f"step {st}")


def test_decode_split_timed_matches_split(gpu):
    """kv_decode_split_timed does the same work as kv_decode_split and records its events."""
    fmt = "q4_0"
    seqs = [Sequence(26, 0, 0, 2500, fmt)]
    q = kvsynth.q_np(26, 0, 1)
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    pool_np, bt = place_pages(seqs, 12, 7, pb)
    pool, btd = to_dev(pool_np, gpu), to_dev(bt, gpu)
    qd, ctx = to_dev(q, gpu), to_dev(np.array([2500], np.int32), gpu)
    outs = []
    for timed in (False, True):
        ws = K.paged.DecodeWorkspace(s, 1, 2500, 0, device=gpu)
        out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
        K.decode_attention(s, qd, pool, btd, ctx, 2500, out, ws.data, phase="split", events=ev)
        K.decode_attention(s, qd, pool, btd, ctx, 2500, out, ws.data, phase="combine")
        torch.cuda.synchronize()
        if timed:
            assert ev[0].elapsed_time(ev[1]) > 0
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert_close(outs[1], oracle_out(q, seqs, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_append_timed_matches_append(gpu, fmt):
    """kv_append_quantize_timed writes the same bytes as kv_append_quantize (a ragged chunk
    of 700 tokens from position 45, so both edge groups are partly covered) and records
    its events."""
    s = K.shape(fmt)
    k, v = kvsynth.kv_tokens_np(27, 0, 0, 0, 745)
    bt = to_dev(np.array([2, 0, 3, 1], np.int32), gpu)
    pools = []
    for timed in (False, True):
        pool = K.paged.PagedPool(fmt, 4, device=gpu)
        pool.data.copy_(torch.from_numpy(np.random.default_rng(5).integers(0, 256, pool.data.numel(), dtype=np.uint8)))
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
        pool.append(to_dev(k[45:], gpu), to_dev(v[45:], gpu), 45, bt, events=ev)
        torch.cuda.synchronize()
        if timed:
            assert ev[0].elapsed_time(ev[1]) > 0
        pools.append(pool.data.cpu().numpy())
    assert np.array_equal(pools[0], pools[1])


def extreme_v(v, fmt):
    """Plant V vectors whose scales leave the folded-constant range: a huge one
    (q4: y = H v has one element 32,000, so d = -4,000; int8: one element 8,000,
    d ~ 63) and tiny ones (fp16 subnormal inputs, d far below 2^-10)."""
    v = v.copy()
    j = np.arange(256)
    for h in range(v.shape[1]):
        kk = 5 + 37 * h
        sign = 1.0 - 2.0 * (np.array([bin(x & kk).count("1") for x in j]) & 1)
        v[50, h] = (2000.0 * sign).astype(np.float16)           # q4: y_kk = 16 * 2000
        v[51, h] = 0
        v[51, h, 3 + h] = 8000.0                                  # int8: d = 8000 / 127
        v[300, h] = (np.arange(256) % 7 - 3).astype(np.float16) * np.float16(2.0 ** -24)
        v[301, h] = (np.arange(256) % 5 - 2).astype(np.float16) * np.float16(2.0 ** -16)
    return v


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_extreme_scales(gpu, fmt):
    """Pages whose V scales fall outside the fast path's exact range (huge, tiny,
    subnormal) take the exact slower path and still match the oracle."""
    T = 700
    k, v = kvsynth.kv_tokens_np(27, 0, 0, 0, T)
    v = extreme_v(v, fmt)
    seqs = [Sequence(27, 0, 0, T, fmt, 4, k, v)]
    q = kvsynth.q_np(27, 0, 1)
    for pps in (0, 1):
        got, status = run_decode(gpu, fmt, seqs, q, pps, seed=5 + pps)
        assert status == 0
        assert_close(got, oracle_out(q, seqs, fmt), what=f"{fmt} pps {pps}")


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_ignores_stale_rows(gpu, fmt):
    """Rows past the context on a sequence's last page may hold anything (records of an
    earlier sequence, NaN scales, the E4M3 NaN code 0x7F): the output depends only on the
    tokens in context."""
    T = 300
    seq = Sequence(29, 0, 0, T, fmt)
    kk, vk = records.kinds(fmt_id(fmt))
    pad = 512 - T

    def junk(a, kind, is_code):
        if is_code:
            val = {records.KIND_INT8: 127, records.KIND_FP8: 0x7F}.get(kind, 15)
        else:
            val = np.nan
        return np.concatenate([a, np.full((pad,) + a.shape[1:], val, a.dtype)])

    kc, ks, vc, vs = seq.rec
    seq.pages = layout.pack_pages(junk(kc, kk, True), junk(ks, kk, False), junk(vc, vk, True),
                                  junk(vs, vk, False), fmt_id(fmt))
    assert seq.pages.shape[0] == seq.n_pages == 2
    q = kvsynth.q_np(29, 0, 1)
    want = oracle_out(q, [seq], fmt)
    for pps in (0, 1):
        got, status = run_decode(gpu, fmt, [seq], q, pps, seed=11 + pps)
        assert status == 0
        assert np.isfinite(got).all()
        assert_close(got, want, what=f"{fmt} pps {pps}")


MERGE_CASES = [
    ("T4096", [4096], 0),
    ("T3000_pps2", [3000], 2),
    ("T200k_pps1", [200000], 1),       # more work items than resident workgroups (counter-fed)
    ("batch", [1000, 4096, 17, 0, 513], 1),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name, lens, pps", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_attention_equals_its_two_phases(gpu, fmt, name, lens, pps):
    """kv_decode_attention is bit-identical to kv_decode_split then kv_decode_combine,
    also when more work items than resident workgroups are fed from the workspace
    counters, which every call leaves at zero for the next."""
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    need = [-(-T // 256) for T in lens]
    n_pool = sum(need) + 1
    rng = np.random.default_rng(len(lens) + pps)
    # valid records are not needed for a bitwise comparison of two merges: random bytes
    # with small positive fp16 scales (set through the oracle's layout of one page)
    one = layout.pack_pages(*records_of_noise(fmt, rng), fmt_id(fmt))[0]
    pool = to_dev(np.tile(one, n_pool), gpu)
    perm = kvsynth.permutation_np(3, n_pool)
    bt = np.zeros((len(lens), max(need)), np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    q = to_dev(kvsynth.q_np(27, 0, len(lens)), gpu)
    ctx, btd = to_dev(np.array(lens, np.int32), gpu), to_dev(bt, gpu)
    max_ctx = max(lens)
    outs = []
    for fused in (True, False, True):
        ws = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
        out = torch.full((len(lens), 24, 256), float("nan"), dtype=torch.float32, device=gpu)
        if fused:
            K.decode_attention(s, q, pool, btd, ctx, max_ctx, out, ws.data, pages_per_split=pps)
            K.decode_attention(s, q, pool, btd, ctx, max_ctx, out, ws.data, pages_per_split=pps)
        else:
            K.decode_attention(s, q, pool, btd, ctx, max_ctx, out, ws.data, pages_per_split=pps, phase="split")
            K.decode_attention(s, q, pool, btd, ctx, max_ctx, out, ws.data, pages_per_split=pps, phase="combine")
        torch.cuda.synchronize()
        assert ws.status() == 0
        assert int(ws.data[4:16].view(torch.int32).abs().sum().item()) == 0, "counters not reset"
        outs.append(out.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1]), f"{fmt} {name}: one call differs from its two phases"
    assert np.array_equal(outs[0], outs[2])


def records_of_noise(fmt, rng):
    """Oracle records of one page of noise vectors (256 tokens, 4 KV heads)."""
    k = (rng.standard_normal((256, 4, 256)) * 2).astype(np.float16)
    v = (rng.standard_normal((256, 4, 256)) * 2).astype(np.float16)
    return oracle_records(k, v, fmt)
