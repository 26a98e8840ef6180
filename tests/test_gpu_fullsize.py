"""Parity at full benchmark sizes, in the launch configuration the benchmark uses.

* One layer of 131,072 tokens in q4_0 (24 query / 4 KV heads), the same in fp4
  and fp8, one layer of 32,768 int8 tokens and one of 1,048,576 q4_0 tokens: the
  cache is written by the append kernel in 2,048-token chunks through a shuffled
  block table, then the decode step appends the last token inside the split
  kernel with the automatic split count. Output and pool equal those of the
  separate append and decode calls bit for bit; every KV head (two at 1,048,576
  tokens) is checked against the fp64 oracle, and sampled pages of those heads
  byte for byte against the oracle's records.
* Four k8v4 sequences of 262,144 / 198,000 / 65,536 / 8,192 tokens in one
  shuffled pool (the 198,000-token one ends in a 112-token page): one KV head
  of every sequence is checked against the oracle.

K and V are drawn on the GPU (seeded, the benchmark's distribution) and appended
chunk by chunk; the checked heads' fp16 K and V are copied back and the oracle
encodes only those heads (its cost is the rotation of every vector of a head).
"""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K
from oracle import attention, layout, records

from gpu_helpers import assert_close, fmt_id

pytestmark = pytest.mark.gpu

CHUNK = 2048


def build_pool(gpu, fmt, cfg, lens, seed, g, filled=None):
    """Draw each sequence's K, V on the GPU in CHUNK-token pieces, append them into one
    pool with a shuffled block table, and return head g's fp16 K and V per sequence
    (g = None: every KV head). The pool has room for lens[b] tokens of sequence b;
    filled[b] (default lens[b]) of them are appended."""
    s = K.shape(fmt)
    filled = lens if filled is None else filled
    pages = [-(-T // 256) for T in lens]
    n_pool = sum(pages)
    perm = kvsynth.permutation_np(seed, n_pool)
    pool = K.paged.PagedPool(fmt, n_pool, device=gpu)
    bt = np.zeros((len(lens), max(pages)), np.int32)
    gain = kvsynth.gain_torch(cfg, 0, s.n_kv_heads, gpu)
    heads = []
    off = 0
    hs = slice(None) if g is None else slice(g, g + 1)
    for b, (T, n) in enumerate(zip(filled, pages)):
        bt[b, :n] = perm[off:off + n]
        off += n
        row = torch.from_numpy(bt[b]).to(gpu)
        gen = torch.Generator(device=gpu)
        gen.manual_seed(kvsynth.torch_seed(cfg, 0, b))
        kh, vh = [], []
        for t0 in range(0, T, CHUNK):
            kd, vd = kvsynth.kv_tokens_torch(gen, min(CHUNK, T - t0), gain, gpu)
            pool.append(kd, vd, t0, row)
            kh.append(kd[:, hs].cpu().numpy())
            vh.append(vd[:, hs].cpu().numpy())
        heads.append((np.concatenate(kh), np.concatenate(vh)))
    torch.cuda.synchronize()
    return s, pool, bt, heads


def decode(gpu, s, pool, bt, q, lens):
    max_ctx = int(max(lens))
    ws = K.paged.DecodeWorkspace(s, len(lens), max_ctx, 0, device=gpu)
    out = torch.empty((len(lens), s.n_q_heads, 256), dtype=torch.float32, device=gpu)
    K.decode_attention(s, torch.from_numpy(q).to(gpu), pool.data, torch.from_numpy(bt).to(gpu),
                       torch.from_numpy(np.array(lens, np.int32)).to(gpu), max_ctx, out, ws.data)
    torch.cuda.synchronize()
    assert ws.status() == 0
    return out.cpu().numpy()


def head_records(k, v, fmt):
    """Oracle records of one KV head's K, V [T, 1, 256]."""
    kk, vk = records.kinds(fmt_id(fmt))
    kc, ks = records.encode(k.astype(np.float64), kk)
    vc, vs = records.encode(v.astype(np.float64), vk)
    return kc, ks, vc, vs


def head_oracle(q_heads, rec, fmt):
    kk, vk = records.kinds(fmt_id(fmt))
    kh = records.decode(rec[0], rec[1], kk)
    vh = records.decode(rec[2], rec[3], vk)
    return attention.decode_attention(q_heads, kh, vh, fmt_id(fmt))


LAYERS = [("q4_0", 131072, 3), ("fp4", 131072, 3), ("fp8", 131072, 3), ("int8", 32768, 2),
          ("q4_0", 1048576, 3)]   # the top of the 128K-1M context range (32 pages per split)


@pytest.mark.parametrize("fmt, T, cfg", LAYERS, ids=[f"{f}_{t}" for f, t, _ in LAYERS])
def test_one_layer_sampled(gpu, fmt, T, cfg):
    """One layer at full size in the benchmark's form: tokens 0 .. T-2 appended in chunks, then
    the decode step that appends token T-1 inside the split kernel (kv_append_decode, the
    library's split size). Output and pool equal the separate calls bit for bit; every KV head
    (two of them at 1,048,576 tokens, to bound the host's oracle time) is checked against the
    oracle, and sampled pages of those heads byte for byte against the oracle's records."""
    heads_checked = [0, 1, 2, 3] if T <= 131072 else [0, 3]
    q = kvsynth.q_np(cfg, 0, 1)
    s, pool, bt, heads = build_pool(gpu, fmt, cfg, [T], seed=31, g=None, filled=[T - 1])
    rng = np.random.default_rng(3131)
    kn = (rng.standard_normal((1, 4, 256)) * 2).astype(np.float16)
    vn = (rng.standard_normal((1, 4, 256)) * 2).astype(np.float16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    btd, ctx, qd = dev(bt), dev(np.array([T], np.int32)), dev(q)
    before = pool.data.clone()
    ws = K.paged.DecodeWorkspace(s, 1, T, 0, device=gpu)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
    K.append_decode(s, dev(kn), dev(vn), qd, pool.data, btd, ctx, T, out, ws.data)
    K.append_quantize(s, dev(kn), dev(vn), T - 1, btd[0].contiguous(), before)
    ws2 = K.paged.DecodeWorkspace(s, 1, T, 0, device=gpu)
    out2 = torch.empty_like(out)
    K.decode_attention(s, qd, before, btd, ctx, T, out2, ws2.data)
    torch.cuda.synchronize()
    assert ws.status() == 0 and ws2.status() == 0
    assert torch.equal(pool.data, before), "pool bytes differ from the separate append"
    got = out.cpu().numpy()
    assert np.array_equal(got, out2.cpu().numpy()), "output differs from the separate calls"
    del before
    kh, vh = heads[0]
    pb = K.page_bytes(s)

    def check_head(g):
        k = np.concatenate([kh[:, g:g + 1], kn[:, g:g + 1]])
        v = np.concatenate([vh[:, g:g + 1], vn[:, g:g + 1]])
        rec = head_records(k, v, fmt)
        return rec, head_oracle(q[0, 6 * g:6 * g + 6], rec, fmt)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(check_head, heads_checked))
    for g, (rec, want) in zip(heads_checked, results):
        assert_close(got[0, 6 * g:6 * g + 6], want, what=f"{fmt} {T}, KV head {g}")
        # sampled pages of the head, byte for byte (first, second, middle and last page);
        # a page packs on its own, so only the sampled pages are packed
        for p in (0, 1, T // 512, (T - 1) // 256):
            one_head = layout.pack_pages(*(r[256 * p:256 * (p + 1)] for r in rec), fmt_id(fmt))[0]
            hs = one_head.shape[0]                            # bytes of one head's K + V planes
            phys = int(bt[0, p])
            dev_bytes = pool.data[phys * pb + g * hs: phys * pb + (g + 1) * hs].cpu().numpy()
            assert np.array_equal(dev_bytes, one_head), f"KV head {g}, page {p}"


def test_k8v4_four_sequences_sampled(gpu):
    fmt, cfg, g = "k8v4", 4, 2
    lens = [262144, 198000, 65536, 8192]
    q = kvsynth.q_np(cfg, 0, len(lens))
    s, pool, bt, heads = build_pool(gpu, fmt, cfg, lens, seed=41, g=g)
    got = decode(gpu, s, pool, bt, q, lens)
    for b, (kh, vh) in enumerate(heads):
        rec = head_records(kh, vh, fmt)
        want = head_oracle(q[b, 6 * g:6 * g + 6], rec, fmt)
        assert_close(got[b, 6 * g:6 * g + 6], want, what=f"k8v4 sequence {b} ({lens[b]} tokens)")


def test_k8v4_benchmark_step_all_heads(gpu):
    """The four-sequence k8v4 step exactly as the benchmark runs it: splits sized from the
    batch's total length (more work items than resident workgroups, so the counter-fed
    kernel form), each sequence's newest token appended inside the split kernel. Every KV
    head of every sequence is checked against the oracle, and the output and the pool are
    bit for bit those of the separate calls (append kernel, then decode attention)."""
    fmt, cfg = "k8v4", 4
    lens = [262144, 198000, 65536, 8192]
    s = K.shape(fmt)
    pps = K.decode_split_pages(s, len(lens), max(lens), sum(lens))
    n_splits = -(-(-(-max(lens) // 256)) // pps)
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    assert n_splits * s.n_kv_heads * len(lens) > cus, "not the counter-fed form"
    q = kvsynth.q_np(cfg, 1, len(lens))
    s, pool, bt, heads = build_pool(gpu, fmt, cfg, lens, seed=43, g=None, filled=[T - 1 for T in lens])
    rng = np.random.default_rng(4343)
    kn = (rng.standard_normal((len(lens), 4, 256)) * 2).astype(np.float16)
    vn = (rng.standard_normal((len(lens), 4, 256)) * 2).astype(np.float16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    btd, ctx, qd = dev(bt), dev(np.array(lens, np.int32)), dev(q)
    max_ctx = max(lens)
    before = pool.data.clone()
    ws = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
    out = torch.empty((len(lens), 24, 256), dtype=torch.float32, device=gpu)
    K.append_decode(s, dev(kn), dev(vn), qd, pool.data, btd, ctx, max_ctx, out, ws.data, pages_per_split=pps)
    # the separate calls on the pool as it was before the step
    for b, T in enumerate(lens):
        K.append_quantize(s, dev(kn[b:b + 1]), dev(vn[b:b + 1]), T - 1, btd[b].contiguous(), before)
    ws2 = K.paged.DecodeWorkspace(s, len(lens), max_ctx, pps, device=gpu)
    out2 = torch.empty_like(out)
    K.decode_attention(s, qd, before, btd, ctx, max_ctx, out2, ws2.data, pages_per_split=pps)
    torch.cuda.synchronize()
    assert ws.status() == 0 and ws2.status() == 0
    assert not ws.data[4:12].cpu().numpy().any(), "work counters not reset"
    assert torch.equal(pool.data, before), "pool bytes differ from the separate append"
    got = out.cpu().numpy()
    assert np.array_equal(got, out2.cpu().numpy()), "output differs from the separate calls"
    del before

    def oracle_head(bg):
        b, g = bg
        kh, vh = heads[b]
        k = np.concatenate([kh[:, g:g + 1], kn[b:b + 1, g:g + 1]])
        v = np.concatenate([vh[:, g:g + 1], vn[b:b + 1, g:g + 1]])
        return head_oracle(q[b, 6 * g:6 * g + 6], head_records(k, v, fmt), fmt)

    # (sequence, KV head) pairs on a few host threads: numpy's large array operations
    # release the interpreter lock
    from concurrent.futures import ThreadPoolExecutor
    pairs = [(b, g) for b in range(len(lens)) for g in range(4)]
    with ThreadPoolExecutor(4) as ex:
        for (b, g), want in zip(pairs, ex.map(oracle_head, pairs)):
            assert_close(got[b, 6 * g:6 * g + 6], want, what=f"k8v4 sequence {b} ({lens[b]} tokens), KV head {g}")


def test_combine_over_more_than_1024_splits(gpu):
    """262,400 q4_0 tokens at one page per split: 1,025 splits, so the merge runs over two
    chunks of split weights. One KV head against the oracle; the one-call decode bitwise
    equal to the split and combine called as two phases."""
    fmt, cfg, g, T = "q4_0", 3, 2, 262400
    q = kvsynth.q_np(cfg, 2, 1)
    s, pool, bt, heads = build_pool(gpu, fmt, cfg, [T], seed=47, g=g)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    btd, ctx, qd = dev(bt), dev(np.array([T], np.int32)), dev(q)
    outs = []
    for phases in (("all",), ("split", "combine")):
        ws = K.paged.DecodeWorkspace(s, 1, T, 1, device=gpu)
        out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
        for ph in phases:
            K.decode_attention(s, qd, pool.data, btd, ctx, T, out, ws.data, pages_per_split=1, phase=ph)
        torch.cuda.synchronize()
        assert ws.status() == 0
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    want = head_oracle(q[0, 6 * g:6 * g + 6], head_records(*heads[0], fmt), fmt)
    assert_close(outs[0][0, 6 * g:6 * g + 6], want, what="q4_0 262,400 tokens at 1,025 splits")
