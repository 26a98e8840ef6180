"""Parity at full benchmark sizes, in the launch configuration the benchmark uses.

* One layer of 131,072 tokens in q4_0 (24 query / 4 KV heads), and the same in
  fp4 and fp8, and one layer of 32,768 int8 tokens: the cache is written by the
  append kernel in 2,048-token chunks through a shuffled block table, decoded
  with the automatic split count; one KV head's six query heads are checked
  against the fp64 oracle, and sampled pages of that head are checked byte for
  byte against the oracle's records.
* Four k8v4 sequences of 262,144 / 198,000 / 65,536 / 8,192 tokens in one
  shuffled pool (the 198,000-token one ends in a 112-token page): one KV head
  of every sequence is checked against the oracle.

K and V are drawn on the GPU (seeded, the benchmark's distribution) and appended
chunk by chunk; the checked head's fp16 K and V are copied back and the oracle
encodes only that head (its cost is the rotation of every vector of that head).
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


def build_pool(gpu, fmt, cfg, lens, seed, g):
    """Draw each sequence's K, V on the GPU in CHUNK-token pieces, append them into one
    pool with a shuffled block table, and return head g's fp16 K and V per sequence."""
    s = K.shape(fmt)
    pages = [-(-T // 256) for T in lens]
    n_pool = sum(pages)
    perm = kvsynth.permutation_np(seed, n_pool)
    pool = K.paged.PagedPool(fmt, n_pool, device=gpu)
    bt = np.zeros((len(lens), max(pages)), np.int32)
    gain = kvsynth.gain_torch(cfg, 0, s.n_kv_heads, gpu)
    heads = []
    off = 0
    for b, (T, n) in enumerate(zip(lens, pages)):
        bt[b, :n] = perm[off:off + n]
        off += n
        row = torch.from_numpy(bt[b]).to(gpu)
        gen = torch.Generator(device=gpu)
        gen.manual_seed(kvsynth.torch_seed(cfg, 0, b))
        kh, vh = [], []
        for t0 in range(0, T, CHUNK):
            kd, vd = kvsynth.kv_tokens_torch(gen, min(CHUNK, T - t0), gain, gpu)
            pool.append(kd, vd, t0, row)
            kh.append(kd[:, g:g + 1].cpu().numpy())
            vh.append(vd[:, g:g + 1].cpu().numpy())
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


LAYERS = [("q4_0", 131072, 3), ("fp4", 131072, 3), ("fp8", 131072, 3), ("int8", 32768, 2)]


@pytest.mark.parametrize("fmt, T, cfg", LAYERS, ids=[f"{f}_{t}" for f, t, _ in LAYERS])
def test_one_layer_sampled(gpu, fmt, T, cfg):
    g = 1
    q = kvsynth.q_np(cfg, 0, 1)
    s, pool, bt, heads = build_pool(gpu, fmt, cfg, [T], seed=31, g=g)
    got = decode(gpu, s, pool, bt, q, [T])
    rec = head_records(*heads[0], fmt)
    want = head_oracle(q[0, 6 * g:6 * g + 6], rec, fmt)
    assert_close(got[0, 6 * g:6 * g + 6], want, what=f"{fmt} {T}, KV head 1")
    # sampled pages of the checked head, byte for byte
    one_head = layout.pack_pages(*rec, fmt_id(fmt))      # pages of a 1-KV-head layout
    hs = one_head.shape[1]                                # bytes of one head's K + V planes
    pb = K.page_bytes(s)
    for p in (0, 1, T // 512, T // 256 - 1):
        phys = int(bt[0, p])
        dev = pool.data[phys * pb + g * hs: phys * pb + (g + 1) * hs].cpu().numpy()
        assert np.array_equal(dev, one_head[p]), f"page {p}"


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
