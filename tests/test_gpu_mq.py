"""GPU parity of causal multi-query attention (kv_decode_attention_mq) against the
oracle's multi_query_attention, and its agreement with decode attention over each
query's prefix (the same split size; the two kernels sum the softmax weights in a
different order, so they agree to fp32 rounding)."""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K
from oracle import attention

from gpu_helpers import Sequence, assert_close, fmt_id, oracle_records, place_pages

pytestmark = pytest.mark.gpu

FMTS = ["int8", "q4_0", "k8v4", "fp4", "fp8"]


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def pool_of(gpu, fmt, seqs, seed):
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    n_pool = sum(x.n_pages for x in seqs) + 3
    pool_np, bt = place_pages(seqs, n_pool, seed, pb)
    return s, to_dev(pool_np, gpu), to_dev(bt, gpu)


def run_mq(gpu, fmt, seqs, q, pps=0, seed=0):
    """q [B, n_q, 24, 256] fp16 -> out [B, n_q, 24, 256], status."""
    s, pool, bt = pool_of(gpu, fmt, seqs, seed)
    B, n_q = q.shape[:2]
    lens = np.array([x.T for x in seqs], np.int32)
    max_ctx = int(max(lens.max(), 1))
    ws = K.paged.DecodeWorkspace(s, B, max_ctx, pps, device=gpu, n_q=n_q)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=gpu)
    K.decode_attention_mq(s, to_dev(q, gpu), pool, bt, to_dev(lens, gpu), max_ctx, out, ws.data,
                          pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws.status()


def oracle_mq(q, seqs, fmt):
    outs = []
    for b, s in enumerate(seqs):
        if s.T == 0:
            outs.append(np.zeros(q.shape[1:]))
            continue
        kh, vh = s.hat()
        outs.append(attention.multi_query_attention(q[b], kh, vh, fmt_id(fmt)))
    return np.stack(outs)


CASES = [
    ("one_query", [700], 1, 0), ("drafts4", [1000], 4, 0), ("drafts4_pps1", [1000], 4, 1),
    ("T_eq_nq", [3], 3, 0), ("T_lt_nq", [2], 5, 0), ("page_edge", [257], 2, 0),
    ("eight", [3000], 8, 0), ("batch_ragged", [4096, 257, 0, 700], 3, 2),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name, lens, n_q, pps", CASES, ids=[c[0] for c in CASES])
def test_mq_matches_oracle(gpu, fmt, name, lens, n_q, pps):
    seqs = [Sequence(61, 0, b, T, fmt) for b, T in enumerate(lens)]
    q = kvsynth.q_np(61, 0, len(lens) * n_q).reshape(len(lens), n_q, 24, 256)
    got, status = run_mq(gpu, fmt, seqs, q, pps, seed=n_q)
    assert status == 0
    want = oracle_mq(q, seqs, fmt)
    assert_close(got, want, what=f"{fmt} {name}")
    for b, T in enumerate(lens):  # queries without context: exactly zero
        for j in range(n_q):
            if T - n_q + j + 1 <= 0:
                assert np.array_equal(got[b, j], np.zeros_like(got[b, j]))


@pytest.mark.parametrize("fmt", FMTS)
def test_mq_rows_equal_decode_over_each_prefix(gpu, fmt):
    """Row j is kv_decode_attention with context T - n_q + j + 1 (same split size), to fp32
    rounding of the summation order."""
    T, n_q, pps = 2500, 5, 2
    seqs = [Sequence(62, 0, 0, T, fmt)]
    q = kvsynth.q_np(62, 0, n_q).reshape(1, n_q, 24, 256)
    got, _ = run_mq(gpu, fmt, seqs, q, pps, seed=5)
    s, pool, bt = pool_of(gpu, fmt, seqs, 5)
    for j in range(n_q):
        ctx = T - n_q + j + 1
        ws = K.paged.DecodeWorkspace(s, 1, T, pps, device=gpu)
        out = torch.empty((1, 24, 256), dtype=torch.float32, device=gpu)
        K.decode_attention(s, to_dev(q[:, j], gpu), pool, bt, torch.tensor([ctx], dtype=torch.int32, device=gpu),
                           T, out, ws.data, pages_per_split=pps)
        torch.cuda.synchronize()
        ref = out.cpu().numpy()[0]
        assert np.max(np.abs(ref - got[0, j])) <= 1e-5 * max(1.0, float(np.max(np.abs(ref)))), j


@pytest.mark.parametrize("fmt", FMTS)
def test_chunked_prefill_end_to_end(gpu, fmt):
    """A prompt read in chunks: append each chunk, then its causal attention, against the
    oracle over the raw inputs' records."""
    T0, chunks = 300, [37, 256, 5]
    T = T0 + sum(chunks)
    k, v = kvsynth.kv_tokens_np(63, 0, 0, 0, T)
    s = K.shape(fmt)
    n_pages = -(-T // 256)
    pool = K.paged.PagedPool(fmt, n_pages + 2, device=gpu)
    bt = torch.tensor(list(range(n_pages + 1, 0, -1))[:n_pages], dtype=torch.int32, device=gpu)
    kd, vd = to_dev(k, gpu), to_dev(v, gpu)
    pool.append(kd[:T0].contiguous(), vd[:T0].contiguous(), 0, bt)
    kc, ks, vc, vs = oracle_records(k, v, fmt)
    seq = Sequence(63, 0, 0, T, fmt, k=k, v=v)
    kh, vh = seq.hat()
    t = T0
    for n in chunks:
        pool.append(kd[t:t + n].contiguous(), vd[t:t + n].contiguous(), t, bt)
        t += n
        q = kvsynth.q_np(63, t, n).reshape(1, n, 24, 256)
        ws = K.paged.DecodeWorkspace(s, 1, t, device=gpu, n_q=n)
        out = torch.empty((1, n, 24, 256), dtype=torch.float32, device=gpu)
        K.decode_attention_mq(s, to_dev(q, gpu), pool.data, bt[None].contiguous(),
                              torch.tensor([t], dtype=torch.int32, device=gpu), t, out, ws.data)
        torch.cuda.synchronize()
        want = attention.multi_query_attention(q[0], kh[:t], vh[:t], fmt_id(fmt))
        assert_close(out.cpu().numpy()[0], want, what=f"{fmt} chunk ending at {t}")
        assert ws.status() == 0


def test_mq_argument_checks(gpu):
    s = K.shape("q4_0")
    pool = torch.zeros(K.page_bytes(s), dtype=torch.uint8, device=gpu)
    q = torch.zeros((1, 0, 24, 256), dtype=torch.float16, device=gpu)
    ws = K.paged.DecodeWorkspace(s, 1, 256, device=gpu)
    with pytest.raises(K.KVError):
        K.decode_attention_mq(s, q, pool, torch.zeros((1, 1), dtype=torch.int32, device=gpu),
                              torch.tensor([1], dtype=torch.int32, device=gpu), 256,
                              torch.zeros((1, 0, 24, 256), dtype=torch.float32, device=gpu), ws.data)
    q = torch.zeros((1, 4, 24, 256), dtype=torch.float16, device=gpu)
    assert K.decode_mq_workspace_bytes(s, 1, 4, 256) > ws.nbytes
    with pytest.raises(K.KVError):  # a workspace sized for one query is too small for four
        K.decode_attention_mq(s, q, pool, torch.zeros((1, 1), dtype=torch.int32, device=gpu),
                              torch.tensor([4], dtype=torch.int32, device=gpu), 256,
                              torch.zeros((1, 4, 24, 256), dtype=torch.float32, device=gpu), ws.data)


@pytest.mark.parametrize("fmt", FMTS)
def test_many_groups_repeatable(gpu, fmt):
    """A 130-token chunk: 65 query groups per KV head, more workgroups than fit at once.
    Three calls give the same bits, within tolerance of the oracle."""
    T, n = 593, 130
    k, v = kvsynth.kv_tokens_np(64, 0, 0, 0, T)
    s = K.shape(fmt)
    pool = K.paged.PagedPool(fmt, 5, device=gpu)
    bt = torch.tensor([4, 3, 2], dtype=torch.int32, device=gpu)
    pool.append(to_dev(k, gpu), to_dev(v, gpu), 0, bt)
    kh, vh = Sequence(64, 0, 0, T, fmt, k=k, v=v).hat()
    q = kvsynth.q_np(64, 1, n).reshape(1, n, 24, 256)
    want = attention.multi_query_attention(q[0], kh, vh, fmt_id(fmt))
    runs = []
    for _ in range(3):
        ws = K.paged.DecodeWorkspace(s, 1, T, device=gpu, n_q=n)
        out = torch.full((1, n, 24, 256), float("nan"), dtype=torch.float32, device=gpu)
        K.decode_attention_mq(s, to_dev(q, gpu), pool.data, bt[None].contiguous(),
                              torch.tensor([T], dtype=torch.int32, device=gpu), T, out, ws.data)
        torch.cuda.synchronize()
        runs.append(out.cpu().numpy()[0])
        assert ws.status() == 0
    assert_close(runs[0], want, what=f"{fmt} 130 queries")
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])
