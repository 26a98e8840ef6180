"""GPU page selection (kv_page_key_sums, kv_select_pages) against the oracle's
declared rule (oracle/selection.py): key sums, page representatives and selections
bit for bit."""

import numpy as np
import pytest
import torch

import kvsynth
import offloaded_kv_cache_amd as K
from oracle import selection as osel

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_sums(gpu, s, k, chunks, cap):
    """Key sums and representatives of keys k appended in the given chunks."""
    sums = torch.zeros((cap, s.n_kv_heads, 256), dtype=torch.int64, device=gpu)
    reps = torch.zeros((cap, s.n_kv_heads, 256), dtype=torch.float16, device=gpu)
    kd = to_dev(k, gpu)
    t = 0
    for n in chunks:
        K.page_key_sums(s, kd[t:t + n].contiguous(), t, sums, reps)
        t += n
    assert t == k.shape[0]
    return sums, reps


def bits(x):
    return x.cpu().numpy().view(np.uint16)


def gpu_select(gpu, s, q, reps, n_pages, k_sel):
    ws = torch.empty(K.select_workspace_bytes(n_pages), dtype=torch.uint8, device=gpu)
    out = torch.full((k_sel,), -1, dtype=torch.int32, device=gpu)
    K.select_pages(s, to_dev(q, gpu), reps, n_pages, k_sel, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:min(k_sel, n_pages)].tolist()


@pytest.mark.parametrize("T, chunks", [(1, [1]), (700, [1, 17, 300, 382]), (4096, [4096]),
                                       (10000, [2048] * 4 + [1808])])
def test_key_sums_bitexact(gpu, T, chunks):
    s = K.shape("q4_0")
    k, _ = kvsynth.kv_tokens_np(41, 0, 0, 0, T)
    cap = -(-T // 256) + 2
    sums, reps = gpu_sums(gpu, s, k, chunks, cap)
    want = osel.key_sums(k, cap)
    assert np.array_equal(sums.cpu().numpy(), want)
    n = -(-T // 256)  # pages the calls touched; the spare ones keep their zeros
    assert np.array_equal(bits(reps)[:n], osel.key_reps(want[:n]).view(np.uint16))
    assert not bits(reps)[n:].any()


def test_representatives_round_once_at_ties_and_extremes(gpu):
    """Keys built so that page sums land on fp16 midpoints (ties to even), just off
    them, in the subnormal range, at zero from cancelling keys and at the top of the
    range."""
    s = K.shape("int8")
    rng = np.random.default_rng(9)
    k = np.zeros((256 * 6, 4, 256), np.float16)
    # page 0: 255 tokens of 2^-24 per element -> a sum / 2^32 below the least subnormal
    k[0:256, :, :] = np.float16(2.0 ** -24)
    k[0:1, :, :] = np.float16(0)
    # page 1: the sum of 256 copies of x is 256 x, so the representative is x exactly
    k[256:512] = rng.standard_normal((1, 4, 256)).astype(np.float16)
    # page 2: the sum is 255 x + y: a value between grid points, ties included for
    # y chosen as x plus or minus half an fp16 spacing of x
    x = rng.standard_normal((4, 256)).astype(np.float16)
    k[512:768] = x
    k[767] = (x.astype(np.float64) + np.spacing(x.astype(np.float16)).astype(np.float64) * 128).astype(np.float16)
    # page 3: cancelling keys (sum 0) and, in elements 0-63, the largest sum (rep 65504)
    k[768:1024:2] = np.float16(65504)
    k[769:1024:2] = np.float16(-65504)
    k[768:1024, :, :64] = np.float16(65504)
    # pages 4, 5: random keys with a large spread
    k[1024:] = (rng.standard_normal((512, 4, 256)) * np.exp2(rng.integers(-20, 12, (512, 4, 256)))).astype(np.float16)
    sums, reps = gpu_sums(gpu, s, k, [300, 700, k.shape[0] - 1000], 6)
    want = osel.key_sums(k)
    assert np.array_equal(sums.cpu().numpy(), want)
    assert np.array_equal(bits(reps), osel.key_reps(want).view(np.uint16))


@pytest.mark.parametrize("T", [256, 700, 8192, 65536 + 100])
@pytest.mark.parametrize("k_sel", [1, 3, 8, 32])
def test_selection_matches_oracle(gpu, T, k_sel):
    s = K.shape("int8")
    k, _ = kvsynth.kv_tokens_np(42, 0, 0, 0, T)
    n = -(-T // 256)
    sums, reps = gpu_sums(gpu, s, k, [T], n)
    for step in range(3):
        q = kvsynth.q_np(42, step, 1)[0]
        want = osel.select_pages(osel.page_scores(q, reps.cpu().numpy()), k_sel)
        assert want == osel.select(q, k, k_sel)
        assert gpu_select(gpu, s, q, reps, n, k_sel) == want, (T, k_sel, step)


def test_selection_ties_and_forced_last_page(gpu):
    """Pages with equal key sums: the lower page wins; the last page is always taken."""
    s = K.shape("q4_0")
    c = [1.0, 4.0, -2.0, 4.0, 3.0, 4.0, -8.0]
    k = np.zeros((256 * len(c), 4, 256), np.float16)
    for p, v in enumerate(c):
        k[256 * p:256 * p + 256, :, 0] = v
    q = np.zeros((24, 256), np.float16)
    q[:, 0] = 1.0
    _, reps = gpu_sums(gpu, s, k, [k.shape[0]], len(c))
    for k_sel in (1, 2, 3, 4, 7, 9):
        want = osel.select(q, k, k_sel)
        assert gpu_select(gpu, s, q, reps, len(c), k_sel) == want, k_sel
    assert osel.select(q, k, 3) == [1, 3, 6]


def test_selection_over_a_million_tokens(gpu):
    """4,096 pages (the streaming workload's host pool per layer), the 2,048-token budget."""
    s = K.shape("int8")
    T = 1 << 20
    gen = torch.Generator(device=gpu)
    gen.manual_seed(kvsynth.torch_seed(5, 0))
    gain = kvsynth.gain_torch(5, 0, 4, gpu)
    sums = torch.zeros((T // 256, 4, 256), dtype=torch.int64, device=gpu)
    reps = torch.zeros((T // 256, 4, 256), dtype=torch.float16, device=gpu)
    for t0 in range(0, T, 65536):
        kd, _ = kvsynth.kv_tokens_torch(gen, 65536, gain, gpu)
        K.page_key_sums(s, kd, t0, sums, reps)
    q = kvsynth.q_np(43, 0, 1)[0]
    got = gpu_select(gpu, s, q, reps, T // 256, 8)
    assert np.array_equal(bits(reps), osel.key_reps(sums.cpu().numpy()).view(np.uint16))
    want = osel.select_pages(osel.page_scores(q, reps.cpu().numpy()), 8)
    assert got == want and got[-1] == T // 256 - 1


def test_selection_of_several_sets_in_one_call(gpu):
    """Sixteen sets (layers) with their own queries and key sums in one call; sums with
    spare pages past the context."""
    s = K.shape("int8")
    L, T, k_sel = 16, 40 * 256 + 9, 8
    n = -(-T // 256)
    sums = torch.zeros((L, n + 3, 4, 256), dtype=torch.int64, device=gpu)
    reps = torch.zeros((L, n + 3, 4, 256), dtype=torch.float16, device=gpu)
    keys = []
    for layer in range(L):
        k, _ = kvsynth.kv_tokens_np(44, layer, 0, 0, T)
        keys.append(k)
        K.page_key_sums(s, to_dev(k, gpu), 0, sums[layer], reps[layer])
    q = kvsynth.q_np(44, 0, L)
    ws = torch.empty(K.select_workspace_bytes(n, L), dtype=torch.uint8, device=gpu)
    out = torch.full((L, k_sel), -1, dtype=torch.int32, device=gpu)
    K.select_pages(s, to_dev(q, gpu), reps, n, k_sel, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for layer in range(L):
        assert got[layer].tolist() == osel.select(q[layer], keys[layer], k_sel), layer
