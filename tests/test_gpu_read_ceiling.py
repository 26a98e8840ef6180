"""GPU test of the benchmark's plain page read (lib/libkvmeasure.so, kv_measure_read_pages).

The read is the split kernel's roofline reference, so it must read exactly the bytes a
decode launch reads: for every work item (split, sequence, KV head) of the split-major
grid, the KV-head part of each of the item's pages (context rounded up to pages, pages
with an id outside the pool skipped). Its per-thread checksums (the xor of the 16-byte
words j * T + thread of each page part (T threads a workgroup), folded to one word) are compared with the same
checksums computed on the host from the pool's bytes; a word read twice or missed, a page
taken from the wrong table entry or KV head, or a wrong item order changes them.
"""

import ctypes as C
import os

import numpy as np
import pytest
import torch

import offloaded_kv_cache_amd as K

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "offloaded_kv_cache_amd", "lib", "libkvmeasure.so")


def _fn():
    fn = C.CDLL(LIB).kv_measure_read_pages
    fn.restype = C.c_int
    fn.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int,
                   C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    return fn


def expected(pool, head_bytes, n_kv, bt, lens, pps, n_splits, threads):
    n_u4 = head_bytes // 16
    per = -(-n_u4 // threads)
    B = len(lens)
    out = np.zeros((n_splits * B * n_kv, threads), np.uint32)
    words = pool.view(np.uint32).reshape(-1, n_kv, n_u4, 4)  # [page][head][word][dword]
    pad = np.zeros((per * threads - n_u4, 4), np.uint32)
    for item in range(n_splits * B * n_kv):
        split, rem = divmod(item, B * n_kv)
        b, g = divmod(rem, n_kv)
        n_pages = min(-(-max(int(lens[b]), 0) // 256), bt.shape[1])
        acc = np.zeros((threads, 4), np.uint32)
        for pg in range(split * pps, min(n_pages, split * pps + pps)):
            phys = int(bt[b, pg])
            if phys < 0 or phys >= words.shape[0]:
                continue
            w = np.concatenate([words[phys, g], pad]).reshape(per, threads, 4)  # word j * threads + t
            acc ^= np.bitwise_xor.reduce(w, axis=0)
        out[item] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return out


@pytest.mark.parametrize("fmt", ["q4_0", "int8", "k8v4", "fp8"])
@pytest.mark.parametrize("n_resident", [0, 7])
@pytest.mark.parametrize("threads", [256, 512])
def test_read_pages_reads_exactly_the_launch_bytes(gpu, fmt, n_resident, threads):
    if not os.path.exists(LIB):
        pytest.fail("lib/libkvmeasure.so is not built (offloaded_kv_cache_amd/build.py builds it)")
    s = K.shape(fmt)
    n_kv = 4
    page_bytes = K.page_bytes(s)
    head_bytes = page_bytes // n_kv
    rng = np.random.default_rng(5)
    n_pool = 23
    pool = rng.integers(0, 256, n_pool * page_bytes, dtype=np.uint8)
    lens = np.array([2000, 513, 0, 256 * 12], np.int32)  # ragged, empty, longer than the table row
    max_pages = 10
    bt = rng.integers(0, n_pool, (4, max_pages)).astype(np.int32)  # (sequences may share pages)
    bt[0, 3] = -1          # a bad page id inside the context: skipped
    bt[1, 1] = n_pool + 5  # another, past the pool
    pps = 3
    n_splits = -(-max_pages // pps)
    dev_pool = torch.from_numpy(pool).to(gpu)
    dev_bt = torch.from_numpy(bt).to(gpu)
    dev_lens = torch.from_numpy(lens).to(gpu)
    stream = torch.cuda.current_stream()
    counter = torch.zeros(2, dtype=torch.int32, device=gpu)
    want = expected(pool, head_bytes, n_kv, bt, lens, pps, n_splits, threads)
    # n_resident 7: 64 items through 7 workgroups and the counter, twice on one counter
    for _ in range(2):
        out = torch.full((n_splits * 4 * n_kv * threads,), -1, dtype=torch.int32, device=gpu)
        r = _fn()(dev_pool.data_ptr(), n_pool, head_bytes, n_kv, dev_bt.data_ptr(), max_pages, dev_lens.data_ptr(),
                  4, pps, n_splits, threads, n_resident, counter.data_ptr(), out.data_ptr(), C.c_void_p(stream.cuda_stream),
                  None, None)
        assert r == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32).reshape(-1, threads)
        assert np.array_equal(got, want)
        assert counter.cpu().tolist() == [0, 0]  # left at zero for the next launch
