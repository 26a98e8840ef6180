"""CPU tests of the HIP library: it loads, exports every declared symbol, and its
host-side logic (rounding, record rules, CLOCK table, argument checks) matches
the oracle. No GPU work is launched here."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import offloaded_kv_cache_amd as K
from offloaded_kv_cache_amd import _native as N
from oracle import layout, records
from oracle.residency import ClockTable

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvcache.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(N.lib, n), n
    assert set(names) == set(N.EXPORTED_SYMBOLS)


def test_version_and_page_bytes():
    assert re.match(r"\d+\.\d+\.\d+", K.version())
    assert K.page_bytes(K.shape("int8")) == 540672
    assert K.page_bytes(K.shape("q4_0")) == 294912
    assert K.page_bytes(K.shape("k8v4")) == 417792
    assert K.page_bytes(K.shape("fp4")) == 294912
    assert K.page_bytes(K.shape("fp8")) == 528384
    # the library's page size equals the oracle layout's for every format
    for name, fmt in records.FORMATS.items():
        assert K.page_bytes(K.shape(name)) == layout.page_bytes(fmt, 4), name


@pytest.mark.parametrize("bad, code", [
    (dict(head_dim=128), N.KV_EUNSUPPORTED),
    (dict(page_tokens=128), N.KV_EUNSUPPORTED),
    (dict(n_q_heads=25), N.KV_EINVAL),
    (dict(n_q_heads=40, n_kv_heads=4), N.KV_EUNSUPPORTED),
])
def test_shape_validation(bad, code):
    args = dict(n_q_heads=24, n_kv_heads=4, head_dim=256, page_tokens=256)
    args.update(bad)
    s = N.KVShape(args["n_q_heads"], args["n_kv_heads"], args["head_dim"], args["page_tokens"], 1)
    assert N.lib.kv_page_bytes(C.byref(s)) == code
    assert N.last_error()
    s.format = 5                       # one past the last format
    s.head_dim, s.page_tokens, s.n_q_heads, s.n_kv_heads = 256, 256, 24, 4
    assert N.lib.kv_page_bytes(C.byref(s)) == N.KV_EINVAL


def test_f64_to_f16_matches_single_rounding():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12),
         1 + 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -30, 1 + 3 * 2.0 ** -11, np.inf, -np.inf],
    ])
    want = records.fp16_rne(vals).view(np.uint16)
    got = np.array([N.host_f64_to_f16(v) for v in vals], np.uint16)
    assert np.array_equal(got, want)
    assert N.host_f64_to_f16(np.nan) & 0x7C00 == 0x7C00


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_host_records_match_oracle(kind):
    rng = np.random.default_rng(10 + kind)
    xs = [(rng.standard_normal(256) * np.where(rng.random(256) < 0.03, 20, 1)).astype(np.float16)
          for _ in range(150)]
    z = np.zeros(256, np.float16)
    xs.append(z)
    t = np.zeros(256, np.float16)
    t[0] = 127 / 16
    t[1:5] = [2.5 / 16, -2.5 / 16, 0.5 / 16, -0.5 / 16]
    xs.append(t)
    xs.append(np.full(256, np.float16(2.0 ** -24)))
    for x in xs:
        codes, scales = N.host_encode_vector(kind, x)
        if kind == 0:
            c, d = records.quantize_int8(x.astype(np.float64))
            assert np.array_equal(codes.view(np.int8), c)
        elif kind == 1:
            c, d = records.quantize_q4(x.astype(np.float64))
            assert np.array_equal(codes, c)
        elif kind == 2:
            c, d = records.quantize_fp4(x.astype(np.float64))
            assert np.array_equal(codes, c)
        else:
            c, d = records.quantize_fp8(x.astype(np.float64))
            d = d.reshape(-1)
            assert np.array_equal(codes, c)
        assert np.array_equal(scales.view(np.uint16), d.view(np.uint16))


def test_clock_matches_oracle_on_random_traces():
    rng = np.random.default_rng(3)
    for n_slots, n_pages in ((4, 10), (16, 300), (128, 4096)):
        a, b = K.Residency(n_slots, n_pages), ClockTable(n_slots, n_pages)
        for _ in range(200):
            sel = rng.choice(n_pages, int(rng.integers(0, n_slots + 1)), replace=False)
            sa, ca = a.select(sel)
            sb, cb = b.select(sel)
            assert list(sa) == list(sb) and ca == cb
            assert a.hand == b.hand
            assert list(a.slot_page) == b.slot_page and list(a.ref) == b.ref


def test_clock_errors_leave_table_unchanged():
    t = K.Residency(4, 10)
    t.select([0, 1, 2])
    snap = (t.slot_page.copy(), t.page_slot.copy(), t.ref.copy(), t.hand)
    for sel, code in (([0, 1, 2, 3, 4], N.KV_ENOSLOTS), ([1, 1], N.KV_EINVAL), ([10], N.KV_EINVAL),
                      ([-1], N.KV_EINVAL)):
        with pytest.raises(K.KVError) as e:
            t.select(sel)
        assert e.value.code == code
        assert np.array_equal(t.slot_page, snap[0]) and np.array_equal(t.page_slot, snap[1])
        assert np.array_equal(t.ref, snap[2]) and t.hand == snap[3]


def test_abi_argument_errors_enqueue_nothing():
    s = K.shape("q4_0")
    P = C.c_void_p
    # NULL buffers are refused before any HIP call
    r = N.lib.kv_decode_attention(C.byref(s), None, 1, None, 1, None, 1, None, 4096, 0.0625, None,
                                  None, 0, 0, None)
    assert r == N.KV_EINVAL
    r = N.lib.kv_append_quantize(C.byref(s), None, None, 1, 0, None, 1, None, 1, None, None)
    assert r == N.KV_EINVAL
    # zero tokens / zero batch are no-ops
    assert N.lib.kv_append_quantize(C.byref(s), None, None, 0, 0, None, 0, None, 0, None, None) == 0
    assert N.lib.kv_decode_attention(C.byref(s), None, 0, None, 0, None, 0, None, 0, 0.0625, None,
                                     None, 0, 0, None) == 0
    # a token range past the block table
    r = N.lib.kv_append_quantize(C.byref(s), P(16), P(16), 300, 0, P(16), 1, P(256), 4, None, None)
    assert r == N.KV_EINVAL and "do not fit" in N.last_error()
    # a start position so large that start_pos + n_tokens would wrap past INT64_MAX (a wrapped
    # sum would pass the range check and send the kernel far outside the block table)
    big = (1 << 63) - 1
    for n in (1, 2, 300):
        r = N.lib.kv_append_quantize(C.byref(s), P(16), P(16), n, big, P(16), 1, P(256), 4, None, None)
        assert r == N.KV_EINVAL and "overflows" in N.last_error()
        r = N.lib.kv_page_key_sums(C.byref(s), P(16), n, big, P(256), P(256), 1 << 40, None)
        assert r == N.KV_EINVAL and "overflows" in N.last_error()
    r = N.lib.kv_append_quantize(C.byref(s), P(16), P(16), 1, big - 1, P(16), 1, P(256), 4, None, None)
    assert r == N.KV_EINVAL and "do not fit" in N.last_error()
    r = N.lib.kv_page_key_sums(C.byref(s), P(16), 300, 256 * 4 - 299, P(256), P(256), 4, None)
    assert r == N.KV_EINVAL and "pages of sums" in N.last_error()
    # misaligned pool
    r = N.lib.kv_append_quantize(C.byref(s), P(16), P(16), 10, 0, P(16), 1, P(258), 4, None, None)
    assert r == N.KV_EALIGN
    # workspace too small
    need = K.decode_workspace_bytes(s, 1, 4096)
    r = N.lib.kv_decode_attention(C.byref(s), P(256), 1, P(256), 16, P(256), 16, P(256), 4096, 0.0625,
                                  P(256), P(256), need - 1, 0, None)
    assert r == N.KV_ESMALL
    # the timed multi-layer gather: nothing to do records nothing and succeeds; its
    # arguments are checked as the untimed call's are
    t1 = K.Residency(4, 10)
    tabs = (N.KVResidency * 1)(t1.c)
    one = np.array([1], np.int32)
    r = N.lib.kv_gather_pages_layers_timed(C.byref(s), 1, tabs, one.ctypes.data_as(P), 0, None, None,
                                           None, None, None, None, None)
    assert r == 0
    r = N.lib.kv_gather_pages_layers_timed(C.byref(s), 1, tabs, one.ctypes.data_as(P), 1, None, None,
                                           P(256), None, None, None, None)
    assert r == N.KV_EINVAL and t1.slot_page.tolist() == [-1] * 4
    # a gather selection larger than the slot pool
    t = K.Residency(2, 10)
    sel = np.array([1, 2, 3], np.int32)
    r = N.lib.kv_gather_pages(C.byref(s), C.byref(t.c), sel.ctypes.data_as(P), 3, P(256), P(256),
                              P(256), None, None)
    assert r == N.KV_ENOSLOTS


def test_workspace_grows_with_context_and_split():
    s = K.shape("q4_0")
    a = K.decode_workspace_bytes(s, 1, 4096, 4)
    b = K.decode_workspace_bytes(s, 1, 131072, 4)
    c = K.decode_workspace_bytes(s, 1, 131072, 1)
    assert a < b < c
    # status word + per-split (m, l) + 256 outputs, for 24 heads
    assert b >= 256 + 24 * 128 * (2 + 256) * 4


def test_split_pages_fill_the_gpu_once():
    q4, k8 = K.shape("q4_0"), K.shape("k8v4")
    # 128K tokens, one sequence, 4-bit K: 512 workgroups of 4 waves -> 4 pages each
    assert K.decode_split_pages(q4, 1, 131072) == 4
    # int8 K runs 8-wave workgroups, one per CU: twice the pages per split
    assert K.decode_split_pages(k8, 1, 131072) == 8
    # four sequences of unequal length: sized by their total, not 4 x the longest
    lens = [262144, 198000, 65536, 8192]
    by_total = K.decode_split_pages(k8, 4, max(lens), sum(lens))
    assert by_total < K.decode_split_pages(k8, 4, max(lens))
    # one grid round: the workgroups that have pages fit on the 256 CUs
    assert sum(-(-(-(-T // 256)) // by_total) for T in lens) * 4 <= 256
    assert K.decode_split_pages(q4, 1, 1) == 1
    with pytest.raises(K.KVError):
        K.decode_split_pages(q4, 2, 100, 201)   # total above batch x max


def test_binding_shares_torchs_hip_runtime():
    """Importing the package before torch still maps a single HIP runtime: two runtimes in
    one process leave the library's launches without the device torch holds."""
    import subprocess
    import sys
    code = ("import offloaded_kv_cache_amd, torch\n"
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_host_fp8_codes_at_every_tie():
    """The library's E4M3 rounding (shared by its kernels) at every midpoint between
    neighbouring magnitudes, just beside each, with both signs, and with a subnormal
    scale that saturates, against the oracle."""
    mids = (records.E4M3[1:] + records.E4M3[:-1]) / 2
    for top in (448.0, 896.0):
        for nudge in (0.0, -1.0, 1.0):
            x = np.zeros(256)
            x[0] = top
            v = mids * (top / 448.0)
            if nudge:
                v = np.nextafter(v.astype(np.float16), np.float16(nudge * np.inf)).astype(np.float64)
            x[1:127] = v
            x[127:253] = -v
            x16 = x.astype(np.float16)
            codes, scales = N.host_encode_vector(3, x16)
            c, d = records.quantize_fp8(x16.astype(np.float64))
            assert np.array_equal(codes, c), (top, nudge)
            assert scales.view(np.uint16)[0] == d.view(np.uint16)[0]
    x = np.zeros(256, np.float16)
    x[0], x[1] = np.float16(627 * 2.0 ** -24), np.float16(-300 * 2.0 ** -24)
    codes, scales = N.host_encode_vector(3, x)
    assert float(scales[0]) == 2.0 ** -24 and codes[0] == 0x7E      # 627 saturates
    assert codes[1] == 0x80 | 0x79                                    # 300 -> 288 = 1.125 * 2^8
    assert np.array_equal(codes, records.quantize_fp8(x.astype(np.float64))[0])


def test_binding_refuses_host_buffers_before_any_launch():
    """A pool, workspace or slot pool in ordinary host memory is refused by the binding
    (ValueError) before the C ABI is called, so no kernel is ever handed a host address;
    a wrong dtype is a TypeError."""
    import torch

    host = torch.zeros(1024, dtype=torch.uint8)
    for name in ("pool", "workspace", "slot_pool"):
        with pytest.raises(ValueError, match="device memory"):
            N._buf(host, name)
    with pytest.raises(ValueError, match="pinned host memory"):
        N._buf(host, "pool", pinned_ok=True)       # the append path also takes pinned memory
    with pytest.raises(TypeError):
        N._buf(torch.zeros(16, dtype=torch.float32), "workspace")
    with pytest.raises(ValueError, match="contiguous"):
        N._buf(torch.zeros((8, 8), dtype=torch.uint8).t(), "pool")
    # whole calls with host tensors stop in the binding as well
    s = K.shape("q4_0")
    q = torch.zeros((1, 24, 256), dtype=torch.float16)
    out = torch.zeros((1, 24, 256), dtype=torch.float32)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    ctx = torch.ones(1, dtype=torch.int32)
    pool = torch.zeros(K.page_bytes(s), dtype=torch.uint8)
    ws = torch.zeros(K.decode_workspace_bytes(s, 1, 256), dtype=torch.uint8)
    with pytest.raises(ValueError):
        K.decode_attention(s, q, pool, bt, ctx, 256, out, ws)
    with pytest.raises(ValueError):
        K.append_decode(s, torch.zeros((1, 4, 256), dtype=torch.float16),
                        torch.zeros((1, 4, 256), dtype=torch.float16), q, pool, bt, ctx, 256, out, ws)


def test_noalloc_refuses_what_its_array_cannot_hold():
    """kv_decode_attention_noalloc checks its arguments and the size of the partials before
    it touches the device: beyond KV_NOALLOC_SCRATCH_BYTES it returns KV_ESMALL."""
    s = K.shape("q4_0")
    P = C.c_void_p
    lib = N.lib
    assert N.NOALLOC_SCRATCH_BYTES == 16 << 20
    r = lib.kv_decode_attention_noalloc(C.byref(s), None, 1, None, 1, None, 1, None, 4096, 0.0625, None,
                                        None, 0, None)
    assert r == N.KV_EINVAL
    r = lib.kv_decode_attention_noalloc(C.byref(s), P(256), 1, P(256), 16, P(256), 16, P(256), 4096, 0.0625,
                                        P(256), P(258), 0, None)
    assert r == N.KV_EALIGN                          # a misaligned status word
    # the largest context that fits at one page per split, then one page (one split) more
    ctx = 256
    while K.decode_workspace_bytes(s, 1, ctx + 256, 1) <= N.NOALLOC_SCRATCH_BYTES:
        ctx += 256
    assert K.decode_workspace_bytes(s, 1, ctx, 1) <= N.NOALLOC_SCRATCH_BYTES
    r = lib.kv_decode_attention_noalloc(C.byref(s), P(256), 1, P(256), 4096, P(256), 4096, P(256), ctx + 256,
                                        0.0625, P(256), None, 1, None)
    assert r == N.KV_ESMALL and "scratch" in N.last_error()
    # a batch far beyond the array at the library's own split size
    r = lib.kv_decode_attention_noalloc(C.byref(s), P(256), 4096, P(256), 4096, P(256), 4096, P(256), 1 << 20,
                                        0.0625, P(256), None, 0, None)
    assert r == N.KV_ESMALL


def test_measurement_library_loads_and_rejects_bad_arguments():
    """lib/libkvmeasure.so (the benchmark's plain read of a decode launch's pages) exports its
    one entry point, which rejects arguments outside its limits before any launch (host only)."""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "offloaded_kv_cache_amd", "lib", "libkvmeasure.so")
    if not os.path.exists(path):
        pytest.skip("measurement library not built")
    fn = C.CDLL(path).kv_measure_read_pages
    fn.restype = C.c_int
    fn.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int,
                   C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    dummy = C.c_void_p(16)  # never dereferenced: every call below is rejected first
    ok = dict(pool=dummy, n=8, hb=73728, nkv=4, bt=dummy, mp=8, ctx=dummy, b=1, pps=2, ns=4, th=256, nr=0, out=dummy)
    def call(**kw):
        a = dict(ok, **kw)
        return fn(a["pool"], a["n"], a["hb"], a["nkv"], a["bt"], a["mp"], a["ctx"], a["b"], a["pps"], a["ns"],
                  a["th"], a["nr"], None, a["out"], None, None, None)
    for bad in (dict(pool=None), dict(bt=None), dict(ctx=None), dict(out=None), dict(hb=0), dict(hb=73720),
                dict(hb=147456 + 16), dict(nkv=0), dict(b=0), dict(mp=0), dict(pps=0), dict(ns=0), dict(n=0),
                dict(nr=-1), dict(th=128), dict(th=1024)):
        assert call(**bad) == -1, bad
