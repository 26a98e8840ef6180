#!/usr/bin/env python3
"""Decode-step benchmark of the quantized, paged KV cache on one MI355X.

Default workload (the headline metric, "KV GB/s streamed in decode attention
(% of 8 TB/s HBM) at 128K q4_0"): 16 full-attention layers, 24 query / 4 KV
heads, head_dim 256, batch 1, q4_0 KV in 256-token pages, context growing to
131,072 tokens. One step = for every layer, quantize-on-append of the step's
new K/V token, then split-K decode attention (query rotation, Q.K, online
softmax, P.V, log-sum-exp combine, rotation back) over the whole context.

Inputs are synthetic (seeded; K, V ~ N(0,1) with 4 outlier channels x20 per
head, Q ~ N(0,1)), drawn on the GPU and resident in HBM before timing.

Prints one JSON line. `value` is algorithmic KV bytes read by attention per
second over the timed steps (wall time of the whole step, appends and
combines included). `roofline` is for the dominant kernel (the split-K
decode kernel): HIP events recorded at that kernel's own start and end on its
launch stream (kv_decode_split_timed), on every 4th layer of each timed step,
inside the timed region. `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same workload.

Other workloads (parity-test shapes, not the metric line): --workload c1
(1 layer, 4,096 tokens, q4_0), c2 (16 layers, 32,768, int8), c4 (16 layers,
4 sequences of 262,144 / 198,000 / 65,536 / 8,192 tokens, k8v4), c5
(16 layers, 1,048,576-token int8 host pool, 128 resident slots per layer,
2,048-token selection per step with ~30% misses, gathered zero-copy), c3fp4
(the default shape with fp4 records: e2m1 codes, power-of-two block scales), c3fp8
(the default shape with fp8 records: E4M3 codes, one scale per vector).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PAGE = 256

WORKLOADS = {
    "c1": dict(fmt="q4_0", layers=1, lens=[4096], cfg=1),
    # the same 4,096-token layer in 112 copies (528 MB, more than the 256 MB Infinity Cache),
    # attended in turn: every launch reads its pages from HBM
    "c1cold": dict(fmt="q4_0", layers=112, lens=[4096], cfg=1),
    "c2": dict(fmt="int8", layers=16, lens=[32768], cfg=2),
    "c3": dict(fmt="q4_0", layers=16, lens=[131072], cfg=3),
    # the headline shape at the top of the 128K-1M context range
    "c3m": dict(fmt="q4_0", layers=16, lens=[1048576], cfg=3),
    "c4": dict(fmt="k8v4", layers=16, lens=[262144, 198000, 65536, 8192], cfg=4, cpu_seq=2),
    "c3fp4": dict(fmt="fp4", layers=16, lens=[131072], cfg=3),
    "c3fp8": dict(fmt="fp8", layers=16, lens=[131072], cfg=3),
}

WORKLOAD_TEXT = {
    "c1": "1 layer, 4,096-token q4_0 context (warm: the layer's 4.7 MB stay in the Infinity Cache)",
    "c1cold": "112 copies of a 1-layer 4,096-token q4_0 context attended in turn (cold: 528 MB, read from HBM)",
    "c2": "16 layers, 32,768-token int8 context",
    "c3": "16 layers, 131,072-token q4_0 context (append 1 token + decode per layer)",
    "c3m": "16 layers, 1,048,576-token q4_0 context (append 1 token + decode per layer)",
    "c4": "16 layers, 4 sequences 262,144/198,000/65,536/8,192 tokens, k8v4",
    "c3fp4": "16 layers, 131,072-token fp4 context (append 1 token + decode per layer)",
    "c3fp8": "16 layers, 131,072-token fp8 context (append 1 token + decode per layer)",
}


def host_info():
    """The host the oracle runs on: CPU model, usable cores, BLAS library and its threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            blas = {"library": pools[0].get("internal_api"), "version": pools[0].get("version"),
                    "threads": max(i.get("num_threads", 1) for i in pools)}
    except Exception:
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "blas": blas}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_token(fmt: str, n_kv_heads: int = 4) -> int:
    rec = {"int8": (264, 264), "q4_0": (144, 144), "k8v4": (264, 144), "fp4": (144, 144), "fp8": (258, 258)}[fmt]
    return n_kv_heads * sum(rec)


def build_resident(args, wl, dev, per_step=1):
    import torch

    import kvsynth
    import offloaded_kv_cache_amd as K

    fmt, L, lens, cfg = wl["fmt"], wl["layers"], wl["lens"], wl["cfg"]
    B = len(lens)
    n_steps = args.warmup + args.steps
    end_lens = lens
    start_lens = [max(1, T - n_steps * per_step) for T in end_lens]
    pages_per_seq = [-(-T // PAGE) for T in end_lens]
    n_pool = sum(pages_per_seq)
    max_pages = max(pages_per_seq)
    s = K.shape(fmt)
    pools, tables = [], []
    append_ev = []
    chunk = 2048
    for layer in range(L):
        pool = K.paged.PagedPool(fmt, n_pool, device=dev)
        perm = torch.from_numpy(kvsynth.permutation_np(1000 * cfg + layer, n_pool)).to(dev)
        bt = torch.zeros((B, max_pages), dtype=torch.int32, device=dev)
        off = 0
        for b in range(B):
            bt[b, :pages_per_seq[b]] = perm[off:off + pages_per_seq[b]]
            off += pages_per_seq[b]
        gain = kvsynth.gain_torch(cfg, layer, 4, dev)
        for b in range(B):
            gen = torch.Generator(device=dev)
            gen.manual_seed(kvsynth.torch_seed(cfg, layer, b))
            row = bt[b].contiguous()
            for t0 in range(0, start_lens[b], chunk):
                n = min(chunk, start_lens[b] - t0)
                k, v = kvsynth.kv_tokens_torch(gen, n, gain, dev)
                # the append kernel's own start and end (events recorded by its launch)
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                pool.append(k, v, t0, row, events=ev if n == chunk else None)
                if n == chunk:
                    append_ev.append(ev)
        pools.append(pool)
        tables.append(bt)
        torch.cuda.synchronize()
        log(f"layer {layer}: prefilled {start_lens} tokens")
    return s, pools, tables, start_lens, max_pages, append_ev


def read_ceiling(args, wl, dev, s, pools, tables, lens_now, max_ctx, pps, per_tok):
    """The roofline reference of the split kernel: a plain read of exactly the bytes one
    decode launch streams (every work item's KV-head part of its pages, through the same
    block tables, split sizes and work-item order, with the split kernel's workgroup size and
    grid policy: one workgroup per item within one round of resident workgroups, a counter
    beyond it;
    lib/libkvmeasure.so), timed like the split kernel with events recorded at the kernel's
    own start and end, over the same layers in the same rotation (so its reads come from
    HBM as the split kernel's do). Returns None when the measurement library is not built."""
    import ctypes as C

    import torch

    path = os.path.join(ROOT, "offloaded_kv_cache_amd", "lib", "libkvmeasure.so")
    if not os.path.exists(path):
        log("read ceiling: lib/libkvmeasure.so not built, skipped")
        return None
    lib = C.CDLL(path)
    fn = lib.kv_measure_read_pages
    fn.restype = C.c_int
    fn.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int,
                   C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    L, B = wl["layers"], len(lens_now)
    # the split kernel's workgroups and their round of residents: four waves, two per CU, for
    # 4-bit K; eight waves, one per CU, for 8-bit K
    four_bit_k = wl["fmt"] in ("q4_0", "fp4")
    threads = 256 if four_bit_k else 512
    n_resident = (2 if four_bit_k else 1) * torch.cuda.get_device_properties(dev).multi_processor_count
    counter = torch.zeros(2, dtype=torch.int32, device=dev)
    n_kv = 4
    head_bytes = per_tok * PAGE // n_kv
    n_splits = -(-(-(-max_ctx // PAGE)) // pps)
    ctx = torch.tensor(lens_now, dtype=torch.int32, device=dev)
    out = torch.empty(n_splits * B * n_kv * threads, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    evs = []
    for rep in range(args.warmup + args.steps):
        for layer in range(L):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)  # (creates the events; the launch records them again)
            bt = tables[layer]
            r = fn(pools[layer].data.data_ptr(), pools[layer].n_pages, head_bytes, n_kv, bt.data_ptr(), bt.shape[1],
                   ctx.data_ptr(), B, pps, n_splits, threads, n_resident, counter.data_ptr(), out.data_ptr(),
                   C.c_void_p(stream.cuda_stream), C.c_void_p(a.cuda_event), C.c_void_p(b.cuda_event))
            if r != 0:
                raise RuntimeError("kv_measure_read_pages rejected its arguments")
            if rep >= args.warmup:
                evs.append((a, b))
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
    nbytes = sum(lens_now) * per_tok
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "plain read of the launch's pages", "avg_launch_us": round(us, 3),
            "achieved": round(achieved, 2), "frac": round(achieved / HBM_PEAK_GBS, 4)}


def run_resident(args, wl, dev):
    import torch

    import kvsynth
    import offloaded_kv_cache_amd as K

    fmt, L, lens, cfg = wl["fmt"], wl["layers"], wl["lens"], wl["cfg"]
    B = len(lens)
    if B > 1 and args.pages_per_split == 0:
        # lengths differ: size the splits by the batch's total, not B x the longest
        args.pages_per_split = K.decode_split_pages(K.shape(fmt), B, max(lens), sum(lens))
    s, pools, tables, start_lens, max_pages, append_ev = build_resident(args, wl, dev)
    torch.cuda.synchronize()
    app_ms = [a.elapsed_time(b) for a, b in append_ev]
    n_steps = args.warmup + args.steps
    max_ctx = max(lens)
    # step inputs, drawn up front and resident in HBM
    gen = torch.Generator(device=dev)
    gen.manual_seed(kvsynth.torch_seed(cfg, 99))
    q_all = torch.randn((n_steps, L, B, 24, 256), generator=gen, device=dev).to(torch.float16)
    knew = torch.randn((n_steps, L, B, 4, 256), generator=gen, device=dev).to(torch.float16)
    vnew = torch.randn((n_steps, L, B, 4, 256), generator=gen, device=dev).to(torch.float16)
    ctx = torch.tensor([[start_lens[b] + st + 1 for b in range(B)] for st in range(n_steps)],
                       dtype=torch.int32, device=dev)
    ws = K.paged.DecodeWorkspace(s, B, max_ctx, args.pages_per_split, device=dev)
    out = torch.empty((B, 24, 256), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    per_tok = kv_bytes_per_token(fmt)
    timed_split = []
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(n_steps)]
    for pair in (p for row in events for p in row):
        for e in pair:
            e.record(stream)  # creates the events before the timed region

    def step(st, timing, strm=None):
        strm = stream if strm is None else strm
        for layer in range(L):
            # the split kernel's own start and end are recorded on its stream (kernel duration
            # without the queueing gap in front of it)
            evs = events[st][layer] if timing and layer % args.event_every == 0 else None
            if args.separate_append:
                for b in range(B):
                    T = start_lens[b] + st + 1
                    pools[layer].append(knew[st, layer, b][None], vnew[st, layer, b][None], T - 1,
                                        tables[layer][b].contiguous() if B > 1 else tables[layer][0])
                K.decode_attention(s, q_all[st, layer], pools[layer].data, tables[layer], ctx[st], max_ctx,
                                   out, ws.data, pages_per_split=args.pages_per_split, phase="split",
                                   stream=strm, events=evs)
                K.decode_attention(s, q_all[st, layer], pools[layer].data, tables[layer], ctx[st], max_ctx,
                                   out, ws.data, pages_per_split=args.pages_per_split, phase="combine",
                                   stream=strm)
            else:
                # one layer's decode step: the token's append runs inside the split kernel
                K.append_decode(s, knew[st, layer], vnew[st, layer], q_all[st, layer], pools[layer].data,
                                tables[layer], ctx[st], max_ctx, out, ws.data,
                                pages_per_split=args.pages_per_split, stream=strm, events=evs)
            if evs is not None:
                timed_split.append((evs[0], evs[1], sum(start_lens[b] + st + 1 for b in range(B)) * per_tok))

    for st in range(args.warmup):
        step(st, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.warmup, n_steps):
        step(st, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"decode status word {ws.status()}")
    kv_bytes = sum(sum(start_lens[b] + st + 1 for b in range(B)) * per_tok * L
                   for st in range(args.warmup, n_steps))
    split_ms = [a.elapsed_time(b) for a, b, _ in timed_split]
    split_bytes = [x for _, _, x in timed_split]
    achieved = sum(split_bytes) / (sum(split_ms) * 1e-3) / 1e9
    # the split size the launches used (the library's own when none was given)
    pps = args.pages_per_split or K.decode_split_pages(s, B, max_ctx, sum(lens) if B > 1 else 0)
    ceiling = None if args.no_read_ceiling else read_ceiling(
        args, wl, dev, s, pools, tables, [start_lens[b] + n_steps for b in range(B)], max_ctx, pps, per_tok)
    # The same timed steps again, each captured once as a HIP graph and replayed (as a serving
    # loop would run a decode step): the appends write the same tokens to the same rows again
    # and the attention reads the same pages. Kernel events cannot be read inside a graph, so
    # the roofline above comes from the eager steps; this is the step time without launch gaps.
    graph = None
    if not args.no_graph and not args.separate_append:
        try:
            cap = torch.cuda.Stream()
            graphs = []
            for st in range(args.warmup, n_steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step(st, False, cap)
                graphs.append(g)
            graphs[0].replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            wall_g = time.perf_counter() - t1
            if ws.status() != 0:
                raise RuntimeError(f"decode status word {ws.status()} after the graph replays")
            graph = {"ms_per_step": round(wall_g / args.steps * 1e3, 4), "value": round(kv_bytes / wall_g / 1e9, 2),
                     "unit": "GB/s"}
        except Exception as ex:  # the eager figures stand on their own
            log(f"graph replay skipped: {ex!r}"[:300])
    res = dict(
        graph=graph,
        read_ceiling=ceiling,
        value=kv_bytes / wall / 1e9,
        ms_per_step=wall / args.steps * 1e3,
        split_us=sum(split_ms) / len(split_ms) * 1e3,
        split_bytes=sum(split_bytes) / len(split_bytes),
        achieved=achieved,
        append_chunk_us=(sum(app_ms) / len(app_ms) * 1e3) if app_ms else None,
        append_chunk_median_us=(sorted(app_ms)[len(app_ms) // 2] * 1e3) if app_ms else None,
        n_append_chunks=len(app_ms),
        pages_per_split=args.pages_per_split,
    )
    return res, (s, pools, tables, start_lens)


def run_multi_query(args, wl, dev):
    """Speculative verification: per layer, append the step's n_q new tokens (one chunk,
    kv_append_quantize) and run their causal attention (kv_decode_attention_mq)."""
    import torch

    import kvsynth
    import offloaded_kv_cache_amd as K

    fmt, L, lens, cfg = wl["fmt"], wl["layers"], wl["lens"], wl["cfg"]
    nq, B = args.queries, len(lens)
    s, pools, tables, start_lens, max_pages, _ = build_resident(args, wl, dev, per_step=nq)
    n_steps = args.warmup + args.steps
    max_ctx = max(lens)
    gen = torch.Generator(device=dev)
    gen.manual_seed(kvsynth.torch_seed(cfg, 98))
    q_all = torch.randn((n_steps, L, B, nq, 24, 256), generator=gen, device=dev).to(torch.float16)
    knew = torch.randn((n_steps, L, B, nq, 4, 256), generator=gen, device=dev).to(torch.float16)
    vnew = torch.randn((n_steps, L, B, nq, 4, 256), generator=gen, device=dev).to(torch.float16)
    ctx = torch.tensor([[start_lens[b] + (st + 1) * nq for b in range(B)] for st in range(n_steps)],
                       dtype=torch.int32, device=dev)
    ws = K.paged.DecodeWorkspace(s, B, max_ctx, args.pages_per_split, device=dev, n_q=nq)
    out = torch.empty((B, nq, 24, 256), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    per_tok = kv_bytes_per_token(fmt)
    timed = []
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(n_steps)]
    for pair in (p for row in events for p in row):
        for e in pair:
            e.record(stream)

    def step(st, timing):
        for layer in range(L):
            for b in range(B):
                T = start_lens[b] + (st + 1) * nq
                pools[layer].append(knew[st, layer, b], vnew[st, layer, b], T - nq, tables[layer][b].contiguous())
            evs = events[st][layer] if timing and layer % args.event_every == 0 else None
            if evs is not None:
                evs[0].record(stream)
            K.decode_attention_mq(s, q_all[st, layer], pools[layer].data, tables[layer], ctx[st], max_ctx, out,
                                  ws.data, pages_per_split=args.pages_per_split, stream=stream)
            if evs is not None:
                evs[1].record(stream)
                timed.append((evs[0], evs[1], sum(start_lens[b] + (st + 1) * nq for b in range(B)) * per_tok))

    for st in range(args.warmup):
        step(st, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.warmup, n_steps):
        step(st, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"decode status word {ws.status()}")
    kv_bytes = sum(sum(start_lens[b] + (st + 1) * nq for b in range(B)) * per_tok * L
                   for st in range(args.warmup, n_steps))
    call_ms = [a.elapsed_time(b) for a, b, _ in timed]
    call_bytes = [x for _, _, x in timed]
    achieved = sum(call_bytes) / (sum(call_ms) * 1e-3) / 1e9
    return dict(value=kv_bytes / wall / 1e9, ms_per_step=wall / args.steps * 1e3,
                call_us=sum(call_ms) / len(call_ms) * 1e3, call_bytes=sum(call_bytes) / len(call_bytes),
                achieved=achieved, query_tokens_per_s=nq * B * args.steps / wall)


def cpu_baseline(args, wl, dev, state):
    """Time the fp64 oracle (as it stands) on one layer's records of the same inputs."""
    import numpy as np
    import torch

    import kvsynth
    from oracle import attention, records

    fmt, cfg = wl["fmt"], wl["cfg"]
    fmt_id = records.FORMATS[fmt]
    kk, vk = records.kinds(fmt_id)
    seq = wl.get("cpu_seq", 0)
    T = min(args.cpu_tokens, wl["lens"][seq])
    gen = torch.Generator(device=dev)
    gen.manual_seed(kvsynth.torch_seed(cfg, 0, seq))
    gain = kvsynth.gain_torch(cfg, 0, 4, dev)
    ks, vs = [], []
    for t0 in range(0, T, 2048):
        k, v = kvsynth.kv_tokens_torch(gen, min(2048, T - t0), gain, dev)
        ks.append(k.cpu().numpy())
        vs.append(v.cpu().numpy())
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    q = torch.randn((1, 24, 256), generator=gen, device=dev).to(torch.float16).cpu().numpy()[0]
    host = host_info()
    threads = (host["blas"] or {}).get("threads") or 1
    # records (the append side), then the timed attention sample: dequantize + attention
    t0 = time.perf_counter()
    kc, ksc = records.encode(k[:2048].astype(np.float64), kk)
    vc, vsc = records.encode(v[:2048].astype(np.float64), vk)
    quant_s = time.perf_counter() - t0
    kc, ksc = records.encode(k.astype(np.float64), kk)
    vc, vsc = records.encode(v.astype(np.float64), vk)
    t0 = time.perf_counter()
    reps = 0
    while True:
        def get_kv(a, b):
            return records.decode(kc[a:b], ksc[a:b], kk), records.decode(vc[a:b], vsc[a:b], vk)
        attention.decode_attention_chunked(q, get_kv, T, 4, fmt_id)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or reps >= 64:
            break
    gbs = T * kv_bytes_per_token(fmt) * reps / el / 1e9
    which = f"sequence {seq} ({wl['lens'][seq]:,} tokens) of the {len(wl['lens'])}" if len(wl["lens"]) > 1 else "the"
    return dict(value=gbs, unit="GB/s", cores=threads, kind="oracle",
                sample=f"1 layer x {T:,} tokens of {which} workload's sequence(s), fp64 dequantize + attention "
                       f"(numpy: BLAS products on {threads} thread(s), elementwise work on 1), {reps} pass(es) "
                       f"in {el:.1f} s; the rate applies to every layer and sequence alike; oracle quantizer "
                       f"on a 2,048-token chunk (4 KV heads, K and V): {quant_s:.2f} s",
                host=host)


C5 = dict(fmt="int8", layers=16, host_tokens=1048576, slots=128, n_sel=8, miss=0.3, cfg=5)


def cpu_baseline_streaming(args):
    """The oracle's streaming step on the host: per layer, the CLOCK step of a selection of 8
    pages (oracle/residency.py) and fp64 attention over the 2,048 selected tokens, for the 16
    layers of a step, repeated for the time budget."""
    import numpy as np

    import kvsynth
    from oracle import attention, records
    from oracle.residency import ClockTable

    c = C5
    n_pages = args.host_tokens // PAGE
    fmt_id = records.FORMATS[c["fmt"]]
    kk, vk = records.kinds(fmt_id)
    ctx = c["n_sel"] * PAGE
    k, v = kvsynth.kv_tokens_np(c["cfg"], 0, 0, 0, ctx)
    kc, ksc = records.encode(k.astype(np.float64), kk)
    vc, vsc = records.encode(v.astype(np.float64), vk)
    q = kvsynth.q_np(c["cfg"], 0, 1)[0]
    rng = np.random.default_rng(1000 * c["cfg"] + 1)
    tables = [ClockTable(c["slots"], n_pages) for _ in range(c["layers"])]
    host = host_info()
    t0 = time.perf_counter()
    steps = 0
    while True:
        for layer in range(c["layers"]):
            tables[layer].select(rng.choice(n_pages, c["n_sel"], replace=False))
            attention.decode_attention(q, records.decode(kc, ksc, kk), records.decode(vc, vsc, vk), fmt_id)
        steps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or steps >= 1000:
            break
    gbs = steps * c["layers"] * ctx * kv_bytes_per_token(c["fmt"]) / el / 1e9
    threads = (host["blas"] or {}).get("threads") or 1
    return dict(value=gbs, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{steps} streaming step(s) of 16 layers x (CLOCK step of 8 pages + fp64 dequantize and "
                       f"attention over the {ctx:,} selected int8 tokens) in {el:.1f} s (numpy: BLAS products on "
                       f"{threads} thread(s), elementwise work on 1)",
                host=host)


def streaming_selection(rng, table, n_pages, n_sel, miss):
    """n_sel distinct logical pages: each a miss (a page not resident) with probability
    `miss`, else a hit (a resident page); from non-resident pages when nothing is resident."""
    resident = [int(p) for p in table.slot_page if p >= 0]
    res = list(rng.permutation(resident))
    res_set = set(resident)
    picked = []
    for _ in range(n_sel):
        if res and rng.random() >= miss:
            picked.append(res.pop())
            continue
        while True:
            p = int(rng.integers(n_pages))
            if p not in res_set and p not in picked:
                break
        picked.append(p)
    return np.array(picked, np.int32)


def run_streaming(args, dev):
    """C5: KV kept in pinned host memory, 128 device slots per layer; each step, per layer,
    8 selected pages go through the CLOCK table and the zero-copy gather, then attention."""
    import torch

    import kvsynth
    import offloaded_kv_cache_amd as K
    from offloaded_kv_cache_amd import _native as N

    c = dict(C5)
    c["host_tokens"] = args.host_tokens
    fmt, L, cfg = c["fmt"], c["layers"], c["cfg"]
    n_pages = c["host_tokens"] // PAGE
    s = K.shape(fmt)
    pb = K.page_bytes(s)
    layer_bytes = n_pages * pb
    log(f"pinning {L * layer_bytes / 1e9:.1f} GB of host memory")
    host = torch.empty(L * layer_bytes, dtype=torch.uint8, pin_memory=True)
    staging = K.paged.PagedPool(fmt, n_pages, device=dev)
    ident = torch.arange(n_pages, dtype=torch.int32, device=dev)
    qsa = args.selection == "qsa"
    if qsa and args.gather_mode != "layers":
        raise SystemExit("--selection qsa chooses every layer's pages at once: use --gather-mode layers")
    key_sums = torch.zeros((L, n_pages, 4, 256), dtype=torch.int64, device=dev) if qsa else None
    key_reps = torch.zeros((L, n_pages, 4, 256), dtype=torch.float16, device=dev) if qsa else None
    for layer in range(L):
        gen = torch.Generator(device=dev)
        gen.manual_seed(kvsynth.torch_seed(cfg, layer))
        gain = kvsynth.gain_torch(cfg, layer, 4, dev)
        for t0 in range(0, c["host_tokens"], 2048):
            k, v = kvsynth.kv_tokens_torch(gen, 2048, gain, dev)
            staging.append(k, v, t0, ident)
            if qsa:
                K.page_key_sums(s, k, t0, key_sums[layer], key_reps[layer])
        host[layer * layer_bytes:(layer + 1) * layer_bytes].copy_(staging.data)
        torch.cuda.synchronize()
    del staging
    log(f"host pool written: {L} layers x {n_pages} pages")
    # per-layer tables and slots; the page-in schedule of --gather-mode: "layers" = one
    # launch pages in all 16 layers' selections, then the layers attend; "serial" = per
    # layer gather then attention; "overlap" = per-layer gathers on a copy stream
    sl = K.streaming.StreamedLayers(s, L, c["slots"], n_pages, c["n_sel"], dev,
                                    overlap=args.gather_mode == "overlap")
    tables = sl.tables
    ctx_tok = c["n_sel"] * PAGE
    ctx = torch.tensor([ctx_tok], dtype=torch.int32, device=dev)
    ws = K.paged.DecodeWorkspace(s, 1, ctx_tok, 0, device=dev)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(1000 * cfg)
    gen = torch.Generator(device=dev)
    gen.manual_seed(kvsynth.torch_seed(cfg, 99))
    n_steps = args.warmup + args.steps
    q_all = torch.randn((n_steps, L, 1, 24, 256), generator=gen, device=dev).to(torch.float16)
    stream = torch.cuda.current_stream()
    # fill every layer's slots with distinct pages (all misses)
    for layer in range(L):
        fill = rng.permutation(n_pages)[:c["slots"]].astype(np.int32)
        for i in range(0, c["slots"], c["n_sel"]):
            K.gather_pages(s, tables[layer], fill[i:i + c["n_sel"]], host[layer * layer_bytes:(layer + 1) * layer_bytes],
                           sl.slots[layer], sl.block_tables[layer], stream=stream)
    torch.cuda.synchronize()
    gather_ev = []
    misses = 0
    gstream = sl.copy_stream if sl.overlap else stream

    host_layers = [host[layer * layer_bytes:(layer + 1) * layer_bytes] for layer in range(L)]
    sel_dev = torch.empty((L, c["n_sel"]), dtype=torch.int32, device=dev)
    sel_ws = torch.empty(K.select_workspace_bytes(n_pages, L), dtype=torch.uint8, device=dev)
    select_ev = []
    # The random draw stands in for the page selection and is input generation, not part of
    # the step: every step's selections are drawn before the timed region, each against a
    # shadow copy of its layer's table that the library's host CLOCK (kv_residency_select,
    # the code the gather calls run) advances step by step, so the real tables later see
    # the same selections and end in the same state.
    drawn = None
    if not qsa:
        shadow = [N.Residency(c["slots"], n_pages) for _ in range(L)]
        for sh, t in zip(shadow, tables):
            sh.slot_page[:], sh.page_slot[:], sh.ref[:] = t.slot_page, t.page_slot, t.ref
            sh.c.hand = t.hand
        drawn = []
        for _ in range(n_steps):
            rows = [streaming_selection(rng, shadow[layer], n_pages, c["n_sel"], c["miss"]) for layer in range(L)]
            for sh, sel in zip(shadow, rows):
                sh.select(sel)
            drawn.append(np.stack(rows))
    # the timed steps' event pairs, created before the timed region
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for pair in step_ev:
        for e in pair:
            e.record(stream)

    def choose(st, timing):
        """Every layer's selection for step st: the random draw made above, or the GPU page
        selection from each layer's query (copied to the host for the CLOCK step)."""
        if not qsa:
            return drawn[st]
        if timing:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        # one call selects for all 16 layers (each from its own query and page representatives)
        K.select_pages(s, q_all[st, :, 0], key_reps, n_pages, c["n_sel"], sel_dev, sel_ws, stream=stream)
        if timing:
            e1.record(stream)
            select_ev.append((e0, e1))
        return sel_dev.cpu().numpy()

    def step(st, timing):
        nonlocal misses
        if args.gather_mode == "layers":
            sels = choose(st, timing)
            # events recorded by the copy kernel's launch: the time of the copies on the GPU
            ev = step_ev[st - args.warmup] if timing else None
            m = int(sl.gather_layers(sels, host_layers, stream, events=ev).sum())
            if timing:
                gather_ev.append((ev[0], ev[1], m))
                misses += m
            for layer in range(L):
                sl.attend(layer, q_all[st, layer], ctx, ctx_tok, out, ws.data, stream)
            return
        for layer in range(L):
            sel = drawn[st][layer]
            if timing:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                if sl.overlap:
                    gstream.wait_event(sl.attended[layer])  # (the gather's own wait, taken first)
                e0.record(gstream)
            m = sl.gather(layer, sel, host_layers[layer], stream)
            if timing:
                e1.record(gstream)
                gather_ev.append((e0, e1, m))
                misses += m
            sl.attend(layer, q_all[st, layer], ctx, ctx_tok, out, ws.data, stream)

    for st in range(args.warmup):
        step(st, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.warmup, n_steps):
        step(st, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"decode status word {ws.status()}")
    if drawn is not None:  # the real tables ended where the shadow tables did
        for sh, t in zip(shadow, tables):
            if not (np.array_equal(sh.slot_page, t.slot_page) and np.array_equal(sh.ref, t.ref)
                    and sh.hand == t.hand):
                raise RuntimeError("residency tables diverged from the drawn selections' shadow tables")
    g_ms = sum(a.elapsed_time(b) for a, b, _ in gather_ev)
    copied = sum(m for _, _, m in gather_ev) * pb
    # pinned host -> device peak on this machine: one large plain copy
    big = host[:min(host.numel(), 1 << 30)]
    dst = torch.empty(big.numel(), dtype=torch.uint8, device=dev)
    dst.copy_(big, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(big, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d = 3 * big.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    kv_bytes = args.steps * L * ctx_tok * kv_bytes_per_token(fmt)
    return dict(value=kv_bytes / wall / 1e9, ms_per_step=wall / args.steps * 1e3,
                gather={"pcie_GBs": round(copied / (g_ms * 1e-3) / 1e9, 2) if g_ms > 0 else None,
                        "h2d_pinned_peak_GBs": round(h2d, 2),
                        "miss_rate": round(misses / (args.steps * L * c["n_sel"]), 4),
                        "pages_copied": int(misses), "bytes_copied": int(copied),
                        "gather_ms_per_step": round(g_ms / args.steps, 4),
                        "gather_timing": "copy kernel (events recorded by its launch)" if args.gather_mode == "layers"
                        else "events around each host call (CLOCK step, launch and copy)",
                        "schedule": args.gather_mode,
                        "selection": args.selection,
                        "selection_ms_per_step": round(sum(a.elapsed_time(b) for a, b in select_ev) / args.steps, 4)
                        if select_ev else None},
                config={"workload": f"16 layers, {c['host_tokens']:,}-token int8 KV in pinned host memory, "
                                    f"{c['slots']} device slots per layer, {c['n_sel']} selected pages per layer "
                                    f"per step (~{int(c['miss'] * 100)}% misses), CLOCK residency + zero-copy gather "
                                    f"+ attention over the {ctx_tok:,} selected tokens",
                        "layers": L, "n_q_heads": 24, "n_kv_heads": 4, "head_dim": 256, "page_tokens": 256,
                        "batch": 1, "kv_format": fmt, "host_tokens": c["host_tokens"], "slots_per_layer": c["slots"],
                        "selected_pages": c["n_sel"], "miss_probability": c["miss"],
                        "page_in": args.gather_mode})


KERNEL_SRCS = [os.path.join(ROOT, "offloaded_kv_cache_amd", "csrc", f)
               for f in ("kv_decode.hip", "kv_encode.h", "kv_internal.h")]


def kernel_code_hash(paths=None) -> str:
    """sha256 of the decode kernel's sources (the kernel file and the headers it
    compiles from) with comments removed and whitespace runs collapsed, so that an
    edit of comments alone keeps the hash (the code the counters measured is
    unchanged)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths or KERNEL_SRCS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def counter_traffic(workload: str):
    """HBM bytes per decode_split launch from the committed counter summary, or None.

    The summary records the code hash (kernel_code_hash) of the kernel its counters
    were taken with; a kernel changed since then gives None."""
    name = {"c3": "decode_q4_0_128k_hbm_bytes.txt", "c3fp4": "decode_fp4_128k_hbm_bytes.txt",
            "c3fp8": "decode_fp8_128k_hbm_bytes.txt", "c2": "decode_int8_32k.txt",
            "c4": "decode_k8v4_4seq.txt"}.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if path is None or not os.path.exists(path):
        return None
    sha = traffic = None
    for line in open(path):
        if line.startswith("kernel code sha256"):
            sha = line.rsplit(":", 1)[1].strip()
        elif line.startswith("decode_split traffic bytes per launch:"):
            traffic = int(float(line.rsplit(":", 1)[1]))
    return traffic if sha == kernel_code_hash() else None


def _short_kernel(name: str) -> str:
    import re
    m = re.search(r"(decode_split<[^>]*>|append_kernel<[^>]*>|decode_combine|read_pages<[^>]*>|gather\w*|select\w*|"
                  r"key_sums\w*|copyBuffer)", name)
    return m.group(1) if m else name[:60]


def summarize_trace(root: str, last: int):
    """Kernel durations from a rocprofv3 --kernel-trace -f csv directory: every dispatch of each
    kernel of this library, then the last `last` dispatches of each decode kernel and of the
    plain page read (the timed steps)."""
    import csv
    import glob
    import statistics as st
    by = {}
    for f in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = _short_kernel(r["Kernel_Name"])
            by.setdefault(k, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    lines = ["  kernel                                    calls    avg us    min us    max us"]
    for k, v in sorted(by.items()):
        d = [(b - a) / 1000 for a, b in v]
        lines.append(f"  {k:40s} {len(d):6d} {st.mean(d):9.2f} {min(d):9.2f} {max(d):9.2f}")
    lines.append(f"last {last} dispatches of each decode kernel:")
    for k, v in sorted(by.items()):
        if "decode" in k or "read_pages" in k:
            d = [(b - a) / 1000 for a, b in sorted(v)[-last:]]
            lines.append(f"  {k:40s} n={len(d)} mean {st.mean(d):9.2f} us  median {st.median(d):9.2f}  "
                         f"min {min(d):8.2f}  max {max(d):8.2f}")
    return "\n".join(lines)


def summarize_counters(root: str):
    """Per kernel, the mean per dispatch of each counter of a rocprofv3 --pmc -f csv directory."""
    import csv
    import glob
    agg = {}
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            agg.setdefault(_short_kernel(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    lines = []
    for k, d in sorted(agg.items()):
        lines.append(f"{k}")
        for c, v in sorted(d.items()):
            lines.append(f"    {c:32s} mean per dispatch {sum(v) / len(v):16.1f}  (dispatches {len(v)})")
    return "\n".join(lines)


def copy_calibration(args, dev):
    """A plain copy of known size: its counter readings scale the decode kernel's."""
    import torch
    n = args.copy_calibration << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"copy_bytes": n, "copies": args.steps, "us_per_copy": round(us, 3),
                      "read_plus_write_GBs": round(2 * n / us / 1e3, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 30; 100 for c5)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS) + ["c5"])
    ap.add_argument("--host-tokens", type=int, default=C5["host_tokens"],
                    help="c5: tokens per layer in the pinned host pool (multiple of 2048)")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--event-every", type=int, default=4, metavar="N",
                    help="record the split kernel's start/stop events on every N-th layer of each "
                         "timed step (all layers do identical work; recording them on every layer "
                         "adds about 2 us of queueing per layer to the step)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append each step's token with its own kernel (kv_append_quantize) before "
                         "kv_decode_attention, instead of the fused kv_append_decode")
    ap.add_argument("--gather-mode", choices=["layers", "serial", "overlap"], default="layers",
                    help="streaming workload: one page-in launch for all layers (default), a gather "
                         "per layer before its attention, or per-layer gathers on a copy stream")
    ap.add_argument("--selection", choices=["random", "qsa"], default="random",
                    help="streaming workload: pages drawn at random with the set miss rate, or chosen on "
                         "the GPU from each layer's query and per-page key representatives (kv_select_pages)")
    ap.add_argument("--queries", type=int, default=1, metavar="N",
                    help="N > 1: speculative verification of N new tokens per step and layer (append "
                         "of the N-token chunk, then kv_decode_attention_mq) instead of one decode token")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the replay of the timed steps as HIP graphs")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain read of the launch's pages (the split kernel's reference)")
    ap.add_argument("--cpu-tokens", type=int, default=131072)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-hash", action="store_true",
                    help="print the code hash of the decode kernel source (comments removed) and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print kernel durations from a rocprofv3 --kernel-trace -f csv output directory and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-dispatch counter means from a rocprofv3 --pmc -f csv output directory and exit")
    ap.add_argument("--last", type=int, default=80, help="with --summarize-trace: decode dispatches of the timed steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB --steps times "
                         "(reference kernel for calibrating HBM byte counters) and exit")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 100 if args.workload == "c5" else 30
    if args.kernel_hash:
        print(kernel_code_hash())
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.last))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: it measures the single-GPU decode path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(args, dev)
        return
    if args.workload == "c5":
        res = run_streaming(args, dev)
        print(json.dumps({
            "metric": "KV GB/s streamed in decode attention (% of 8 TB/s HBM), c5 workload (pages gathered from a host pool)",
            "value": round(res["value"], 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8 KV, fp32 accumulate", "data": "synthetic",
            "config": res["config"], "gather": res["gather"],
            "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_streaming(args)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.queries > 1:
        res = run_multi_query(args, wl, dev)
        fmt = wl["fmt"]
        print(json.dumps({
            "metric": f"KV GB/s streamed in causal multi-query attention ({args.queries} queries per "
                      f"sequence) at {args.workload} shape",
            "value": round(res["value"], 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": f"{fmt} KV, fp32 accumulate", "data": "synthetic",
            "config": {"workload": f"{args.workload} shape, {args.queries} new tokens per step and layer "
                                   "(chunk append + causal multi-query attention)",
                       "layers": wl["layers"], "context": wl["lens"], "kv_format": fmt,
                       "queries": args.queries, "pages_per_split": args.pages_per_split or "auto"},
            "query_tokens_per_s": round(res["query_tokens_per_s"], 1),
            "roofline": {"bound": "hbm", "kernel": "decode_split + decode_combine (one call)",
                         "achieved": round(res["achieved"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(res["achieved"] / HBM_PEAK_GBS, 4), "traffic": None,
                         "avg_launch_us": round(res["call_us"], 3), "bytes_per_launch": int(res["call_bytes"])},
            "cpu_baseline": None}), flush=True)
        return
    res, state = run_resident(args, wl, dev)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wl, dev, state)
    fmt = wl["fmt"]
    metric = "KV GB/s streamed in decode attention (% of 8 TB/s HBM) at 128K q4_0"
    if args.workload != "c3":
        metric = f"KV GB/s streamed in decode attention (% of 8 TB/s HBM), {args.workload} workload"
    line = {
        "metric": metric,
        "value": round(res["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"q4_0": "q4_0 KV, fp32 accumulate", "int8": "int8 KV, fp32 accumulate",
                  "k8v4": "int8 K / q4_0 V, fp32 accumulate", "fp4": "fp4 (e2m1) KV, fp32 accumulate",
                  "fp8": "fp8 (e4m3) KV, fp32 accumulate"}[fmt],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload],
                   "layers": wl["layers"], "n_q_heads": 24, "n_kv_heads": 4, "head_dim": 256,
                   "page_tokens": 256, "batch": len(wl["lens"]), "context": wl["lens"],
                   "kv_format": fmt, "pages_per_split": args.pages_per_split or "auto",
                   "append": "separate kernel" if args.separate_append else "fused into the split kernel"},
        "pct_of_hbm_peak": round(100 * res["value"] / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "decode_split", "achieved": round(res["achieved"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(res["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(args.workload), "avg_launch_us": round(res["split_us"], 3),
                     "bytes_per_launch": int(res["split_bytes"])},
        # a plain read of the same launch's pages on the same GPU, and the split kernel's rate
        # as a fraction of it
        "read_ceiling": res.get("read_ceiling"),
        # the same steps captured as HIP graphs and replayed (no launch gaps; not `value`)
        "graph_replay": res.get("graph"),
        "frac_of_read_ceiling": (round(res["achieved"] / res["read_ceiling"]["achieved"], 4)
                                 if res.get("read_ceiling") else None),
        # the chunk append kernel over the prefill's chunks: mean (what a kernel trace's average
        # gives, first chunks of every layer included) and median
        "append_2048_chunk_us": round(res["append_chunk_us"], 3) if res["append_chunk_us"] else None,
        "append_2048_chunk_median_us": (round(res["append_chunk_median_us"], 3)
                                        if res.get("append_chunk_median_us") else None),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
