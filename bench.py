#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections ...]

Prints ONE JSON line. ``value`` is the headline: decode at 128K context over
an FP8 E4M3 block-paged cache (1 sequence, 32 query / 8 KV heads, head_dim 128,
2048-token pages, 32 split-KV partitions), in GB/s of algorithmic bytes. One
step = quantize-on-write of the newest token, the split-KV kernel and the
log-sum-exp combine -- every step of the decode path -- issued as one
attn_decode_append_paged call (the write runs inside the split kernel); the
same step as two calls (write kernel, then attn_decode_paged) and replayed from
a HIP graph are reported beside it. Four copies of the 256 MiB
cache are used in rotation so that no step finds its cache in the 256 MB
last-level cache. The same line carries the 32K chunked-prefill throughput
(useful causal TFLOP/s; one step = 8 chunks of 4096 tokens, each a write then a
prefill), the q8 and q16 verify at 128K, the 256K decode, the batched decodes
(8 x 1K-4K E4M3, 16 x 16K E5M2), the draft's sliding-window attention at 32K
and 128K, the 64K prefill in 4096- and 8192-token chunks, the write kernel's
rate, the small prefill+decode workload's latency,
the cost of a decode call with nothing to read, the roofline of the dominant
kernels, and the CPU oracle timed on a bounded sample of the headline
workload.

Each section times its steps twice: a plain loop gives the step rate, and a
second loop of the same steps, with timing-only HIP events that the library
attaches to every launch of the dominant kernel on its stream, gives that
kernel's launch durations (average, and 10th/50th/90th percentiles).

Inputs are synthetic and seeded (attention_paged_flashattention_amd.synth) and
already resident in HBM when a timed region starts.
"""

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS_16 = 2500.0    # MI355X dense fp16 / bf16 MFMA
METRIC = "paged-attn decode GB/s (%HBM peak) @128K FP8 KV; prefill TFLOP/s @32K"
SECTIONS = ["decode128k", "prefill32k", "verify128k", "verify_q16", "decode256k", "decode_b8",
            "decode_b16", "window", "prefill64k", "prefill128k", "prefill256k", "small", "empty",
            "copy"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the HIP runtime already loaded by torch.

    The events are timing-only: created with hipEventDisableSystemFence, so
    recording one does not write back and invalidate the caches around the
    kernel it brackets (the default system-scope fence adds several
    microseconds to each bracketed launch and to the step)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime first)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value


def source_hash(*names):
    """Hash of the named kernel sources with comments and whitespace removed:
    counters stay attached to the code they were taken on, not its comments."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_paged_flashattention_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters(name, kernel_sha):
    """HBM traffic per launch from the committed rocprofv3 --pmc summary, or
    None when absent or taken on a different version of the kernel."""
    path = os.path.join(ROOT, "profiles", f"{name}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_sha:
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i, True)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def pct(v, q):
    """q-th percentile (nearest rank) of a list."""
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))]


def decode_like_section(ev, case, steps, warmup, copies, q_len, name, window=None, graph=False,
                        fused=False):
    """Write the newest q_len tokens of every sequence, then decode/verify
    (or the sliding-window attention when ``window`` is set). With ``fused``
    the two are one call (attn_decode_append_paged). Returns a result dict with
    the step time and the split kernel's times; with ``graph`` also the step
    time when the same steps are replayed from a captured HIP graph."""
    import torch
    from attention_paged_flashattention_amd import pagedattn as pa
    from attention_paged_flashattention_amd import runner

    dc = runner.DeviceCase(case)
    dc.write_all()
    kcs = [dc.key_cache] + [dc.key_cache.clone() for _ in range(copies - 1)]
    vcs = [dc.value_cache] + [dc.value_cache.clone() for _ in range(copies - 1)]
    newest = dc.last_token_rows(q_len)
    k_new, v_new, s_new = dc.k[newest].contiguous(), dc.v[newest].contiguous(), dc.slots[newest].contiguous()
    c = case
    assert not fused or (window is None and len(newest) == c.batch * q_len)
    parts = c.meta.get("partitions", 0)
    if window is not None:
        wsb = pa.pa_window_workspace_bytes(c.batch, q_len, c.num_q_heads, c.num_kv_heads,
                                           c.head_dim, parts, dc.max_ctx, window)
    else:
        op = pa.PA_OP_DECODE if q_len == 1 else pa.PA_OP_VERIFY
        wsb = pa.pa_workspace_bytes(op, c.batch, q_len, c.num_q_heads, c.num_kv_heads,
                                    c.head_dim, parts, dc.max_ctx)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dc.device)
    q4 = dc.q.view(c.batch, q_len, c.num_q_heads, c.head_dim)
    qv = dc.q if (q_len == 1 and window is None and not fused) else q4
    out = torch.empty_like(qv)
    starts = [ev.create() for _ in range(steps)]
    stops = [ev.create() for _ in range(steps)]
    new_shape = (c.batch, q_len, c.num_kv_heads, c.head_dim)

    def step_calls(i, stream=None):
        """The bound calls of one step on cache copy i (marshalled once: the
        timed loops only issue calls)."""
        common = dict(num_partitions=parts, workspace=ws, out=out, stream=stream)
        if fused:
            return [pa.bind_attn_decode_append_paged(
                q4, k_new.view(new_shape), v_new.view(new_shape), kcs[i], vcs[i], c.cache_fmt,
                dc.block_tables, dc.ctx_lens, dc.max_ctx, c.softmax_scale, dc.k_scale,
                dc.v_scale, **common)[0]]
        w = pa.bind_kv_cache_write_fp8(k_new, v_new, s_new, kcs[i], vcs[i], c.cache_fmt,
                                       dc.k_scale, dc.v_scale, stream=stream)
        args = (qv, kcs[i], vcs[i], c.cache_fmt, dc.block_tables, dc.ctx_lens, dc.max_ctx,
                c.softmax_scale, dc.k_scale, dc.v_scale)
        if window is not None:
            a = pa.bind_attn_window_paged(args[0], window, *args[1:], **common)[0]
        elif q_len == 1:
            a = pa.bind_attn_decode_paged(*args, **common)[0]
        else:
            a = pa.bind_attn_verify_paged(*args, **common)[0]
        return [w, a]

    calls = [step_calls(i) for i in range(copies)]
    torch.cuda.synchronize()

    def step(i, record):
        cs = calls[i % copies]
        for f in cs[:-1]:
            f()
        if record:
            pa.pa_profile_next_call(starts[i], stops[i])
        cs[-1]()

    # the step rate from a loop with no events; the split kernel's launch
    # durations from a second timed loop of the same steps with an event pair
    # attached to every split launch (events still cost the stream a little,
    # which would otherwise be billed to the step)
    ms = timed(lambda i, rec: step(i, False), steps, warmup)
    ms_ev = timed(step, steps, 0)
    kern = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    # keys the rows can see: the whole context, or the window plus the block
    seen = [int(x) if window is None else min(int(x), window + q_len) for x in c.ctx_lens]
    kv_bytes = sum(seen) * c.num_kv_heads * c.head_dim * 2 * (1 if c.cache_fmt != "f16" else 2)
    rows = c.batch * q_len * c.num_q_heads
    qo = rows * c.head_dim * 2
    meta = sum(-(-int(x) // c.block_size) for x in seen) * 4 + \
        (0 if c.k_scale is None else 2 * c.num_kv_heads * 4)
    newest_n = len(newest)
    write_bytes = newest_n * c.num_kv_heads * c.head_dim * (2 * 2 + 2) + newest_n * 8
    step_bytes = kv_bytes + meta + 2 * qo + write_bytes
    # the fused kernel also reads the new tokens and writes their codes (no
    # slot array: slots come from the block table it reads anyway)
    fused_write = newest_n * c.num_kv_heads * c.head_dim * (2 * 2 + 2)
    split_bytes = kv_bytes + meta + qo + (fused_write if fused else 0)
    kern_ms = sum(kern) / len(kern)
    graph_ms = None
    if graph:
        side = torch.cuda.Stream()
        graph_ms = graph_step_ms([f for i in range(copies) for f in step_calls(i, side)], side,
                                 copies, steps, warmup)
    del kcs, vcs, dc, calls
    torch.cuda.empty_cache()
    return dict(name=name, ms_per_step=ms, ms_per_step_with_events=ms_ev, step_bytes=step_bytes,
                GBps=step_bytes / ms / 1e6,
                split_us_p10=pct(kern, 10) * 1e3, split_us_p50=pct(kern, 50) * 1e3,
                split_us_p90=pct(kern, 90) * 1e3,
                split_ms=kern_ms, split_bytes=split_bytes,
                split_GBps=split_bytes / kern_ms / 1e6, graph_ms_per_step=graph_ms,
                partitions=(pa.pa_decode_partitions(c.batch, q_len, c.num_q_heads, c.num_kv_heads,
                                                    c.head_dim, dc_max(c)) if window is None else
                            None) if parts == 0 else parts)


def graph_step_ms(calls, side, copies, steps, warmup):
    """One graph holds the calls of one step per cache copy, captured on the
    side stream they are bound to; replays run back to back and the step time
    is the replay time over the steps replayed."""
    import torch
    side.wait_stream(torch.cuda.current_stream())
    for f in calls:                   # eager warm-up on the side stream
        f()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for f in calls:
            f()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    for _ in range(max(1, warmup // copies)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / (reps * copies)
    del g
    return ms


def dc_max(c):
    return int(max(int(x) for x in c.ctx_lens))


def prefill_section(ev, case, steps, warmup, time_writes=False):
    """Chunked prefill of one sequence: each step writes chunk c's K/V and
    runs its prefill against the paged prefix (ctx = chunk (c + 1))."""
    import torch
    from attention_paged_flashattention_amd import pagedattn as pa
    from attention_paged_flashattention_amd import runner

    dc = runner.DeviceCase(case)
    chunk = case.meta["chunk"]
    total = int(case.ctx_lens[0])
    n = total // chunk
    dev = dc.device
    cu = torch.tensor([0, chunk], dtype=torch.int32, device=dev)
    ctxs = [torch.tensor([chunk * (i + 1)], dtype=torch.int32, device=dev) for i in range(n)]
    out = torch.empty((chunk, case.num_q_heads, case.head_dim), dtype=dc.q.dtype, device=dev)
    starts = [[ev.create() for _ in range(n)] for _ in range(steps)]
    stops = [[ev.create() for _ in range(n)] for _ in range(steps)]
    writes, attns = [], []
    for ci in range(n):
        s, e = ci * chunk, (ci + 1) * chunk
        writes.append(pa.bind_kv_cache_write_fp8(dc.k[s:e], dc.v[s:e], dc.slots[s:e], dc.key_cache,
                                                 dc.value_cache, case.cache_fmt, dc.k_scale,
                                                 dc.v_scale))
        attns.append(pa.bind_attn_prefill_paged(dc.q[s:e], cu, chunk, dc.key_cache, dc.value_cache,
                                                case.cache_fmt, dc.block_tables, ctxs[ci], e,
                                                case.softmax_scale, dc.k_scale, dc.v_scale,
                                                out=out)[0])
    torch.cuda.synchronize()

    def step(i, record):
        for ci in range(n):
            writes[ci]()
            if record:
                pa.pa_profile_next_call(starts[i][ci], stops[i][ci])
            attns[ci]()

    ms = timed(lambda i, rec: step(i, False), steps, warmup)
    timed(step, steps, 0)
    per_chunk = [[ev.elapsed_ms(a, b) for a, b in zip(sa, so)] for sa, so in zip(starts, stops)]
    D, Hq = case.head_dim, case.num_q_heads
    chunk_flops = [4 * D * Hq * (chunk * chunk * ci + chunk * (chunk + 1) // 2) for ci in range(n)]
    flops = sum(chunk_flops)
    step_kern = [sum(x) for x in per_chunk]
    kern_ms = sum(step_kern) / steps
    last_ms = sum(x[-1] for x in per_chunk) / steps
    res = dict(name=case.name, chunk=chunk, ms_per_step=ms, flops=flops, TFLOPs=flops / ms / 1e9,
               kernel_ms=kern_ms, kernel_TFLOPs=flops / kern_ms / 1e9,
               kernel_ms_p10=pct(step_kern, 10), kernel_ms_p50=pct(step_kern, 50),
               kernel_ms_p90=pct(step_kern, 90),
               last_chunk_ms=last_ms, last_chunk_TFLOPs=chunk_flops[-1] / last_ms / 1e9,
               launches_per_step=n)
    if time_writes:
        # the write kernel alone: every chunk's write again (same bytes), events
        # around each launch
        ws = [[ev.create() for _ in range(n)] for _ in range(steps)]
        we = [[ev.create() for _ in range(n)] for _ in range(steps)]

        def wstep(i, record):
            for ci in range(n):
                if record:
                    pa.pa_profile_next_call(ws[i][ci], we[i][ci])
                writes[ci]()

        timed(wstep, steps, 1)
        wt = [ev.elapsed_ms(a, b) for sa, so in zip(ws, we) for a, b in zip(sa, so)]
        src_bytes = 2 if case.kv_dtype in ("f16", "bf16") else 4
        cache_bytes = 2 if case.cache_fmt == "f16" else 1
        per_tok = case.num_kv_heads * case.head_dim * 2 * (src_bytes + cache_bytes) + 8
        wbytes = chunk * per_tok + (0 if case.k_scale is None else 2 * case.num_kv_heads * 4)
        wavg = sum(wt) / len(wt)
        res.update(write_bytes_per_launch=wbytes, write_us=wavg * 1e3,
                   write_GBps=wbytes / wavg / 1e6)
    del dc
    torch.cuda.empty_cache()
    return res


def small_section(ev, steps):
    """The small workload: prefill of 64 tokens (Hq 4, Hkv 1, D 64, fp16
    cache, 16-token pages) and the decode at position 64; latency of each
    call pair (write + attention), events around the pair on the stream."""
    import torch
    from attention_paged_flashattention_amd import pagedattn as pa
    from attention_paged_flashattention_amd import runner, synth

    case = synth.prefill_decode_small()
    dc = runner.DeviceCase(case)
    dev = dc.device
    cu = torch.tensor([0, 64], dtype=torch.int32, device=dev)
    ctx64 = torch.tensor([64], dtype=torch.int32, device=dev)
    ctx65 = torch.tensor([65], dtype=torch.int32, device=dev)
    wpf = pa.bind_kv_cache_write_fp8(dc.k[:64], dc.v[:64], dc.slots[:64], dc.key_cache,
                                     dc.value_cache, "f16")
    pf = pa.bind_attn_prefill_paged(dc.q[:64], cu, 64, dc.key_cache, dc.value_cache, "f16",
                                    dc.block_tables, ctx64, 64, case.softmax_scale)[0]
    wdec = pa.bind_kv_cache_write_fp8(dc.k[64:65], dc.v[64:65], dc.slots[64:65], dc.key_cache,
                                      dc.value_cache, "f16")
    qd = dc.q[64:65].contiguous()
    dec = pa.bind_attn_decode_paged(qd, dc.key_cache, dc.value_cache, "f16", dc.block_tables,
                                    ctx65, 65, case.softmax_scale)[0]
    fdec = pa.bind_attn_decode_append_paged(qd.view(1, 1, 4, 64), dc.k[64:65].view(1, 1, 1, 64),
                                            dc.v[64:65].view(1, 1, 1, 64), dc.key_cache,
                                            dc.value_cache, "f16", dc.block_tables, ctx65, 65,
                                            case.softmax_scale)[0]
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, calls in (("prefill64_us", (wpf, pf)), ("decode_at_64_us", (wdec, dec)),
                        ("decode_at_64_fused_write_us", (fdec,))):
        evs = [(ev.create(), ev.create()) for _ in range(steps)]
        for c in calls:
            c()
        torch.cuda.synchronize()
        for a, b in evs:
            ev.record(a, stream)
            for c in calls:
                c()
            ev.record(b, stream)
        torch.cuda.synchronize()
        t = [ev.elapsed_ms(a, b) * 1e3 for a, b in evs]
        res[name] = round(pct(t, 50), 2)
    del dc
    torch.cuda.empty_cache()
    return res


def empty_section(ev, steps):
    """A decode call of the 128K headline shape whose context is empty: the
    grid is launched and every work-group finds nothing to read. Its time is
    the fixed cost of the two launches (split + combine), events around the
    call on the stream."""
    import torch
    from attention_paged_flashattention_amd import pagedattn as pa

    dev = "cuda:0"
    nb, hkv, bs, d, hq = 8, 8, 2048, 128, 32
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8, device=dev)
    vc = torch.zeros((nb, hkv, bs // 64, d, 64), dtype=torch.uint8, device=dev)
    bt = torch.zeros((1, 64), dtype=torch.int32, device=dev)
    ctx = torch.zeros((1,), dtype=torch.int32, device=dev)
    sc = torch.ones((hkv,), dtype=torch.float32, device=dev)
    q = torch.zeros((1, hq, d), dtype=torch.float16, device=dev)
    call = pa.bind_attn_decode_paged(q, kc, vc, "e4m3", bt, ctx, 131072, 0.0884, sc, sc,
                                     num_partitions=32)[0]
    stream = torch.cuda.current_stream().cuda_stream
    call()
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    for a, b in evs:
        ev.record(a, stream)
        call()
        ev.record(b, stream)
    torch.cuda.synchronize()
    t = [ev.elapsed_ms(a, b) * 1e3 for a, b in evs]
    return dict(decode_call_us=round(pct(t, 50), 2))


def copy_section(ev, steps):
    """Achievable HBM bandwidth of a plain device copy (context, and the
    calibration kernel for the traffic counters)."""
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes=2 * nbytes, ms=ms, GBps=2 * nbytes / ms / 1e6)


def cpu_baseline(gpu_ms):
    """The oracle, as it stands, timed on the host's cores for every workload
    (tests/oracle_pool.py: the work is split by (sequence, KV head) over worker
    processes with one BLAS thread each; oracle/ itself is unchanged). The
    oracle's paged cache is built first, untimed (on the GPU side the cache is
    resident too); timed is one step of the workload: the write of the newest
    tokens and the attention of every row (for the 32K prefill: the last 4096-
    token chunk, every row, which is also its heaviest). ``value`` is the 128K
    decode step in GB/s of algorithmic bytes, the unit of the headline.
    ``gpu_ms`` maps workload names to the GPU's step time for the same step."""
    import numpy as np
    from attention_paged_flashattention_amd import synth
    from tests.oracle_pool import OraclePool, default_workers, row_tasks

    workers = default_workers()
    per = {}

    def decode_step(case, name, q_len, unit_bytes):
        pairs = [(b, g) for b in range(case.batch) for g in range(case.num_kv_heads)]
        with OraclePool(case, workers=workers) as pool:
            t0 = time.perf_counter()
            # every token but the newest q_len of each sequence: setup
            tasks = []
            for b, g in pairs:
                c = int(case.ctx_lens[b])
                step = max(1, -(-(c - q_len) // max(1, 32 // len(pairs))))
                for lo in range(0, c - q_len, step):
                    tasks.append({"write": [dict(b=b, g=g, t_lo=lo, t_hi=min(c - q_len, lo + step))]})
            pool.run(tasks)
            setup = time.perf_counter() - t0
            tasks = []
            for b, g in pairs:
                c = int(case.ctx_lens[b])
                t, _ = row_tasks(case, b, g, np.arange(q_len))
                t[0]["write"] = [dict(b=b, g=g, t_lo=c - q_len, t_hi=c)]
                tasks += t
            pool.run(tasks)
            wall = pool.last_wall
        kv = sum(int(x) for x in case.ctx_lens) * case.num_kv_heads * case.head_dim * 2
        per[name] = dict(oracle_s=round(wall, 3), setup_s=round(setup, 1), unit=unit_bytes,
                         oracle_GBps=round(kv / wall / 1e9, 4),
                         gpu_ms=None if gpu_ms.get(name) is None else round(gpu_ms[name], 4))
        if gpu_ms.get(name):
            per[name]["gpu_over_oracle"] = round(wall * 1e3 / gpu_ms[name], 1)
        log(f"cpu baseline {name}: {wall:.2f} s on {workers} workers")

    decode_step(synth.headline_decode_128k(), "decode_128k_e4m3_bs2048_p32", 1, "step")
    decode_step(synth.batched_decode_e4m3(), "decode_b8_1k4k_e4m3_bs16", 1, "step")
    decode_step(synth.verify_q8_128k(), "verify_q8_b4_128k_e5m2_bs2048", 8, "step")
    decode_step(synth.long_decode_256k(), "decode_256k_e4m3_bs2048_p64", 1, "step")

    # workload 1: the 64-token prefill and the decode at 64, every row (tiny)
    small = synth.prefill_decode_small()
    with OraclePool(small, workers=1) as pool:
        pool.build([(0, 0)], token_range=(0, 64))
        t, _ = row_tasks(small, 0, 0, np.arange(64), keys=64)
        pool.run(t)
        w_pf = pool.last_wall
        t, _ = row_tasks(small, 0, 0, np.arange(64, 65))
        t[0]["write"] = [dict(b=0, g=0, t_lo=64, t_hi=65)]
        pool.run(t)
        w_dec = pool.last_wall
    per["prefill64_decode_fp16_d64"] = dict(oracle_s=round(w_pf + w_dec, 4), unit="prefill 64 + decode")

    # the 32K prefill: the last chunk (ctx 32768), write + every row
    case = synth.chunked_prefill_32k()
    chunk = case.meta["chunk"]
    with OraclePool(case, workers=workers) as pool:
        t0 = time.perf_counter()
        pool.build([(0, g) for g in range(case.num_kv_heads)], token_range=(0, 32768 - chunk),
                   pieces=4)
        setup = time.perf_counter() - t0
        tasks = []
        for g in range(case.num_kv_heads):
            t, _ = row_tasks(case, 0, g, np.arange(32768 - chunk, 32768), split=8)
            t[0]["write"] = [dict(b=0, g=g, t_lo=32768 - chunk, t_hi=32768)]
            tasks += t
        pool.run(tasks)
        wall = pool.last_wall
    flops = 4 * 128 * 32 * (chunk * (32768 - chunk) + chunk * (chunk + 1) // 2)
    per["prefill32k_chunk4k_bf16_e4m3_bs2048"] = dict(
        oracle_s=round(wall, 2), setup_s=round(setup, 1), unit="last 4096-token chunk",
        oracle_TFLOPs=round(flops / wall / 1e12, 5),
        gpu_ms=None if gpu_ms.get("prefill32k_last_chunk") is None
        else round(gpu_ms["prefill32k_last_chunk"], 4))
    if gpu_ms.get("prefill32k_last_chunk"):
        per["prefill32k_chunk4k_bf16_e4m3_bs2048"]["gpu_over_oracle"] = round(
            wall * 1e3 / gpu_ms["prefill32k_last_chunk"], 1)
    log(f"cpu baseline prefill 32K last chunk: {wall:.2f} s")

    h = per["decode_128k_e4m3_bs2048_p32"]
    return dict(value=h["oracle_GBps"], unit="GB/s", cores=os.cpu_count(), workers=workers,
                kind="oracle",
                sample=("every workload at full size, one step each (the 32K prefill: its last "
                        "4096-token chunk); the oracle's cache built untimed; numpy float64 in "
                        f"{workers} worker processes with one BLAS thread each, split by "
                        "(sequence, KV head); value = the 128K E4M3 decode step"),
                per_config=per)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated subset of " + ",".join(SECTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py: this build runs on exactly one GPU (no sharding, no collectives); "
              f"--gpus {args.gpus} / WORLD_SIZE {ws} is not supported", file=sys.stderr)
        sys.exit(2)
    sections = [s for s in args.sections.split(",") if s]
    for s in sections:
        if s not in SECTIONS:
            ap.error(f"unknown section {s}")

    import torch
    from attention_paged_flashattention_amd import build as build_mod
    if not os.path.exists(build_mod.OUT):
        build_mod.build()
    from attention_paged_flashattention_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ev = HipEvents()
    K, W = args.steps, args.warmup
    res = {}

    if "copy" in sections:
        log("section copy")
        res["copy"] = copy_section(ev, max(5, K // 2))
    if "decode128k" in sections:
        log("section decode128k")
        res["decode128k"] = decode_like_section(ev, synth.headline_decode_128k(), K, W, 4, 1,
                                                "decode_128k_e4m3_bs2048_p32", graph=True,
                                                fused=True)
        log("section decode128k, write and decode as two calls")
        res["decode128k_2call"] = decode_like_section(ev, synth.headline_decode_128k(), K, W, 4, 1,
                                                      "decode_128k_e4m3_bs2048_p32", graph=True)
    if "prefill32k" in sections:
        log("section prefill32k")
        res["prefill32k"] = prefill_section(ev, synth.chunked_prefill_32k(), max(10, K // 5),
                                            max(1, W // 5), time_writes=True)
    if "verify128k" in sections:
        log("section verify128k")
        res["verify128k"] = decode_like_section(ev, synth.verify_q8_128k(), K, W, 1, 8,
                                                "verify_q8_b4_128k_e5m2_bs2048")
        res["verify128k_fused"] = decode_like_section(ev, synth.verify_q8_128k(), K, W, 1, 8,
                                                      "verify_q8_b4_128k_e5m2_bs2048", fused=True)
    if "verify_q16" in sections:
        log("section verify_q16")
        res["verify_q16"] = decode_like_section(ev, synth.verify_q16_128k(), K, W, 1, 16,
                                                "verify_q16_b4_128k_e5m2_bs2048")
    if "decode256k" in sections:
        log("section decode256k")
        res["decode256k"] = decode_like_section(ev, synth.long_decode_256k(), K, W, 1, 1,
                                                "decode_256k_e4m3_bs2048_p64", fused=True)
    if "decode_b8" in sections:
        log("section decode_b8")
        res["decode_b8"] = decode_like_section(ev, synth.batched_decode_e4m3(), K, W, 8, 1,
                                               "decode_b8_1k4k_e4m3_bs16")
        res["decode_b8_fused"] = decode_like_section(ev, synth.batched_decode_e4m3(), K, W, 8, 1,
                                                     "decode_b8_1k4k_e4m3_bs16", fused=True)
    if "decode_b16" in sections:
        log("section decode_b16")
        res["decode_b16"] = decode_like_section(ev, synth.batched_decode_e5m2_16k(), K, W, 2, 1,
                                                "decode_b16_16k_e5m2_bs16")
        res["decode_b16_fused"] = decode_like_section(ev, synth.batched_decode_e5m2_16k(), K, W, 2,
                                                      1, "decode_b16_16k_e5m2_bs16", fused=True)
    if "window" in sections:
        for ctx in (32768, 131072):
            log(f"section window ctx {ctx}")
            wc = synth.window_draft_q8(ctx=ctx)
            # 8 cache copies: the 34 MB a step reads must not stay in the 256 MB
            # last-level cache from one step to the next
            res[f"window_{ctx}"] = decode_like_section(ev, wc, K, W, 8, 8, wc.name,
                                                       window=wc.meta["window"])
    if "prefill64k" in sections:
        for chunk in (4096, 8192):
            log(f"section prefill64k chunk {chunk}")
            res[f"prefill64k_{chunk}"] = prefill_section(ev, synth.chunked_prefill_64k(chunk=chunk),
                                                         max(5, K // 10), 1)
    for tot, sec in ((131072, "prefill128k"), (262144, "prefill256k")):
        if sec in sections:
            base = synth.chunked_prefill_long(tot, 4096)
            for chunk in (4096, 8192):
                log(f"section {sec} chunk {chunk}")
                case = dataclasses.replace(base, meta=dict(base.meta, chunk=chunk),
                                           name=base.name.replace("chunk4k", f"chunk{chunk // 1024}k"))
                res[f"{sec}_{chunk}"] = prefill_section(ev, case, 3 if tot == 131072 else 2, 1)
            del base
    if "small" in sections:
        log("section small")
        res["small"] = small_section(ev, K)
    if "empty" in sections:
        log("section empty")
        res["empty"] = empty_section(ev, K)

    cpu = None
    if not args.no_cpu_baseline and "decode128k" in sections:
        log("cpu baseline (oracle)")
        gpu_ms = {}
        for key, name in (("decode128k", "decode_128k_e4m3_bs2048_p32"),
                          ("decode_b8_fused", "decode_b8_1k4k_e4m3_bs16"),
                          ("verify128k_fused", "verify_q8_b4_128k_e5m2_bs2048"),
                          ("decode256k", "decode_256k_e4m3_bs2048_p64")):
            if key in res:
                gpu_ms[name] = res[key]["ms_per_step"]
        if "prefill32k" in res:
            gpu_ms["prefill32k_last_chunk"] = res["prefill32k"]["last_chunk_ms"]
        cpu = cpu_baseline(gpu_ms)

    dec_sha = source_hash("attn_decode.hip", "pa_device.h")
    pf_sha = source_hash("attn_prefill.hip", "pa_device.h")
    line = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": W, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    h = res.get("decode128k")
    if h:
        line.update(value=round(h["GBps"], 1), unit="GB/s", ms_per_step=round(h["ms_per_step"], 5),
                    ms_per_step_with_kernel_events=round(h["ms_per_step_with_events"], 5))
        if h["graph_ms_per_step"]:
            line["decode_128k_graph_replay"] = {
                "ms_per_step": round(h["graph_ms_per_step"], 5),
                "GBps": round(h["step_bytes"] / h["graph_ms_per_step"] / 1e6, 1),
                "frac_of_hbm_peak": round(h["step_bytes"] / h["graph_ms_per_step"] / 1e6
                                          / HBM_PEAK_GBPS, 4)}
        h2 = res.get("decode128k_2call")
        if h2:
            line["decode_128k_two_calls"] = {
                "what": "kv_cache_write_fp8 + attn_decode_paged (write kernel, split, combine)",
                "GBps": round(h2["GBps"], 1), "us_per_step": round(h2["ms_per_step"] * 1e3, 2),
                "frac_of_hbm_peak": round(h2["GBps"] / HBM_PEAK_GBPS, 4),
                "split_kernel_us": round(h2["split_ms"] * 1e3, 2),
                "graph_replay_us_per_step": round(h2["graph_ms_per_step"] * 1e3, 2)
                if h2["graph_ms_per_step"] else None}
        line["dtype"] = "fp16"
        line["config"] = {"workload": h["name"], "batch": 1, "context": 131072,
                          "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                          "block_size": 2048, "kv_cache": "fp8_e4m3 per-head scales",
                          "partitions": h["partitions"], "cache_copies_rotated": 4,
                          "step": "attn_decode_append_paged: quantize-on-write of the new "
                                  "token fused into the split kernel, then the combine"}
        ach = h["split_GBps"]
        tr = counters("decode_split_128k_e4m3", dec_sha)
        line["roofline"] = {"bound": "hbm", "kernel": "decode_split_kernel",
                            "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": tr,
                            "algorithmic_bytes_per_launch": h["split_bytes"],
                            "avg_launch_us": round(h["split_ms"] * 1e3, 2),
                            "p10_p50_p90_us": [round(h["split_us_p10"], 2), round(h["split_us_p50"], 2),
                                               round(h["split_us_p90"], 2)]}
    else:
        line.update(value=None, unit="GB/s", ms_per_step=None, dtype="fp16", config={})
    p = res.get("prefill32k")
    if p:
        line["prefill_32k"] = {"workload": "prefill32k_chunk4k_bf16_e4m3_bs2048",
                               "TFLOPs": round(p["TFLOPs"], 1), "ms_per_step": round(p["ms_per_step"], 3),
                               "frac_of_peak": round(p["TFLOPs"] / MFMA_PEAK_TFLOPS_16, 4),
                               "useful_causal_flops": p["flops"],
                               "last_chunk_TFLOPs": round(p["last_chunk_TFLOPs"], 1),
                               "last_chunk_ms": round(p["last_chunk_ms"], 3), "dtype": "bf16",
                               "kernel_ms_per_step_p10_p50_p90": [round(p["kernel_ms_p10"], 3),
                                                                  round(p["kernel_ms_p50"], 3),
                                                                  round(p["kernel_ms_p90"], 3)]}
        line["write_kernel"] = {"workload": "4096-token chunk writes of the 32K prefill (bf16 -> E4M3)",
                                "GBps": round(p["write_GBps"], 1), "us_per_launch": round(p["write_us"], 2),
                                "bytes_per_launch": p["write_bytes_per_launch"],
                                "frac_of_hbm_peak": round(p["write_GBps"] / HBM_PEAK_GBPS, 4)}
        trp = counters("prefill_32k_e4m3", pf_sha)
        line["roofline_prefill"] = {"bound": "mfma", "kernel": "prefill_kernel",
                                    "achieved": round(p["kernel_TFLOPs"], 1),
                                    "peak": MFMA_PEAK_TFLOPS_16, "unit": "TFLOP/s",
                                    "frac": round(p["kernel_TFLOPs"] / MFMA_PEAK_TFLOPS_16, 4),
                                    "traffic": trp,
                                    "algorithmic_flops_per_step": p["flops"],
                                    "avg_launch_us": round(p["kernel_ms"] / p["launches_per_step"] * 1e3, 1)}
    for key, out_key in [("verify128k", "verify_q8_128k"),
                         ("verify128k_fused", "verify_q8_128k_fused_write"),
                         ("verify_q16", "verify_q16_128k"),
                         ("decode256k", "decode_256k_fused_write"), ("decode_b8", "decode_b8"),
                         ("decode_b8_fused", "decode_b8_fused_write"),
                         ("decode_b16", "decode_b16_16k_e5m2"),
                         ("decode_b16_fused", "decode_b16_16k_e5m2_fused_write")]:
        r = res.get(key)
        if r:
            line[out_key] = {"workload": r["name"], "GBps": round(r["GBps"], 1),
                             "us_per_step": round(r["ms_per_step"] * 1e3, 2),
                             "frac_of_hbm_peak": round(r["GBps"] / HBM_PEAK_GBPS, 4),
                             "split_kernel_GBps": round(r["split_GBps"], 1),
                             "split_kernel_us": round(r["split_ms"] * 1e3, 2),
                             "split_kernel_frac": round(r["split_GBps"] / HBM_PEAK_GBPS, 4),
                             "split_us_p10_p50_p90": [round(r["split_us_p10"], 2),
                                                      round(r["split_us_p50"], 2),
                                                      round(r["split_us_p90"], 2)],
                             "partitions": r["partitions"]}
    for ctx in (32768, 131072):
        r = res.get(f"window_{ctx}")
        if r:
            line[f"window_draft_q8_{ctx // 1024}k"] = {
                "workload": r["name"], "window": 4096, "GBps": round(r["GBps"], 1),
                "us_per_step": round(r["ms_per_step"] * 1e3, 2),
                "split_kernel_us": round(r["split_ms"] * 1e3, 2),
                "split_kernel_GBps": round(r["split_GBps"], 1),
                "bytes_in_window_per_step": r["step_bytes"]}
    for sec, tag in (("prefill64k", "64k"), ("prefill128k", "128k"), ("prefill256k", "256k")):
        for chunk in (4096, 8192):
            r = res.get(f"{sec}_{chunk}")
            if r:
                line[f"prefill_{tag}_chunk{chunk // 1024}k"] = {
                    "workload": r["name"], "TFLOPs": round(r["TFLOPs"], 1),
                    "ms_per_step": round(r["ms_per_step"], 3),
                    "frac_of_peak": round(r["TFLOPs"] / MFMA_PEAK_TFLOPS_16, 4),
                    "kernel_TFLOPs": round(r["kernel_TFLOPs"], 1),
                    "last_chunk_TFLOPs": round(r["last_chunk_TFLOPs"], 1),
                    "launches_per_step": r["launches_per_step"]}
    if "small" in res:
        line["small_prefill64_decode_latency"] = dict(res["small"], workload="prefill64_decode_fp16_d64")
    if "empty" in res:
        line["empty_context_decode"] = dict(res["empty"], shape="128K headline launch, ctx 0")
    if "copy" in res:
        line["hbm_copy_GBps"] = round(res["copy"]["GBps"], 1)
    if cpu:
        line["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                for k, v in cpu.items() if k != "seconds"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
