#!/usr/bin/env python3
"""MSA hot-path benchmark on one MI355X.

A step is one decode pass of the whole hot path on the batch-16, 131072-token
workload, one msa_decode call: index scores of the new token against every
cached index key, causal block max-pool and top-16, then attention of all 32
query heads over their group's 16 kept blocks. Eight query sets are rotated
so that the kept blocks change from step to step. Steps are issued back to
back between two events; the same step replayed from a captured graph and
the two-call form (msa_index_topk + msa_sparse_attn_decode) are timed
alongside.

The headline value is algorithmic HBM bytes per step / time (GB/s): every
index key once, the kept K/V blocks once, plus the queries, outputs and
selections. The prefill leg (131072-token prefill, 32 heads / 4 groups) is
reported alongside in TFLOP/s against the bf16 MFMA peak. The CPU oracle is
timed on a bounded sample of the same decode batch.

The 1M-token prefill in 32768-row chunks with E4M3 index data is timed too
(index TFLOP/s against the fp8 MFMA peak), and the decode step with E4M3
index data on the same caches (its figure is the cold-cache step: the
E4M3 keys fit the last-level cache; the warm step is reported beside it).
The 131072-token prefill also times the
sparse branch's backward (msa_sparse_attn_backward), and both prefills are
timed again with query-block-shared selections (msa_index_topk_qblock +
msa_sparse_attn_prefill_qblock), and the index projections of its tokens
(msa_index_project, hidden size 6144 as a stand-in). Prefill legs report the
minimum and the median over five timed steps after one warm-up.

The 4 x 1048576-token decode (uniform lengths, then mixed lengths {256k,
512k, 768k, 1M} on the same caches) is timed the same way, each against the
70%-of-HBM-peak step time; the 4096-token one-group prefill reports latency
(it is too small to fill the chip); the 1M chunked prefill times five passes
of its 32 chunks after one untimed pass. A loop of independent MFMAs gives
the measured bf16 and fp8 matrix ceilings next to the published peaks.

Back-to-back steps re-read the same caches, so part of a working set that
fits the 256 MB last-level cache may be served from it; each decode leg also
reports a cold-cache time (a 1 GiB read between steps, per-step events). A
streaming read of 512 MiB (best of plain and nontemporal loads), timed in the
same run, gives the measured HBM read ceiling next to the published 8 TB/s,
and a streaming copy of 512 MiB the ceiling of an even read/write mix (the
token-level sparse prefill's kernels read and write about as much).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-chunked]
       [--decode-only] [--prefill-only] [--no-cpu-baseline] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0
METRIC = "MSA decode HBM GB/s (% peak) @128k/1M; prefill TFLOP/s (% MFMA peak)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def pinned(torch):
    def alloc(shape, np_dtype):
        import numpy as np
        tdt = {np.uint16: torch.int16, np.uint8: torch.uint8}[np.dtype(np_dtype).type]
        return torch.empty(shape, dtype=tdt, pin_memory=True)
    return alloc


def to_dev(torch, t, bf16=True):
    d = t.to("cuda", non_blocking=True)
    return d.view(torch.bfloat16) if (bf16 and d.dtype == torch.int16) else d


def np_view(t):
    import numpy as np
    a = t.numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode step (every index key of every
    sequence once, kept blocks once, queries, outputs and selections)."""
    k_idx = sum(w.kv_lens) * 128 * (1 if w.index_fp8 else 2)
    kept = 0
    for n in w.kv_lens:  # workload lengths are whole blocks, so each kept block is 128 keys
        kept += w.G * min(w.topk, (n - 1) // 128 + 1) * 128 * 128 * 2 * 2
    small = w.B * (w.H * 128 * 2 * 2 + w.G * 128 * (1 if w.index_fp8 else 2) + w.G * w.topk * 4)
    return k_idx + kept + small, k_idx


def _probe_lib():
    """The benchmark's ceiling probes (libmsa_probe.so)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_30_amd", "libmsa_probe.so"))
    lib.msa_probe_stream_read.restype = ctypes.c_int
    lib.msa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.msa_probe_stream_copy.restype = ctypes.c_int
    lib.msa_probe_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def _stream_read(torch, lib, buf, wgs, sink, nontemporal=0):
    import ctypes
    rc = lib.msa_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), wgs,
                                   nontemporal, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError("stream-read probe failed: %d" % rc)


def cold_ms(torch, fn, steps, warmup, flush_cache=True, per_step=None):
    """Average ms of fn(s) with the last-level cache flushed before each step:
    a 1 GiB buffer is read between steps (reads, so no dirty lines are left to
    write back during the step) and every step is bracketed by its own event
    pair (the events add a few microseconds per step). The per-step times go
    into the list `per_step` when one is given."""
    lib = _probe_lib()
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    for s in range(warmup):
        fn(s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        if flush_cache:
            _stream_read(torch, lib, flush, 16384, sink)
        evs[s][0].record()
        fn(warmup + s)
        evs[s][1].record()
    torch.cuda.synchronize()
    del flush, sink
    times = [a.elapsed_time(b) for a, b in evs]
    if per_step is not None:
        per_step.extend(times)
    return sum(times) / steps


def run_decode(torch, msa, w, steps, warmup, nsets=8):
    import numpy as np
    from msa_synth import workloads as wl
    t0 = time.time()
    alloc = pinned(torch)
    kh, vh, kih = wl.gen_caches(w, alloc=alloc)
    sets = [wl.gen_queries(w, set_id=s, alloc=alloc) for s in range(nsets)]
    log("decode inputs generated in %.1fs" % (time.time() - t0))
    k, v = to_dev(torch, kh), to_dev(torch, vh)
    ki = to_dev(torch, kih, bf16=not w.index_fp8)
    qs = [(to_dev(torch, q), to_dev(torch, qi, bf16=not w.index_fp8)) for q, qi in sets]
    kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk,
                     index_dtype=msa.FP8_E4M3 if w.index_fp8 else msa.BF16)
    ws_i = msa.workspace(cfg, w.B, 1, w.Nmax, msa.WS_INDEX_TOPK)
    ws_d = msa.workspace(cfg, w.B, 1, w.Nmax, msa.WS_SPARSE_DECODE)
    sel = torch.empty((w.B, 1, w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, 1, w.H, 128), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    ws_f = msa.workspace(cfg, w.B, 1, w.Nmax, msa.WS_DECODE)

    def step(s, ev=None):
        """One decode step (msa_decode)."""
        q, qi = qs[s % nsets]
        if ev is not None:
            ev[0].record()
        msa.decode(cfg, q, qi, ki, k, v, kv, sel=sel, out=out, workspace=ws_f)
        if ev is not None:
            ev[1].record()

    def step_two_calls(s, ev=None):
        """The same step as msa_index_topk + msa_sparse_attn_decode."""
        q, qi = qs[s % nsets]
        if ev is not None:
            ev[0].record()
        msa.index_topk(cfg, qi, ki, kv, None, sel=sel, workspace=ws_i)
        if ev is not None:
            ev[1].record()
        msa.sparse_attn_decode(cfg, q, k, v, kv, sel, out=out, workspace=ws_d)
        if ev is not None:
            ev[2].record()

    def timed(fn, nev):
        """Average ms per step over `steps` back-to-back steps between two events
        (nothing else in the stream), then, if nev > 0, a second run with nev
        events per step for the per-call breakdown."""
        for s in range(warmup):
            fn(s)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for s in range(steps):
            fn(warmup + s)
        end.record()
        torch.cuda.synchronize()
        total = start.elapsed_time(end) / steps
        per = []
        if nev > 0:
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
            torch.cuda.synchronize()
            for s in range(steps):
                fn(warmup + s, evs[s])
            torch.cuda.synchronize()
            per = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(nev - 1)]
        return total, per

    nbm = -(-w.Nmax // 128)
    pooled = torch.full((w.B, 1, w.G, nbm), float("-inf"), dtype=torch.float32, device="cuda")

    def step_pool(s, ev=None):
        """The index scan alone (msa_index_pool): the dominant kernel of a step."""
        _, qi = qs[s % nsets]
        msa.index_pool(cfg, qi, ki, kv, pooled=pooled)

    # Back-to-back launches between two events: the average launch duration
    # (no event packets between launches).
    pool_ms, _ = timed(step_pool, 0)
    ms_two, (idx_ms, att_ms) = timed(step_two_calls, 3)
    # Serving loops replay a captured graph per step: one graph per query set,
    # each a single msa_decode call (the inputs are the graph's own buffers).
    for s in range(nsets):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    for s in range(nsets):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            step(s)
        graphs.append(gph)
    torch.cuda.synchronize()

    def step_graph(s, ev=None):
        if ev is not None:
            ev[0].record()
        graphs[s % nsets].replay()
        if ev is not None:
            ev[1].record()

    ms_graph, _ = timed(step_graph, 0)
    # The headline step: eager msa_decode calls back to back (faster here than
    # replaying a graph per step).
    wall0 = time.perf_counter()
    ms_total, _ = timed(step, 0)
    wall = time.perf_counter() - wall0
    ms_cold = cold_ms(torch, step, steps, warmup)
    ev_times = []
    ms_ev = cold_ms(torch, step, steps, warmup, flush_cache=False, per_step=ev_times)
    ev_times.sort()
    host = dict(k=np_view(kh), v=np_view(vh), ki=np_view(kih), q=np_view(sets[0][0]),
                qi=np_view(sets[0][1]))
    return dict(ms_per_step=ms_total, wall_s=wall, graph_ms=ms_graph, two_call_ms=ms_two,
                cold_ms=ms_cold, events_ms=ms_ev, events_min_ms=ev_times[0],
                events_median_ms=ev_times[len(ev_times) // 2],
                idx_ms=idx_ms, att_ms=att_ms, pool_ms=pool_ms, host=host, k=k, v=v)


def run_decode_fp8_index(torch, msa, w, k, v, steps, warmup, nsets=8):
    """The same decode step with E4M3 index queries and keys (the K/V caches
    of the bf16 run, already on the GPU): msa_decode back to back, and the
    index scan alone through msa_index_pool."""
    from msa_synth import workloads as wl
    alloc = pinned(torch)
    ki = to_dev(torch, wl.gen_index_cache(w, alloc=alloc), bf16=False).view(torch.float8_e4m3fn)
    qs = []
    for s in range(nsets):
        qh, qih = wl.gen_queries(w, set_id=s, alloc=alloc)
        qs.append((to_dev(torch, qh), to_dev(torch, qih, bf16=False).view(torch.float8_e4m3fn)))
    kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk,
                     index_dtype=msa.FP8_E4M3)
    ws = msa.workspace(cfg, w.B, 1, w.Nmax, msa.WS_DECODE)
    sel = torch.empty((w.B, 1, w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, 1, w.H, 128), dtype=torch.bfloat16, device="cuda")
    pooled = torch.full((w.B, 1, w.G, -(-w.Nmax // 128)), float("-inf"), dtype=torch.float32,
                        device="cuda")

    def run(fn):
        for s in range(warmup):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for s in range(steps):
            fn(warmup + s)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def step(s):
        msa.decode(cfg, qs[s % nsets][0], qs[s % nsets][1], ki, k, v, kv, sel=sel, out=out,
                   workspace=ws)

    ms_step = run(step)
    ms_cold = cold_ms(torch, step, steps, warmup)
    ms_pool = run(lambda s: msa.index_pool(cfg, qs[s % nsets][1], ki, kv, pooled=pooled))
    nbytes, kidx_bytes = decode_bytes(w)
    scan_bytes = kidx_bytes + w.B * w.G * 128 + w.B * w.G * (-(-w.Nmax // 128)) * 4
    del ki, qs, ws, pooled
    torch.cuda.empty_cache()
    # The 256 MiB of E4M3 keys fit the last-level cache, so back-to-back steps
    # find them there: the cold-cache step (cache flushed before every step)
    # is the leg's figure, the warm one is reported beside it.
    return {"workload": w.name, "ms_per_step": round(ms_cold, 5),
            "GB/s": round(nbytes / (ms_cold * 1e-3) / 1e9, 2),
            "frac_hbm_peak": round(nbytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "cold cache (1 GiB flush before each step)",
            "algorithmic_bytes_per_step": nbytes,
            "warm_ms_per_step": round(ms_step, 5),
            "warm_GB/s": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
            "warm_frac_hbm_peak": round(nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "idx_scan_kernel<true, false> (E4M3 keys, cached loads, via msa_index_pool)": {
                "ms": round(ms_pool, 5), "bytes": scan_bytes,
                "GB/s": round(scan_bytes / (ms_pool * 1e-3) / 1e9, 2)}}


# Host threads one GPU's job may use on a shared machine (the host's cores are
# split between its GPUs); the oracle uses all of them.
CPU_SHARE = 16


def host_cpu():
    """CPU model, logical CPUs of the host, CPUs this process may run on, and
    the threads the oracle uses: every CPU of the process, at most the one-GPU
    share of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return dict(cpu_model=model, host_logical_cpus=os.cpu_count() or 1,
                process_cpus=avail, threads=max(1, min(avail, CPU_SHARE)))


def cpu_baseline_decode(w, sets, budget_rows=None):
    """The oracle (as written, untuned) on the decode batch: every row of the
    first query sets, as many sets as give every host thread a row (the oracle
    threads over rows)."""
    import numpy as np
    import oracle
    orc = oracle.default()
    ocfg = oracle.Config(groups=w.G, heads_per_group=w.R, topk=w.topk,
                         index_dtype=oracle.E4M3 if w.index_fp8 else oracle.BF16)
    cpu = host_cpu()
    nsets = max(1, min(len(sets), -(-cpu["threads"] // w.B)))
    rows = w.B if budget_rows is None else min(budget_rows, w.B)
    threads = max(1, min(cpu["threads"], rows * nsets))
    # The query sets stacked as one batch over the same caches: the caches
    # are repeated by view (sequence b of set s reads cache b).
    host = sets[0]
    kv1 = np.array(w.kv_lens[:rows], np.int32)
    kv = np.tile(kv1, nsets)
    qs = kv - 1
    sl = slice(0, rows)
    q = np.concatenate([st["q"][sl] for st in sets[:nsets]])
    qi = np.concatenate([st["qi"][sl] for st in sets[:nsets]])
    ki = np.broadcast_to(host["ki"][sl][None], (nsets,) + host["ki"][sl].shape).reshape(
        (nsets * rows,) + host["ki"].shape[1:])
    k = np.broadcast_to(host["k"][sl][None], (nsets,) + host["k"][sl].shape).reshape(
        (nsets * rows,) + host["k"].shape[1:])
    v = np.broadcast_to(host["v"][sl][None], (nsets,) + host["v"][sl].shape).reshape(
        (nsets * rows,) + host["v"].shape[1:])
    t0 = time.perf_counter()
    sel, _ = orc.index_topk(ocfg, qi, ki, kv, qs, threads=threads)
    orc.sparse_attn(ocfg, q, k, v, kv, qs, sel, threads=threads)
    dt = time.perf_counter() - t0
    sub = w.__class__(**{**w.__dict__, "B": rows, "kv_lens": list(w.kv_lens[:rows])})
    nbytes, _ = decode_bytes(sub)
    res = dict(value=round(nsets * nbytes / dt / 1e9, 4), unit="GB/s", cores=threads,
               kind="oracle",
               sample="%d decode steps (query sets) of %d rows (all %d groups, %d heads, "
                      "%d-token contexts): index top-k + sparse attention, %.2f s wall" %
                      (nsets, rows, w.G, w.H, w.Nmax, dt))
    res.update({k_: v_ for k_, v_ in cpu.items() if k_ != "threads"})
    return res


def sparse_work(torch, w, sel, q0):
    """Algorithmic flops of the sparse branch (4*d per (row, head, attended
    key), counted exactly from the selection) and the irreducible bytes of
    the KV-major schedule: each kept (row, group, slot) reads the row's R
    query heads once and writes and reads back one partial (R x (2d + 8) B),
    plus the output and every kept block's K and V once."""
    L = sel.shape[1]
    pos = torch.arange(L, device="cuda", dtype=torch.int64).view(1, L, 1, 1) + q0
    s64 = sel.to(torch.int64)
    valid = (s64 >= 0) & (s64 * 128 <= pos)
    keys = torch.clamp(pos - s64 * 128 + 1, max=128) * valid
    n_keys = float(keys.sum().item())
    n_slots = float(valid.sum().item())
    n_blocks = 0
    for g in range(w.G):
        n_blocks += int(torch.unique(s64[..., g, :][valid[..., g, :]]).numel())
    f_att = 4.0 * 128 * w.R * n_keys
    nbytes = (n_slots * w.R * 128 * 2 + 2 * n_slots * w.R * (128 * 2 + 8) +
              L * w.H * 128 * 2 + n_blocks * 128 * 128 * 2 * 2)
    return f_att, nbytes


def cpu_baseline_prefill(w, host, n_rows=128, seed=0x4D534143):
    """The oracle (as written, untuned) on a uniform random sample of the
    prefill's rows (index top-k + sparse attention per row); the sampled rate
    stands for the whole prefill, whose per-row cost the uniform sample
    averages."""
    import numpy as np
    import oracle
    orc = oracle.default()
    ocfg = oracle.Config(groups=w.G, heads_per_group=w.R, topk=w.topk,
                         index_dtype=oracle.E4M3 if w.index_fp8 else oracle.BF16)
    rows_i = np.sort(np.random.default_rng(seed).choice(w.T, n_rows, replace=False))
    rows = np.stack([np.zeros_like(rows_i), rows_i], axis=1).astype(np.int32)
    kv = np.array(w.kv_lens, np.int32)
    qs = np.array(w.q_start, np.int32)
    cpu = host_cpu()
    threads = cpu["threads"]
    t0 = time.perf_counter()
    sel, _ = orc.index_topk(ocfg, host["qi"], host["ki"], kv, qs, rows=rows, threads=threads)
    orc.sparse_attn(ocfg, host["q"], host["k"], host["v"], kv, qs, sel, rows=rows,
                    threads=threads)
    dt = time.perf_counter() - t0
    res = dict(value=round(n_rows / dt, 2), unit="tokens/s", cores=threads, kind="oracle",
               sample="%d uniform random rows of the %d-token prefill (all groups and heads): "
                      "index top-k + sparse attention, %.2f s wall; the rate stands for the "
                      "whole prefill (extrapolated)" % (n_rows, w.T, dt))
    res.update({k_: v_ for k_, v_ in cpu.items() if k_ != "threads"})
    return res


def run_prefill(torch, msa, w, steps=5, warmup=3, cpu_baseline=False):
    import numpy as np
    from msa_synth import workloads as wl
    t0 = time.time()
    alloc = pinned(torch)
    kh, vh, kih = wl.gen_caches(w, alloc=alloc)
    qh, qih = wl.gen_queries(w, alloc=alloc)
    log("prefill inputs generated in %.1fs" % (time.time() - t0))
    k, v, ki = to_dev(torch, kh), to_dev(torch, vh), to_dev(torch, kih, bf16=not w.index_fp8)
    q, qi = to_dev(torch, qh), to_dev(torch, qih, bf16=not w.index_fp8)
    host = dict(k=np_view(kh), v=np_view(vh), ki=np_view(kih), q=np_view(qh),
                qi=np_view(qih)) if cpu_baseline else None
    del kh, vh, kih, qh, qih
    kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")
    qs = torch.tensor(w.q_start, dtype=torch.int32, device="cuda")
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk,
                     index_dtype=msa.FP8_E4M3 if w.index_fp8 else msa.BF16)
    ws_i = msa.workspace(cfg, w.B, w.T, w.Nmax, msa.WS_INDEX_TOPK)
    sel = torch.empty((w.B, w.T, w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, w.H, 128), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    idx_ms, att_ms = [], []
    for s in range(warmup + steps):
        ev[0].record()
        msa.index_topk(cfg, qi, ki, kv, qs, sel=sel, workspace=ws_i)
        ev[1].record()
        msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qs, out=out)
        ev[2].record()
        torch.cuda.synchronize()
        if s >= warmup:
            idx_ms.append(ev[0].elapsed_time(ev[1]))
            att_ms.append(ev[1].elapsed_time(ev[2]))
    # Backward of the sparse branch for the same selections (msa_sparse_attn_backward),
    # from the forward's out and lse and a seeded upstream gradient.
    lse = torch.empty((w.B, w.T, w.H), dtype=torch.float32, device="cuda")
    msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qs, out=out, lse=lse)
    g = torch.Generator(device="cuda")
    g.manual_seed(0x4D53410B)
    dout = torch.randn((w.B, w.T, w.H, 128), generator=g, device="cuda").to(torch.bfloat16)
    ws_b = msa.workspace(cfg, w.B, w.T, w.Nmax, msa.WS_SPARSE_BACKWARD)
    grads = msa.sparse_attn_backward(cfg, q, k, v, kv, sel, out, lse, dout, q_start=qs,
                                     workspace=ws_b)
    bwd_ms = []
    for s in range(steps):
        ev[0].record()
        msa.sparse_attn_backward(cfg, q, k, v, kv, sel, out, lse, dout, q_start=qs,
                                 dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws_b)
        ev[1].record()
        torch.cuda.synchronize()
        bwd_ms.append(ev[0].elapsed_time(ev[1]))
    del grads, ws_b, dout, lse
    L = w.T
    f_idx = 2.0 * 128 * w.G * L * (L + 1) / 2
    f_att, kv_bytes = sparse_work(torch, w, sel, w.q_start[0])
    ti, ta = min(idx_ms), min(att_ms)
    tb = min(bwd_ms)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    res = dict(workload=w.name, index_ms=round(ti, 3), sparse_ms=round(ta, 3),
               index_tflops=round(f_idx / ti / 1e9, 2), sparse_tflops=round(f_att / ta / 1e9, 2),
               index_flops=f_idx, sparse_flops=f_att,
               index_frac_bf16_peak=round(f_idx / ti / 1e9 / BF16_PEAK_TFLOPS, 4),
               sparse_frac_bf16_peak=round(f_att / ta / 1e9 / BF16_PEAK_TFLOPS, 4),
               sparse_schedule_bytes=kv_bytes,
               sparse_schedule_gbs=round(kv_bytes / ta / 1e6, 1),
               total_tflops=round((f_idx + f_att) / (ti + ta) / 1e9, 2),
               timed_steps=steps, times_are="min over the timed steps",
               index_ms_median=round(med(idx_ms), 3), sparse_ms_median=round(med(att_ms), 3),
               backward_ms_median=round(med(bwd_ms), 3),
               backward_ms=round(tb, 3),
               backward_flops=2 * f_att,
               backward_tflops=round(2 * f_att / tb / 1e9, 2),
               backward_frac_bf16_peak=round(2 * f_att / tb / 1e9 / BF16_PEAK_TFLOPS, 4),
               backward_note="msa_sparse_attn_backward; flops = dP, dq, dk, dv products "
                             "(8*d per row, head and attended key, twice the forward's; the "
                             "tile kernel also recomputes S once)")
    del q, qi, k, v, ki, sel, out, ws_i
    torch.cuda.empty_cache()
    if host is not None:
        cb = cpu_baseline_prefill(w, host)
        cb["gpu_tokens_per_s"] = round(L / ((ti + ta) * 1e-3), 1)
        cb["gpu_over_oracle"] = round(cb["gpu_tokens_per_s"] / cb["value"], 1)
        res["cpu_baseline"] = cb
    return res


def run_projection(torch, msa, M=131072, h=6144, G=4, steps=5, warmup=3):
    """Index projections (msa_index_project) for the 131072 tokens of the
    prefill: hidden [M, h] x w[(G+1)*dI, h]^T, bf16 in and out. The pages give
    no hidden size; 6144 is a stand-in."""
    import numpy as np
    import msa_synth as ms
    hid = torch.empty((M, h), dtype=torch.bfloat16, device="cuda")
    w = torch.empty(((G + 1) * 128, h), dtype=torch.bfloat16, device="cuda")
    hh = ms.fill_normal_bf16(np.empty((M, h), np.uint16), 0x4D534150)
    hid.copy_(torch.from_numpy(hh.view(np.int16)).view(torch.bfloat16))
    wh = ms.fill_normal_bf16(np.empty(((G + 1) * 128, h), np.uint16), 0x4D534151)
    w.copy_(torch.from_numpy(wh.view(np.int16)).view(torch.bfloat16) / float(np.sqrt(h)))
    del hh, wh
    cfg = msa.Config(num_kv_groups=G, heads_per_group=8, topk=16)
    q, k = msa.index_project(cfg, hid, w)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for s in range(warmup + steps):
        ev[0].record()
        msa.index_project(cfg, hid, w, q_idx=q, k_idx=k)
        ev[1].record()
        torch.cuda.synchronize()
        if s >= warmup:
            times.append(ev[0].elapsed_time(ev[1]))
    t = min(times)
    flops = 2.0 * M * h * (G + 1) * 128
    del hid, w, q, k
    torch.cuda.empty_cache()
    return dict(workload="index_projection_L131072_h6144", ms=round(t, 4),
                ms_median=round(sorted(times)[len(times) // 2], 4), flops=flops,
                tflops=round(flops / t / 1e9, 2),
                frac_bf16_peak=round(flops / t / 1e9 / BF16_PEAK_TFLOPS, 4),
                note="hidden size 6144 is a stand-in (the pages give none)")


def qblock_rows(torch, sel_blk, q0, L):
    """Per-row selections [1, L, G, K] from query-block selections [1, NQ, G, K]
    (row i takes the selection of its block, slot (q0 + i)//128 - q0//128)."""
    i = torch.arange(L, device="cuda", dtype=torch.int64)
    slots = (q0 + i) // 128 - q0 // 128
    return sel_blk[:, slots]


def run_prefill_qblock(torch, msa, w, steps=5, warmup=3):
    """The 131072-token prefill with query-block-shared selections (each
    128-row query block keeps one top-16): msa_index_topk_qblock +
    msa_sparse_attn_prefill_qblock, sparse flops counted exactly per row."""
    from msa_synth import workloads as wl
    alloc = pinned(torch)
    kh, vh, kih = wl.gen_caches(w, alloc=alloc)
    qh, qih = wl.gen_queries(w, alloc=alloc)
    k, v, ki = to_dev(torch, kh), to_dev(torch, vh), to_dev(torch, kih, bf16=not w.index_fp8)
    q, qi = to_dev(torch, qh), to_dev(torch, qih, bf16=not w.index_fp8)
    del kh, vh, kih, qh, qih
    kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")
    qs = torch.tensor(w.q_start, dtype=torch.int32, device="cuda")
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk)
    sel = torch.empty((w.B, msa.qblock_slots(w.T), w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, w.H, 128), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    idx_ms, att_ms = [], []
    for s in range(warmup + steps):
        ev[0].record()
        msa.index_topk_qblock(cfg, qi, ki, kv, qs, sel=sel)
        ev[1].record()
        msa.sparse_attn_prefill_qblock(cfg, q, k, v, kv, sel, q_start=qs, out=out)
        ev[2].record()
        torch.cuda.synchronize()
        if s >= warmup:
            idx_ms.append(ev[0].elapsed_time(ev[1]))
            att_ms.append(ev[1].elapsed_time(ev[2]))
    L = w.T
    f_idx = 2.0 * 128 * w.G * L * (L + 1) / 2
    f_att, _ = sparse_work(torch, w, qblock_rows(torch, sel, w.q_start[0], L), w.q_start[0])
    ti, ta = min(idx_ms), min(att_ms)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    res = dict(workload=w.name + "_qblock", selection="query-block-shared (one top-16 per "
               "128-row query block)", index_ms=round(ti, 3), sparse_ms=round(ta, 3),
               timed_steps=steps, times_are="min over the timed steps",
               index_ms_median=round(med(idx_ms), 3), sparse_ms_median=round(med(att_ms), 3),
               index_tflops=round(f_idx / ti / 1e9, 2), sparse_tflops=round(f_att / ta / 1e9, 2),
               sparse_flops=f_att,
               index_frac_bf16_peak=round(f_idx / ti / 1e9 / BF16_PEAK_TFLOPS, 4),
               sparse_frac_bf16_peak=round(f_att / ta / 1e9 / BF16_PEAK_TFLOPS, 4),
               total_tflops=round((f_idx + f_att) / (ti + ta) / 1e9, 2))
    del q, qi, k, v, ki, sel, out
    torch.cuda.empty_cache()
    return res


def run_chunked(torch, msa, w, passes=5):
    """The 1M-token prefill in 32768-row chunks with E4M3 index data: every
    chunk runs msa_index_topk and msa_sparse_attn_prefill over the cache of
    the tokens before and in it. Inputs are generated once and resident in
    HBM; one untimed pass, then `passes` timed passes of all 32 chunks (each
    call between its own events); min and median over the passes."""
    from msa_synth import workloads as wl
    t0 = time.time()
    alloc = pinned(torch)
    kh, vh, kih = wl.gen_caches(w, alloc=alloc)
    qh, qih = wl.gen_queries(w, row0=0, rows=w.Nmax, alloc=alloc)
    log("chunked-prefill inputs generated in %.1fs" % (time.time() - t0))
    k, v, ki = to_dev(torch, kh), to_dev(torch, vh), to_dev(torch, kih, bf16=False)
    q, qi = to_dev(torch, qh), to_dev(torch, qih, bf16=False)
    del kh, vh, kih, qh, qih
    qi = qi.view(torch.float8_e4m3fn)
    ki = ki.view(torch.float8_e4m3fn)
    C, L = w.chunk, w.Nmax
    nch = L // C
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk, index_dtype=msa.FP8_E4M3)
    ws_p = msa.workspace(cfg, 1, C, L, msa.WS_SPARSE_PREFILL)
    sel = torch.empty((1, C, w.G, w.topk), dtype=torch.int32, device="cuda")
    selq = torch.empty((1, msa.qblock_slots(C), w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((1, C, w.H, 128), dtype=torch.bfloat16, device="cuda")
    lens = [torch.tensor([(c + 1) * C], dtype=torch.int32, device="cuda") for c in range(nch)]
    starts = [torch.tensor([c * C], dtype=torch.int32, device="cuda") for c in range(nch)]

    def one_variant(index_call, attn_call, sel_buf, rows_sel):
        """Times `passes` passes after one untimed pass that also counts the
        sparse flops of every chunk (the selections repeat from pass to pass)."""
        f_att = 0.0
        ti, ta = [], []
        for rep in range(1 + passes):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nch)]
            for c in range(nch):
                rows = slice(c * C, (c + 1) * C)
                ev[c][0].record()
                index_call(qi[:, rows], lens[c], starts[c], sel_buf)
                ev[c][1].record()
                attn_call(q[:, rows], lens[c], starts[c], sel_buf)
                ev[c][2].record()
                if rep == 0:
                    torch.cuda.synchronize()
                    f_att += sparse_work(torch, w, rows_sel(sel_buf, c), c * C)[0]
            torch.cuda.synchronize()
            if rep > 0:
                ti.append(sum(e[0].elapsed_time(e[1]) for e in ev))
                ta.append(sum(e[1].elapsed_time(e[2]) for e in ev))
        return f_att, ti, ta

    f_att, ti_l, ta_l = one_variant(
        lambda qi_c, kv_c, qs_c, sb: msa.index_topk(cfg, qi_c, ki, kv_c, qs_c, sel=sb),
        lambda q_c, kv_c, qs_c, sb: msa.sparse_attn_prefill(cfg, q_c, k, v, kv_c, sb,
                                                             q_start=qs_c, out=out,
                                                             workspace=ws_p),
        sel, lambda sb, c: sb)
    fq_att, tqi_l, tqa_l = one_variant(
        lambda qi_c, kv_c, qs_c, sb: msa.index_topk_qblock(cfg, qi_c, ki, kv_c, qs_c, sel=sb),
        lambda q_c, kv_c, qs_c, sb: msa.sparse_attn_prefill_qblock(cfg, q_c, k, v, kv_c, sb,
                                                                    q_start=qs_c, out=out),
        selq, lambda sb, c: qblock_rows(torch, sb, c * C, C))
    med = lambda xs: sorted(xs)[len(xs) // 2]
    ti, ta, tqi, tqa = min(ti_l), min(ta_l), min(tqi_l), min(tqa_l)
    f_idx = 2.0 * 128 * w.G * L * (L + 1) / 2
    qblock = dict(selection="query-block-shared (one top-16 per 128-row query block)",
                  index_ms=round(tqi, 2), sparse_ms=round(tqa, 2),
                  index_ms_median=round(med(tqi_l), 2), sparse_ms_median=round(med(tqa_l), 2),
                  index_tflops=round(f_idx / tqi / 1e9, 2),
                  index_frac_fp8_peak=round(f_idx / tqi / 1e9 / FP8_PEAK_TFLOPS, 4),
                  sparse_tflops=round(fq_att / tqa / 1e9, 2),
                  sparse_frac_bf16_peak=round(fq_att / tqa / 1e9 / BF16_PEAK_TFLOPS, 4),
                  total_tflops=round((f_idx + fq_att) / (tqi + tqa) / 1e9, 2))
    res = dict(workload=w.name, chunks=nch, timed_passes=passes,
               times_are="min over the timed passes (each the sum of its 32 chunks' calls)",
               index_ms=round(ti, 2), sparse_ms=round(ta, 2),
               index_ms_median=round(med(ti_l), 2), sparse_ms_median=round(med(ta_l), 2),
               index_tflops=round(f_idx / ti / 1e9, 2),
               index_frac_fp8_peak=round(f_idx / ti / 1e9 / FP8_PEAK_TFLOPS, 4),
               sparse_flops=f_att,
               sparse_tflops=round(f_att / ta / 1e9, 2),
               sparse_frac_bf16_peak=round(f_att / ta / 1e9 / BF16_PEAK_TFLOPS, 4),
               total_tflops=round((f_idx + f_att) / (ti + ta) / 1e9, 2),
               note="index in E4M3 (mixed precision total)", qblock=qblock)
    del q, qi, k, v, ki, sel, selq, out, ws_p
    torch.cuda.empty_cache()
    return res


def run_decode_long(torch, msa, steps, warmup, nsets=8):
    """The 4 x 1048576-token decode: uniform lengths, then the mixed lengths
    {262144, 524288, 786432, 1048576} on the same caches (the mixed workload
    has the same contents). For each: msa_decode back to back between two
    events with eight query sets rotating, the same with a 1 GiB read between
    steps (cold cache), and the index scan alone (msa_index_pool) against the
    HBM peak."""
    from msa_synth import workloads as wl
    wu, wm = wl.workload(4), wl.workload(4, mixed=True)
    t0 = time.time()
    alloc = pinned(torch)
    kh, vh, kih = wl.gen_caches(wu, alloc=alloc)
    sets = [wl.gen_queries(wu, set_id=s, alloc=alloc) for s in range(nsets)]
    log("1M decode inputs generated in %.1fs" % (time.time() - t0))
    k, v, ki = to_dev(torch, kh), to_dev(torch, vh), to_dev(torch, kih)
    qs = [(to_dev(torch, q), to_dev(torch, qi)) for q, qi in sets]
    del kh, vh, kih, sets
    cfg = msa.Config(num_kv_groups=wu.G, heads_per_group=wu.R, topk=wu.topk)
    ws = msa.workspace(cfg, wu.B, 1, wu.Nmax, msa.WS_DECODE)
    sel = torch.empty((wu.B, 1, wu.G, wu.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((wu.B, 1, wu.H, 128), dtype=torch.bfloat16, device="cuda")
    nbm = -(-wu.Nmax // 128)
    pooled = torch.full((wu.B, 1, wu.G, nbm), float("-inf"), dtype=torch.float32, device="cuda")

    def back_to_back(fn):
        for s in range(warmup):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for s in range(steps):
            fn(warmup + s)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {}
    for w in (wu, wm):
        kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")

        def step(s):
            msa.decode(cfg, qs[s % nsets][0], qs[s % nsets][1], ki, k, v, kv, sel=sel, out=out,
                       workspace=ws)

        ms_step = back_to_back(step)
        per = []
        ms_cold = cold_ms(torch, step, steps, warmup, per_step=per)
        per.sort()
        ms_pool = back_to_back(lambda s: msa.index_pool(cfg, qs[s % nsets][1], ki, kv,
                                                        pooled=pooled))
        nbytes, kidx_bytes = decode_bytes(w)
        scan_bytes = (kidx_bytes + w.B * w.G * 128 * 2 +
                      sum(w.G * (-(-n // 128)) * 4 for n in w.kv_lens))
        target_ms = nbytes / (0.7 * HBM_PEAK_GBS * 1e9) * 1e3
        gbs = nbytes / (ms_step * 1e-3) / 1e9
        res[w.name] = {
            "ms_per_step": round(ms_step, 5), "GB/s": round(gbs, 2),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": nbytes,
            "target_ms_at_70pct": round(target_ms, 5),
            "meets_70pct": ms_step <= target_ms,
            "cold_cache_ms_per_step": round(ms_cold, 5),
            "cold_cache_min_ms": round(per[0], 5),
            "cold_cache_median_ms": round(per[len(per) // 2], 5),
            "cold_cache_GB/s": round(nbytes / (ms_cold * 1e-3) / 1e9, 2),
            "idx_scan_kernel<false, true> (bf16 keys, streaming loads, via msa_index_pool)": {
                "ms": round(ms_pool, 5), "bytes": scan_bytes,
                "GB/s": round(scan_bytes / (ms_pool * 1e-3) / 1e9, 2),
                "frac_hbm_peak": round(scan_bytes / (ms_pool * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    del k, v, ki, qs, ws, sel, out, pooled
    torch.cuda.empty_cache()
    return res


def run_small_prefill(torch, msa, steps=20, warmup=3):
    """The 4096-token prefill with one group of two heads: latency of
    msa_index_topk, msa_sparse_attn_prefill and the pair, and of the
    last-token decode step (msa_decode with the 4096-token cache), each call
    between its own events; then the pair replayed from a HIP graph; min and
    median over `steps`."""
    from msa_synth import workloads as wl
    w = wl.workload(1)
    kh, vh, kih = wl.gen_caches(w)
    qh, qih = wl.gen_queries(w)
    k, v, ki = (torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)
                for a in (kh, vh, kih))
    q, qi = (torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16) for a in (qh, qih))
    kv = torch.tensor(w.kv_lens, dtype=torch.int32, device="cuda")
    qs = torch.tensor(w.q_start, dtype=torch.int32, device="cuda")
    cfg = msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk)
    ws_i = msa.workspace(cfg, w.B, w.T, w.Nmax, msa.WS_INDEX_TOPK)
    ws_p = msa.workspace(cfg, w.B, w.T, w.Nmax, msa.WS_SPARSE_PREFILL)
    ws_d = msa.workspace(cfg, w.B, 1, w.Nmax, msa.WS_DECODE)
    sel = torch.empty((w.B, w.T, w.G, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, w.H, 128), dtype=torch.bfloat16, device="cuda")
    dsel = torch.empty((w.B, 1, w.G, w.topk), dtype=torch.int32, device="cuda")
    dout = torch.empty((w.B, 1, w.H, 128), dtype=torch.bfloat16, device="cuda")
    q_last, qi_last = q[:, -1:].contiguous(), qi[:, -1:].contiguous()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    t_idx, t_att, t_pair, t_dec = [], [], [], []
    for s in range(warmup + steps):
        ev[0].record()
        msa.index_topk(cfg, qi, ki, kv, qs, sel=sel, workspace=ws_i)
        ev[1].record()
        msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qs, out=out, workspace=ws_p)
        ev[2].record()
        torch.cuda.synchronize()
        ev[3].record()
        msa.decode(cfg, q_last, qi_last, ki, k, v, kv, sel=dsel, out=dout, workspace=ws_d)
        ev[4].record()
        torch.cuda.synchronize()
        if s >= warmup:
            t_idx.append(ev[0].elapsed_time(ev[1]) * 1e3)
            t_att.append(ev[1].elapsed_time(ev[2]) * 1e3)
            t_pair.append(ev[0].elapsed_time(ev[2]) * 1e3)
            t_dec.append(ev[3].elapsed_time(ev[4]) * 1e3)
    # The same pair replayed from a HIP graph, as a fixed-shape serving loop
    # replays it: the device-side latency without the host's marshalling and
    # launch costs (the eager figures above start on an idle GPU, so they
    # hold both). The replays must reproduce the eager selection and output.
    eager_sel, eager_out = sel.clone(), out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        msa.index_topk(cfg, qi, ki, kv, qs, sel=sel, workspace=ws_i)
        msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qs, out=out, workspace=ws_p)
    torch.cuda.synchronize()
    t_graph = []
    for s in range(warmup + steps):
        ev[0].record()
        graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        if s >= warmup:
            t_graph.append(ev[0].elapsed_time(ev[1]) * 1e3)
    graph_equal = bool(torch.equal(sel, eager_sel) and torch.equal(out, eager_out))
    del graph
    med = lambda xs: sorted(xs)[len(xs) // 2]
    L = w.T
    f_idx = 2.0 * 128 * w.G * L * (L + 1) / 2
    f_att, _ = sparse_work(torch, w, sel, 0)
    res = {"workload": w.name, "unit": "us", "timed_steps": steps,
           "prefill_us_min": round(min(t_pair), 2), "prefill_us_median": round(med(t_pair), 2),
           "index_topk_us_min": round(min(t_idx), 2), "index_topk_us_median": round(med(t_idx), 2),
           "sparse_attn_us_min": round(min(t_att), 2),
           "sparse_attn_us_median": round(med(t_att), 2),
           "last_token_decode_us_min": round(min(t_dec), 2),
           "last_token_decode_us_median": round(med(t_dec), 2),
           "graph_prefill_us_min": round(min(t_graph), 2),
           "graph_prefill_us_median": round(med(t_graph), 2),
           "graph_matches_eager": graph_equal,
           "index_flops": f_idx, "sparse_flops": f_att,
           "note": "latency figures (32 query tiles; the work is too small to fill the chip)"}
    del k, v, ki, q, qi, sel, out, dsel, dout, ws_i, ws_p, ws_d
    torch.cuda.empty_cache()
    return res


# The sources the decode index kernel is built from: its own file, the shared
# device helpers and the internal constants.
DECODE_KERNEL_SOURCES = ("msa_internal.h", "msa_device.h", "msa_decode.hip")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_30_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(torch, mib=512, reps=5):
    """A plain device-to-device copy of known size (read and write `mib` MiB)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return {"bytes_read": mib << 20, "bytes_written": mib << 20, "ms": round(ms, 5)}


def read_ceiling(torch, mib=512, reps=20):
    """The HBM read ceiling measured live: a streaming read of `mib` MiB
    (16-byte loads, nothing stored) from the benchmark's probe library, best
    of plain and nontemporal loads and of two workgroup counts, back-to-back
    launches between two events."""
    lib = _probe_lib()
    nbytes = mib << 20
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    best = 0.0
    for nt, wgs in ((0, 2048), (0, 16384), (1, 2048), (1, 16384)):
        def launch():
            _stream_read(torch, lib, buf, wgs, sink, nt)
        for _ in range(3):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9)
    del buf, sink
    return round(best, 1)


def copy_ceiling(torch, mib=512, reps=20):
    """The HBM bandwidth of an even mix of reads and writes, measured live: a
    streaming copy of `mib` MiB between two device buffers (16-byte loads and
    stores) from the probe library, best of plain and nontemporal stores and
    of two workgroup counts; bytes counted = read + written."""
    import ctypes
    lib = _probe_lib()
    nbytes = mib << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for nt, wgs in ((0, 2048), (0, 16384), (1, 2048), (1, 16384)):
        def launch():
            rc = lib.msa_probe_stream_copy(ctypes.c_void_p(src.data_ptr()),
                                           ctypes.c_void_p(dst.data_ptr()), nbytes, wgs, nt,
                                           stream)
            if rc != 0:
                raise RuntimeError("stream-copy probe failed: %d" % rc)
        for _ in range(3):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9)
    del src, dst
    return round(best, 1)


def mfma_ceiling(torch, wgs=1024, reps=10):
    """The MFMA throughput measured live: the probe library's loop of
    independent 32x32x16 bf16 (or 32x32x64 E4M3) MFMAs with no memory
    traffic, on 1024 workgroups of four waves (four per SIMD), back-to-back
    launches between two events, after the chip has run the loop for a few
    launches (the clock under sustained matrix load)."""
    import ctypes
    lib = _probe_lib()
    lib.msa_probe_mfma.restype = ctypes.c_int
    lib.msa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    res = {}
    for fp8, iters, peak, name in ((0, 4096, BF16_PEAK_TFLOPS, "bf16"),
                                   (1, 2048, FP8_PEAK_TFLOPS, "fp8")):
        flops = ctypes.c_double(0.0)

        def launch():
            rc = lib.msa_probe_mfma(fp8, wgs, iters, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.byref(flops),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError("MFMA probe failed: %d" % rc)
        for _ in range(5):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        tf = flops.value / (a.elapsed_time(b) / reps * 1e-3) / 1e12
        res[name] = {"value": round(tf, 1), "unit": "TFLOP/s", "frac_of_peak": round(tf / peak, 4)}
    res["what"] = ("independent MFMAs from registers (32x32x16 bf16; 32x32x64 E4M3 with unit "
                   "scales), 1024 workgroups of four waves, measured in this run")
    del sink
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (the reference kernel for "
                         "scaling HBM byte counters)")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the 1M-token chunked prefill with E4M3 index data")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill leg (for profiling its kernels)")
    ap.add_argument("--short-prefill-only", action="store_true",
                    help="run only the 4096-token prefill latency leg (for profiling its "
                         "kernels)")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the 16 x 131072 decode legs (bf16 and E4M3 index data), "
                         "for profiling their kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_30_amd as msa
    from msa_synth import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msa.load()

    if args.short_prefill_only:
        print(json.dumps({"prefill_L4096_G1": run_small_prefill(
            torch, msa, steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.prefill_only:
        res = {"prefill": run_prefill(torch, msa, wl.workload(3), steps=args.steps,
                                      warmup=args.warmup),
               "prefill_qblock": run_prefill_qblock(torch, msa, wl.workload(3)),
               "index_projection": run_projection(torch, msa)}
        if not args.no_chunked:
            res["chunked_prefill"] = run_chunked(torch, msa, wl.workload(5))
        print(json.dumps(res), flush=True)
        return
    w = wl.workload(2)
    res = run_decode(torch, msa, w, args.steps, args.warmup)
    nbytes, kidx_bytes = decode_bytes(w)
    value = nbytes / (res["ms_per_step"] * 1e-3) / 1e9
    # Dominant kernel: the decode index scan (streams every index key once),
    # timed alone through msa_index_pool: k_idx + q_idx read, pooled written.
    nbm = -(-w.Nmax // 128)
    scan_bytes = kidx_bytes + w.B * w.G * 128 * 2 + w.B * w.G * nbm * 4
    achieved = scan_bytes / (res["pool_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.Nmax, "kv_groups": w.G,
                   "heads_per_group": w.R, "head_dim": 128, "index_dim": 128, "block": 128,
                   "topk": w.topk, "index_dtype": "bf16", "parallelism": "none (1 GPU)"},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": nbytes,
        "calls_ms": {"msa_decode": round(res["ms_per_step"], 5),
                     "msa_decode_graph_replay": round(res["graph_ms"], 5),
                     "two_call_step": round(res["two_call_ms"], 5),
                     "msa_index_pool": round(res["pool_ms"], 5),
                     "msa_index_topk": round(res["idx_ms"], 5),
                     "msa_sparse_attn_decode": round(res["att_ms"], 5),
                     "msa_decode_cold_cache": round(res["cold_ms"], 5),
                     "msa_decode_per_step_events_warm": round(res["events_ms"], 5),
                     "msa_decode_per_step_events_warm_min": round(res["events_min_ms"], 5),
                     "msa_decode_per_step_events_warm_median": round(res["events_median_ms"], 5)},
        "cold_cache_GB/s": round(nbytes / (res["cold_ms"] * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "idx_scan_kernel<false, true> (bf16 keys, streaming loads, via msa_index_pool)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("idx_scan_kernel", w.name),
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "launch_ms": round(res["pool_ms"], 5)},
    }
    ceiling = read_ceiling(torch)
    line["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling, 4)
    line["read_ceiling"] = {"value": ceiling, "unit": "GB/s",
                            "what": "streaming read of 512 MiB (16-byte loads, best of plain and "
                                    "nontemporal loads and of 2048 and 16384 workgroups), "
                                    "measured in this run"}
    line["copy_ceiling"] = {"value": copy_ceiling(torch), "unit": "GB/s",
                            "what": "streaming copy of 512 MiB between two buffers (16-byte loads "
                                    "and stores, best of plain and nontemporal stores and of 2048 "
                                    "and 16384 workgroups), read + written bytes, measured in this "
                                    "run: the ceiling of an even read/write mix"}
    line["mfma_ceiling"] = mfma_ceiling(torch)
    if args.calibrate_copy:
        line["copy_calibration"] = copy_calibration(torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w, [res["host"]])
    res.pop("host")
    line["decode_fp8_index"] = run_decode_fp8_index(torch, msa, wl.workload(2, fp8_index=True),
                                                    res.pop("k"), res.pop("v"), args.steps,
                                                    args.warmup)
    torch.cuda.empty_cache()
    if args.decode_only:
        print(json.dumps(line), flush=True)
        return
    line["decode_1M"] = run_decode_long(torch, msa, args.steps, args.warmup)
    line["prefill_L4096_G1"] = run_small_prefill(torch, msa)
    if not args.no_prefill:
        line["prefill"] = run_prefill(torch, msa, wl.workload(3),
                                      cpu_baseline=not args.no_cpu_baseline)
        # The token-level sparse branch is bound by its schedule's traffic
        # (half of it writes): its modelled bytes per second against the copy
        # ceiling measured above.
        line["prefill"]["sparse_schedule_frac_of_copy_ceiling"] = round(
            line["prefill"]["sparse_schedule_gbs"] / line["copy_ceiling"]["value"], 4)
        line["prefill_qblock"] = run_prefill_qblock(torch, msa, wl.workload(3))
        line["index_projection"] = run_projection(torch, msa)
    if not args.no_prefill and not args.no_chunked:
        line["chunked_prefill"] = run_chunked(torch, msa, wl.workload(5))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
