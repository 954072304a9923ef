"""Shapes and seeded contents of the MSA workloads (input generation only).

Five workloads stand in for the pages' length axis (32k -> 512k -> 1M tokens,
prefill and decode); none of the pages uses a public dataset for speed, so
all contents are synthetic:
  Q, K, V        ~ N(0, 1) rounded to bfloat16;
  q_idx, k_idx   uniform integers in [-4, 4], stored as bfloat16 (or as FP8
                 E4M3FN for the 1M chunked prefill) so that index scores are
                 exact in fp32.
Every tensor has its own counter-based stream (msa_synth.stream_seed), so a
slice (one prefill chunk, one decode query set) can be generated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import fill_int_bf16, fill_int_e4m3, fill_normal_bf16, stream_seed

HEAD_DIM = 128
INDEX_DIM = 128
BLOCK = 128
TOPK = 16


@dataclass
class Workload:
    cid: int                 # workload id (seed base)
    name: str
    phase: str               # "prefill", "decode" or "chunked"
    B: int
    T: int                   # query rows per call
    Nmax: int                # cache stride (tokens)
    kv_lens: list
    q_start: list            # position of query row 0 per sequence
    G: int = 4
    R: int = 8
    topk: int = TOPK
    index_fp8: bool = False
    chunk: int = 0           # chunked prefill: rows per call
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def H(self):
        return self.G * self.R


def workload(cid, mixed=False, scale=1, fp8_index=False):
    """The named workload; `scale` > 1 divides every length (for quick tests);
    `fp8_index` stores a decode workload's index data as E4M3FN (same values)."""
    w = _workload(cid, mixed, scale)
    if fp8_index and w.phase == "decode":
        w.index_fp8 = True
        w.name += "_fp8idx"
    return w


def _workload(cid, mixed, scale):
    if cid == 1:
        L = 4096 // scale
        return Workload(1, "prefill_L%d_G1_R2" % L, "prefill", 1, L, L, [L], [0], G=1, R=2)
    if cid == 2:
        N = 131072 // scale
        return Workload(2, "decode_B16_N%d" % N, "decode", 16, 1, N, [N] * 16, [N - 1] * 16)
    if cid == 3:
        L = 131072 // scale
        return Workload(3, "prefill_L%d" % L, "prefill", 1, L, L, [L], [0])
    if cid == 4:
        N = 1048576 // scale
        if mixed:
            lens = [N // 4, N // 2, 3 * N // 4, N]
            return Workload(4, "decode_B4_mixed_N%d" % N, "decode", 4, 1, N, lens,
                            [n - 1 for n in lens], note="mixed lengths")
        return Workload(4, "decode_B4_N%d" % N, "decode", 4, 1, N, [N] * 4, [N - 1] * 4)
    if cid == 5:
        L = 1048576 // scale
        C = 32768 // scale
        return Workload(5, "prefill_L%d_chunk%d_fp8idx" % (L, C), "chunked", 1, C, L, [C], [0],
                        index_fp8=True, chunk=C)
    raise ValueError(cid)


def _fill_index(buf, seed, offset, fp8):
    if fp8:
        return fill_int_e4m3(buf, seed, -4, 4, offset=offset)
    return fill_int_bf16(buf, seed, -4, 4, offset=offset)


def _alloc(shape, dtype, alloc):
    if alloc is None:
        return np.empty(shape, dtype)
    return alloc(shape, dtype)


def gen_caches(w: Workload, alloc=None):
    """k_cache, v_cache [B,G,Nmax,d] bf16 bits and k_idx [B,Nmax,dI] (bf16 or E4M3 bits).

    `alloc(shape, numpy_dtype)` may return any writable contiguous buffer with
    numpy-like ``.size`` (numpy array or CPU torch tensor); default numpy.
    """
    k = _alloc((w.B, w.G, w.Nmax, HEAD_DIM), np.uint16, alloc)
    v = _alloc((w.B, w.G, w.Nmax, HEAD_DIM), np.uint16, alloc)
    fill_normal_bf16(k, stream_seed(w.cid, "k_cache"))
    fill_normal_bf16(v, stream_seed(w.cid, "v_cache"))
    return k, v, gen_index_cache(w, alloc)


def gen_index_cache(w: Workload, alloc=None):
    """k_idx [B,Nmax,dI] alone (bf16 or E4M3 bits), as gen_caches makes it."""
    ki = _alloc((w.B, w.Nmax, INDEX_DIM), np.uint8 if w.index_fp8 else np.uint16, alloc)
    _fill_index(ki, stream_seed(w.cid, "k_idx"), 0, w.index_fp8)
    return ki


def gen_queries(w: Workload, row0=0, rows=None, set_id=0, alloc=None):
    """q [B,rows,H,d] bf16 bits and q_idx [B,rows,G,dI] for query rows [row0, row0+rows).

    For a prefill the row index is the absolute position (rows of the whole
    sequence); `set_id` selects an independent set of decode queries.
    """
    rows = w.T if rows is None else rows
    q = _alloc((w.B, rows, w.H, HEAD_DIM), np.uint16, alloc)
    qi = _alloc((w.B, rows, w.G, INDEX_DIM), np.uint8 if w.index_fp8 else np.uint16, alloc)
    # Sequence b's rows are one contiguous counter range of a long per-tensor stream.
    total_rows = max(w.Nmax, rows) + 8
    for b in range(w.B):
        qb = q[b]
        qib = qi[b]
        base = (set_id * w.B + b) * total_rows
        fill_normal_bf16(qb, stream_seed(w.cid, "q"), offset=(base + row0) * w.H * HEAD_DIM)
        _fill_index(qib, stream_seed(w.cid, "q_idx"), (base + row0) * w.G * INDEX_DIM,
                    w.index_fp8)
    return q, qi
