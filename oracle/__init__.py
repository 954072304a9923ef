"""CPU oracle for MiniMax Sparse Attention — TEST INFRASTRUCTURE ONLY.

ctypes front end of ``msa_oracle.c``: a plain fp64 statement of the method
(index scoring, causal block max-pool, top-k, sparse softmax attention; plus
textbook dense causal attention for invariants; the sparse branch's
gradients for fixed selections), and in plain numpy ``cache_append``, the
cache write of new tokens, and ``index_project``, the index projections. Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does, and the two share no code.

Arrays are numpy, row-major:
  q_idx [B,T,G,dI] (uint16 bf16 bits or uint8 E4M3FN bits), k_idx [B,N,dI],
  q [B,T,H,d] uint16, k_cache / v_cache [B,G,N,d] uint16,
  kv_lens [B] int32, q_start [B] int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "msa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

BF16, E4M3 = 0, 1


def build(force: bool = True, source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compiles the oracle with gcc (-O2, fp64, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread",
                               "-I", _HERE, source, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_double), ("index_dtype", ctypes.c_int32)]


@dataclass
class Config:
    """Shapes of one MSA layer (names follow the pages' sparse_attention_config)."""
    groups: int = 4              # G = KV heads = index heads (sparse_num_index_heads)
    heads_per_group: int = 8     # R
    head_dim: int = 128          # d
    index_dim: int = 128         # d_I (sparse_index_dim)
    block_size: int = 128        # S (sparse_block_size)
    topk: int = 16               # K (sparse_topk_blocks)
    softmax_scale: float = 0.0   # <= 0: 1/sqrt(d)
    index_dtype: int = BF16

    def c(self) -> _Cfg:
        return _Cfg(self.groups, self.heads_per_group, self.head_dim, self.index_dim,
                    self.block_size, self.topk, float(self.softmax_scale), self.index_dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """One loaded build of the oracle library (the tests also load variants)."""

    def __init__(self, path: str | None = None):
        path = path or LIBRARY
        if path == LIBRARY and not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        vp, i32, i64, P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER
        cfgp = P(_Cfg)
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_index_topk_row.argtypes = [cfgp, vp, vp, i64, vp, vp]
        lib.oracle_sparse_attn_row.argtypes = [cfgp, vp, vp, vp, i64, i64, vp, vp, vp]
        lib.oracle_dense_causal_row.argtypes = [cfgp, vp, vp, vp, i64, i64, vp, vp]
        lib.oracle_index_topk_rows.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, i64, vp, vp,
                                               i32, vp, vp]
        lib.oracle_index_pool_row.argtypes = [cfgp, vp, vp, i64, vp]
        lib.oracle_index_pool_rows.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, i64, vp, vp,
                                               i32, i64, vp]
        lib.oracle_sparse_attn_rows.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, vp, i64, vp, vp,
                                                vp, i32, vp, vp]
        lib.oracle_dense_causal_rows.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, vp, i64, vp, vp,
                                                 i32, vp, vp]
        lib.oracle_index_topk_qblock.argtypes = [cfgp, vp, i32, vp, i64, i64, i64, vp, vp]
        lib.oracle_sparse_attn_backward.argtypes = [cfgp, i32, i32, i64, vp, vp, vp, vp, vp, vp,
                                                    vp, i32, vp, vp, vp]
        lib.oracle_index_topk_qblocks.argtypes = [cfgp, i32, i64, vp, vp, vp, vp, i64, vp, vp,
                                                  i32, vp, vp]
        for f in (lib.oracle_sparse_attn_backward,
                  lib.oracle_index_topk_qblock, lib.oracle_index_topk_qblocks,
                  lib.oracle_index_pool_row, lib.oracle_index_pool_rows,
                  lib.oracle_index_topk_row, lib.oracle_sparse_attn_row,
                  lib.oracle_dense_causal_row, lib.oracle_index_topk_rows,
                  lib.oracle_sparse_attn_rows, lib.oracle_dense_causal_rows):
            f.restype = ctypes.c_int
        self.lib = lib

    # -- element decoders -------------------------------------------------
    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(bits)

    def e4m3_value(self, bits: int) -> float:
        return self.lib.oracle_e4m3_value(bits)

    # -- batched, row-listed calls ---------------------------------------
    @staticmethod
    def _rows(rows, B, T):
        if rows is None:
            bb, ii = np.meshgrid(np.arange(B, dtype=np.int32), np.arange(T, dtype=np.int32),
                                 indexing="ij")
            return bb.reshape(-1).copy(), ii.reshape(-1).copy()
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
        return np.ascontiguousarray(rows[:, 0]), np.ascontiguousarray(rows[:, 1])

    def index_topk(self, cfg: Config, q_idx, k_idx, kv_lens, q_start, rows=None, threads=None):
        """sel [n,G,K] int32 and pooled scores [n,G,K] float64 for the listed (b, i) rows."""
        q_idx = np.ascontiguousarray(q_idx)
        k_idx = np.ascontiguousarray(k_idx)
        B, T = q_idx.shape[0], q_idx.shape[1]
        n_stride = k_idx.shape[1]
        rb, ri = self._rows(rows, B, T)
        n = rb.size
        sel = np.empty((n, cfg.groups, cfg.topk), np.int32)
        scores = np.empty((n, cfg.groups, cfg.topk), np.float64)
        c = cfg.c()
        rc = self.lib.oracle_index_topk_rows(
            ctypes.byref(c), T, n_stride, _ptr(q_idx), _ptr(k_idx), _ptr(_c(kv_lens, np.int32)),
            _ptr(_c(q_start, np.int32)), n, _ptr(rb), _ptr(ri), threads or _threads(),
            _ptr(sel), _ptr(scores))
        if rc:
            raise ValueError("oracle_index_topk_rows rejected its arguments")
        return sel, scores

    def index_topk_qblock(self, cfg: Config, q_idx, k_idx, kv_lens, q_start, items=None,
                          threads=None):
        """Query-block-shared selection: sel [n,G,K] int32 and scores [n,G,K]
        float64 for the listed (b, slot) items (default: every slot of every
        sequence, slot = query block - q_start // S, qblock_slots(T, S) slots)."""
        q_idx = np.ascontiguousarray(q_idx)
        k_idx = np.ascontiguousarray(k_idx)
        B, T = q_idx.shape[0], q_idx.shape[1]
        n_stride = k_idx.shape[1]
        if items is None:
            nq = qblock_slots(T, cfg.block_size)
            ib, isl = self._rows(None, B, nq)
        else:
            ib, isl = self._rows(items, B, 1 << 30)
        n = ib.size
        sel = np.empty((n, cfg.groups, cfg.topk), np.int32)
        scores = np.empty((n, cfg.groups, cfg.topk), np.float64)
        c = cfg.c()
        rc = self.lib.oracle_index_topk_qblocks(
            ctypes.byref(c), T, n_stride, _ptr(q_idx), _ptr(k_idx), _ptr(_c(kv_lens, np.int32)),
            _ptr(_c(q_start, np.int32)), n, _ptr(ib), _ptr(isl), threads or _threads(),
            _ptr(sel), _ptr(scores))
        if rc:
            raise ValueError("oracle_index_topk_qblocks rejected its arguments")
        return sel, scores

    def index_pool(self, cfg: Config, q_idx, k_idx, kv_lens, q_start, rows=None, nb=None,
                   threads=None):
        """Pooled block scores [n,G,nb] float64 for the listed (b, i) rows; blocks
        past a row's position are -inf. nb defaults to ceil(n_stride / S)."""
        q_idx = np.ascontiguousarray(q_idx)
        k_idx = np.ascontiguousarray(k_idx)
        B, T = q_idx.shape[0], q_idx.shape[1]
        n_stride = k_idx.shape[1]
        nb = -(-n_stride // cfg.block_size) if nb is None else nb
        rb, ri = self._rows(rows, B, T)
        n = rb.size
        pooled = np.empty((n, cfg.groups, nb), np.float64)
        c = cfg.c()
        rc = self.lib.oracle_index_pool_rows(
            ctypes.byref(c), T, n_stride, _ptr(q_idx), _ptr(k_idx), _ptr(_c(kv_lens, np.int32)),
            _ptr(_c(q_start, np.int32)), n, _ptr(rb), _ptr(ri), threads or _threads(), nb,
            _ptr(pooled))
        if rc:
            raise ValueError("oracle_index_pool_rows rejected its arguments")
        return pooled

    def sparse_attn(self, cfg: Config, q, k_cache, v_cache, kv_lens, q_start, sel, rows=None,
                    threads=None):
        """out [n,H,d] float64 and lse [n,H] float64; sel is [n,G,K] for the listed rows."""
        q = _c(q, np.uint16)
        k_cache = _c(k_cache, np.uint16)
        v_cache = _c(v_cache, np.uint16)
        B, T = q.shape[0], q.shape[1]
        n_stride = k_cache.shape[2]
        rb, ri = self._rows(rows, B, T)
        n = rb.size
        sel = _c(sel, np.int32).reshape(n, cfg.groups, cfg.topk)
        H = cfg.groups * cfg.heads_per_group
        out = np.empty((n, H, cfg.head_dim), np.float64)
        lse = np.empty((n, H), np.float64)
        c = cfg.c()
        rc = self.lib.oracle_sparse_attn_rows(
            ctypes.byref(c), T, n_stride, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(_c(kv_lens, np.int32)), _ptr(_c(q_start, np.int32)), n, _ptr(rb), _ptr(ri),
            _ptr(sel), threads or _threads(), _ptr(out), _ptr(lse))
        if rc:
            raise ValueError("oracle_sparse_attn_rows rejected its arguments")
        return out, lse

    def sparse_attn_backward(self, cfg: Config, q, k_cache, v_cache, kv_lens, q_start, sel,
                             dout, threads=None):
        """Gradients of the sparse branch for fixed selections: dq [B,T,H,d],
        dk and dv [B,G,N,d] (float64) for sel [B,T,G,K] and the upstream
        gradient dout [B,T,H,d] (bf16 bits)."""
        q = _c(q, np.uint16)
        k_cache = _c(k_cache, np.uint16)
        v_cache = _c(v_cache, np.uint16)
        dout = _c(dout, np.uint16)
        B, T = q.shape[0], q.shape[1]
        n_stride = k_cache.shape[2]
        H = cfg.groups * cfg.heads_per_group
        sel = _c(sel, np.int32).reshape(B, T, cfg.groups, cfg.topk)
        dq = np.empty((B, T, H, cfg.head_dim), np.float64)
        dk = np.empty((B, cfg.groups, n_stride, cfg.head_dim), np.float64)
        dv = np.empty_like(dk)
        c = cfg.c()
        rc = self.lib.oracle_sparse_attn_backward(
            ctypes.byref(c), B, T, n_stride, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(_c(kv_lens, np.int32)), _ptr(_c(q_start, np.int32)), _ptr(sel), _ptr(dout),
            threads or _threads(), _ptr(dq), _ptr(dk), _ptr(dv))
        if rc:
            raise ValueError("oracle_sparse_attn_backward rejected its arguments")
        return dq, dk, dv

    def dense_causal(self, cfg: Config, q, k_cache, v_cache, kv_lens, q_start, rows=None,
                     threads=None):
        """Dense causal GQA attention: out [n,H,d], lse [n,H] (float64)."""
        q = _c(q, np.uint16)
        k_cache = _c(k_cache, np.uint16)
        v_cache = _c(v_cache, np.uint16)
        B, T = q.shape[0], q.shape[1]
        n_stride = k_cache.shape[2]
        rb, ri = self._rows(rows, B, T)
        n = rb.size
        H = cfg.groups * cfg.heads_per_group
        out = np.empty((n, H, cfg.head_dim), np.float64)
        lse = np.empty((n, H), np.float64)
        c = cfg.c()
        rc = self.lib.oracle_dense_causal_rows(
            ctypes.byref(c), T, n_stride, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(_c(kv_lens, np.int32)), _ptr(_c(q_start, np.int32)), n, _ptr(rb), _ptr(ri),
            threads or _threads(), _ptr(out), _ptr(lse))
        if rc:
            raise ValueError("oracle_dense_causal_rows rejected its arguments")
        return out, lse


def qblock_slots(T: int, S: int) -> int:
    """Query blocks that T consecutive positions can touch: ceil((T-1)/S) + 1."""
    return 0 if T <= 0 else (T - 1 + S - 1) // S + 1


def qblock_rows_sel(sel_blk, q_start, T, S, rows=None):
    """Per-row selections [n,G,K] from query-block selections [B,nslots,G,K]:
    row i of sequence b takes the selection of its block, slot
    (q_start[b] + i) // S - q_start[b] // S; rows default to every (b, i)."""
    sel_blk = np.asarray(sel_blk)
    q_start = np.asarray(q_start, np.int64)
    B = sel_blk.shape[0]
    rb, ri = Oracle._rows(rows, B, T)
    slots = (q_start[rb] + ri) // S - q_start[rb] // S
    return np.ascontiguousarray(sel_blk[rb, slots]).astype(np.int32)


def cache_append(k_new, v_new, k_idx_new, pos0, k_cache, v_cache, k_idx):
    """The caches after appending T new tokens per sequence (new arrays; the
    inputs are not modified). The decode step reads the new token's K, V and
    index key from the caches (Tencent article, section 二: the index query
    scores every cached key, the new one included), so each new row t of
    sequence b is stored at position pos0[b] + t; positions outside the cache
    [0, Nmax) are skipped. Shapes: k_new, v_new [B,T,G,d]; k_idx_new [B,T,dI];
    k_cache, v_cache [B,G,Nmax,d]; k_idx [B,Nmax,dI]; any element dtype (the
    bits are copied unchanged)."""
    k_cache, v_cache, k_idx = k_cache.copy(), v_cache.copy(), k_idx.copy()
    B, G, Nmax = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    T = k_new.shape[1]
    for b in range(B):
        for t in range(T):
            pos = int(pos0[b]) + t
            if pos < 0 or pos >= Nmax:
                continue
            for g in range(G):
                k_cache[b, g, pos, :] = k_new[b, t, g, :]
                v_cache[b, g, pos, :] = v_new[b, t, g, :]
            k_idx[b, pos, :] = k_idx_new[b, t, :]
    return k_cache, v_cache, k_idx


def _bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) as float64: the top half of an fp32."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _f64_to_bf16_bits(x) -> np.ndarray:
    """float64 values rounded once to bf16 (8 significant bits, nearest, ties
    to even) as bit patterns; the values here are finite and within the
    normal bf16 range."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # np.rint rounds ties to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def index_project(hidden, w, groups, index_dim=128):
    """Index projections, the step ahead of the index branch (Tencent article,
    section 二: one lightweight index query per GQA group from each token's
    hidden state; the index keys from the tokens the same way): with hidden
    [M, h] and w [(G+1)*dI, h] as bf16 bits, the exact sums
      q[m, g, c] = sum_k hidden[m, k] * w[g*dI + c, k]     (g < G)
      k[m, c]    = sum_k hidden[m, k] * w[G*dI + c, k]
    in float64 (a matmul), and the same rounded once to bf16 bits.
    Returns (q [M,G,dI] float64, k [M,dI] float64, q bits, k bits)."""
    h64 = _bf16_bits_to_f64(hidden)
    w64 = _bf16_bits_to_f64(w)
    G, dI = groups, index_dim
    if w64.shape != ((G + 1) * dI, h64.shape[-1]):
        raise ValueError("w must be [(G+1)*dI, h]")
    c = h64 @ w64.T                          # [M, (G+1)*dI]
    q = c[:, :G * dI].reshape(-1, G, dI)
    k = c[:, G * dI:]
    return q, k, _f64_to_bf16_bits(q), _f64_to_bf16_bits(k)


def _threads() -> int:
    return max(1, min(os.cpu_count() or 1, 64))


_default = None


def default() -> Oracle:
    """The oracle built from this directory's source."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
