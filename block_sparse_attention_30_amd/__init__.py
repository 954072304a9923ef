"""Python binding of libmsa (MiniMax Sparse Attention on gfx950).

Argument marshalling only: every step of the method runs in the HIP kernels
of libmsa.so, called through its C ABI (include/msa.h) with ctypes. PyTorch
supplies device memory and the current HIP stream. There is no CPU fallback:
if libmsa.so is missing or a call fails, an exception is raised.

Names follow the pages' sparse_attention_config (sparse_index_dim,
sparse_num_index_heads, sparse_topk_blocks, sparse_block_size).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = ["Config", "MsaError", "index_topk", "sparse_attn_prefill", "sparse_attn_decode",
           "workspace_size", "workspace", "library_path", "load", "BF16", "FP8_E4M3",
           "WS_INDEX_TOPK", "WS_SPARSE_PREFILL", "WS_SPARSE_DECODE", "WS_DECODE", "decode"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmsa.so")

BF16, FP8_E4M3 = 0, 1
WS_INDEX_TOPK, WS_SPARSE_PREFILL, WS_SPARSE_DECODE, WS_DECODE, WS_SPARSE_BACKWARD = 0, 1, 2, 3, 4
_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED",
           3: "MSA_ERR_WORKSPACE", 4: "MSA_ERR_HIP"}


class MsaError(RuntimeError):
    """A libmsa call returned a non-zero msa_status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s: %s" % (_STATUS.get(status, status), detail))


class _CConfig(ctypes.Structure):
    _fields_ = [("num_kv_groups", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("index_dtype", ctypes.c_int32)]


@dataclass(frozen=True)
class Config:
    """One MSA layer's shapes (msa_config)."""
    num_kv_groups: int = 4        # G = KV heads = sparse_num_index_heads
    heads_per_group: int = 8      # R
    head_dim: int = 128           # d
    index_dim: int = 128          # sparse_index_dim
    block_size: int = 128         # sparse_block_size
    topk: int = 16                # sparse_topk_blocks
    softmax_scale: float = 0.0    # 0: 1/sqrt(head_dim)
    index_dtype: int = BF16

    @property
    def num_heads(self) -> int:
        return self.num_kv_groups * self.heads_per_group

    def _c(self) -> _CConfig:
        c = _CCONFIGS.get(self)
        if c is None:
            c = _CConfig(self.num_kv_groups, self.heads_per_group, self.head_dim, self.index_dim,
                         self.block_size, self.topk, float(self.softmax_scale), self.index_dtype)
            _CCONFIGS[self] = c
        return c


_CCONFIGS = {}


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Loads libmsa.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libmsa.so is not built; run block_sparse_attention_30_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(_CConfig)
    lib.msa_index_topk.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_index_pool.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.msa_sparse_attn_prefill.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
    lib.msa_sparse_attn_decode.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_decode.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_decode_no_alloc.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp]
    lib.msa_decode_no_alloc.restype = ctypes.c_int
    lib.msa_decode_no_alloc_max_scratch.argtypes = []
    lib.msa_decode_no_alloc_max_scratch.restype = sz
    lib.msa_cache_append.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_index_topk_qblock.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_sparse_attn_prefill_qblock.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                                   vp, vp, vp]
    lib.msa_sparse_attn_backward.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_backward.restype = ctypes.c_int
    lib.msa_index_project.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp]
    lib.msa_index_project.restype = ctypes.c_int
    lib.msa_qblock_slots.argtypes = [i32]
    lib.msa_qblock_slots.restype = i32
    for f in (lib.msa_index_topk, lib.msa_index_pool, lib.msa_sparse_attn_prefill,
              lib.msa_sparse_attn_decode, lib.msa_decode, lib.msa_cache_append,
              lib.msa_index_topk_qblock, lib.msa_sparse_attn_prefill_qblock):
        f.restype = ctypes.c_int
    lib.msa_workspace_size.argtypes = [cfgp, i32, i32, i32, i32]
    lib.msa_workspace_size.restype = sz
    lib.msa_status_string.argtypes = [ctypes.c_int]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MsaError(status, load().msa_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _on_device:
    """Makes `dev` the current device for a call (a no-op when it already is)."""

    def __init__(self, dev):
        self.dev = dev
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if self.dev.index is not None and cur != self.dev.index:
            self.prev = cur
            torch.cuda.set_device(self.dev.index)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def _need(t, name, dtypes, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU (libmsa has no CPU path)" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, has %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


_INDEX_DTYPES = {BF16: (torch.bfloat16,), FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}


def workspace(cfg: Config, B: int, T: int, Nmax: int, which: int, device="cuda"):
    """A workspace for the named call: plain scratch (no initialisation needed),
    reusable by later calls on the same stream whose size fits in it."""
    return torch.empty(max(workspace_size(cfg, B, T, Nmax, which), 256), dtype=torch.uint8,
                       device=device)


def workspace_size(cfg: Config, B: int, T: int, Nmax: int, which: int) -> int:
    n = load().msa_workspace_size(ctypes.byref(cfg._c()), B, T, Nmax, which)
    if n == ctypes.c_size_t(-1).value:
        raise MsaError(1, load().msa_last_error().decode(errors="replace") or "invalid config")
    return int(n)


def _workspace(cfg, B, T, Nmax, which, device, workspace):
    need = workspace_size(cfg, B, T, Nmax, which)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _lens(t, name, B, device):
    _need(t, name, (torch.int32,), 1, device)
    if t.shape[0] != B:
        raise ValueError("%s must have B = %d entries" % (name, B))


def index_topk(cfg: Config, q_idx, k_idx, kv_lens, q_start=None, sel=None, sel_scores=None,
               want_scores: bool = False, workspace=None):
    """Index branch: sel [B,T,G,K] int32 (and pooled scores [B,T,G,K] fp32).

    q_idx [B,T,G,dI] and k_idx [B,Nmax,dI] are bf16 (or float8_e4m3fn / uint8
    E4M3FN bits when cfg.index_dtype == FP8_E4M3); kv_lens [B] int32;
    q_start [B] int32 or None (then q_start = kv_lens - T).
    """
    dev = q_idx.device
    _need(q_idx, "q_idx", _INDEX_DTYPES[cfg.index_dtype], 4)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    B, T, G, dI = q_idx.shape
    Nmax = k_idx.shape[1]
    if G != cfg.num_kv_groups or dI != cfg.index_dim or k_idx.shape[0] != B or \
            k_idx.shape[2] != cfg.index_dim:
        raise ValueError("q_idx/k_idx shapes do not match the config")
    _lens(kv_lens, "kv_lens", B, dev)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    if sel is None:
        sel = torch.empty((B, T, G, cfg.topk), dtype=torch.int32, device=dev)
    _need(sel, "sel", (torch.int32,), 4, dev)
    if tuple(sel.shape) != (B, T, G, cfg.topk):
        raise ValueError("sel must be [B,T,G,K]")
    if want_scores and sel_scores is None:
        sel_scores = torch.empty((B, T, G, cfg.topk), dtype=torch.float32, device=dev)
    if sel_scores is not None:
        _need(sel_scores, "sel_scores", (torch.float32,), 4, dev)
        if sel_scores.shape != sel.shape:
            raise ValueError("sel_scores must be [B,T,G,K]")
    ws, nws = _workspace(cfg, B, T, Nmax, WS_INDEX_TOPK, dev, workspace)
    with _on_device(dev):
        _check(load().msa_index_topk(ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q_idx),
                                     _ptr(k_idx), _ptr(kv_lens), _ptr(q_start), _ptr(sel),
                                     _ptr(sel_scores), _ptr(ws), nws, _stream(dev)))
    return (sel, sel_scores) if (want_scores or sel_scores is not None) else sel


def index_pool(cfg: Config, q_idx, k_idx, kv_lens, q_start=None, pooled=None):
    """Index scores max-pooled per block: pooled [B,T,G,ceil(Nmax/S)] fp32.

    Entries past a row's position (and rows outside the cache) are left as
    they were; a new `pooled` starts filled with -inf.
    """
    dev = q_idx.device
    _need(q_idx, "q_idx", _INDEX_DTYPES[cfg.index_dtype], 4)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    B, T, G, dI = q_idx.shape
    Nmax = k_idx.shape[1]
    if G != cfg.num_kv_groups or dI != cfg.index_dim or k_idx.shape[0] != B or \
            k_idx.shape[2] != cfg.index_dim:
        raise ValueError("q_idx/k_idx shapes do not match the config")
    _lens(kv_lens, "kv_lens", B, dev)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    nbm = -(-Nmax // cfg.block_size)
    if pooled is None:
        pooled = torch.full((B, T, G, nbm), float("-inf"), dtype=torch.float32, device=dev)
    _need(pooled, "pooled", (torch.float32,), 4, dev)
    if tuple(pooled.shape) != (B, T, G, nbm):
        raise ValueError("pooled must be [B,T,G,ceil(Nmax/S)]")
    with _on_device(dev):
        _check(load().msa_index_pool(ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q_idx),
                                     _ptr(k_idx), _ptr(kv_lens), _ptr(q_start), _ptr(pooled),
                                     _stream(dev)))
    return pooled


def _sparse_checks(cfg, q, k_cache, v_cache, kv_lens, sel, T_expected=None):
    dev = q.device
    _need(q, "q", (torch.bfloat16,), 4)
    _need(k_cache, "k_cache", (torch.bfloat16,), 4, dev)
    _need(v_cache, "v_cache", (torch.bfloat16,), 4, dev)
    B, T, H, d = q.shape
    if T_expected is not None and T != T_expected:
        raise ValueError("q must have T = %d" % T_expected)
    if H != cfg.num_heads or d != cfg.head_dim:
        raise ValueError("q must be [B,T,G*R,d]")
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or \
            k_cache.shape[1] != cfg.num_kv_groups or k_cache.shape[3] != cfg.head_dim:
        raise ValueError("k_cache / v_cache must both be [B,G,Nmax,d]")
    _lens(kv_lens, "kv_lens", B, dev)
    _need(sel, "sel", (torch.int32,), 4, dev)
    if tuple(sel.shape) != (B, T, cfg.num_kv_groups, cfg.topk):
        raise ValueError("sel must be [B,T,G,K]")
    return dev, B, T, k_cache.shape[2]


def _outputs(cfg, dev, B, T, out, lse, want_lse):
    if out is None:
        out = torch.empty((B, T, cfg.num_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    _need(out, "out", (torch.bfloat16,), 4, dev)
    if tuple(out.shape) != (B, T, cfg.num_heads, cfg.head_dim):
        raise ValueError("out must be [B,T,H,d]")
    if want_lse and lse is None:
        lse = torch.empty((B, T, cfg.num_heads), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), 3, dev)
        if tuple(lse.shape) != (B, T, cfg.num_heads):
            raise ValueError("lse must be [B,T,H]")
    return out, lse


def sparse_attn_prefill(cfg: Config, q, k_cache, v_cache, kv_lens, sel, q_start=None, out=None,
                        lse=None, want_lse: bool = False, workspace=None):
    """Sparse branch for T rows per sequence: out [B,T,H,d] bf16 (and lse [B,T,H])."""
    dev, B, T, Nmax = _sparse_checks(cfg, q, k_cache, v_cache, kv_lens, sel)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    out, lse = _outputs(cfg, dev, B, T, out, lse, want_lse)
    ws, nws = _workspace(cfg, B, T, Nmax, WS_SPARSE_PREFILL, dev, workspace)
    with _on_device(dev):
        _check(load().msa_sparse_attn_prefill(
            ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(kv_lens), _ptr(q_start), _ptr(sel), _ptr(out), _ptr(lse), _ptr(ws), nws,
            _stream(dev)))
    return (out, lse) if (want_lse or lse is not None) else out


def sparse_attn_decode(cfg: Config, q, k_cache, v_cache, kv_lens, sel, out=None, lse=None,
                       want_lse: bool = False, workspace=None):
    """Sparse branch for one new token per sequence (q [B,1,H,d], position kv_lens-1)."""
    dev, B, T, Nmax = _sparse_checks(cfg, q, k_cache, v_cache, kv_lens, sel, T_expected=1)
    out, lse = _outputs(cfg, dev, B, 1, out, lse, want_lse)
    ws, nws = _workspace(cfg, B, 1, Nmax, WS_SPARSE_DECODE, dev, workspace)
    with _on_device(dev):
        _check(load().msa_sparse_attn_decode(
            ctypes.byref(cfg._c()), B, Nmax, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(kv_lens), _ptr(sel), _ptr(out), _ptr(lse), _ptr(ws), nws, _stream(dev)))
    return (out, lse) if (want_lse or lse is not None) else out


def decode(cfg: Config, q, q_idx, k_idx, k_cache, v_cache, kv_lens, sel=None, sel_scores=None,
           out=None, lse=None, want_scores: bool = False, want_lse: bool = False,
           workspace=None):
    """One decode step in a single launch: index top-k and sparse attention for
    the token at position kv_lens - 1. Returns (sel, out) plus sel_scores / lse
    when requested, as (sel, sel_scores, out, lse) in that case."""
    dev, B, T, Nmax = _sparse_checks(cfg, q, k_cache, v_cache, kv_lens,
                                     sel if sel is not None else torch.empty(
                                         (q.shape[0], 1, cfg.num_kv_groups, cfg.topk),
                                         dtype=torch.int32, device=q.device), T_expected=1)
    _need(q_idx, "q_idx", _INDEX_DTYPES[cfg.index_dtype], 4, dev)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    if tuple(q_idx.shape) != (B, 1, cfg.num_kv_groups, cfg.index_dim) or \
            tuple(k_idx.shape) != (B, Nmax, cfg.index_dim):
        raise ValueError("q_idx must be [B,1,G,dI] and k_idx [B,Nmax,dI]")
    if sel is None:
        sel = torch.empty((B, 1, cfg.num_kv_groups, cfg.topk), dtype=torch.int32, device=dev)
    if want_scores and sel_scores is None:
        sel_scores = torch.empty(sel.shape, dtype=torch.float32, device=dev)
    if sel_scores is not None:
        _need(sel_scores, "sel_scores", (torch.float32,), 4, dev)
        if sel_scores.shape != sel.shape:
            raise ValueError("sel_scores must be [B,1,G,K]")
    out, lse = _outputs(cfg, dev, B, 1, out, lse, want_lse)
    ws, nws = _workspace(cfg, B, 1, Nmax, WS_DECODE, dev, workspace)
    with _on_device(dev):
        _check(load().msa_decode(ctypes.byref(cfg._c()), B, Nmax, _ptr(q), _ptr(q_idx),
                                 _ptr(k_idx), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens),
                                 _ptr(sel), _ptr(sel_scores), _ptr(out), _ptr(lse), _ptr(ws),
                                 nws, _stream(dev)))
    if want_scores or want_lse or sel_scores is not None or lse is not None:
        return sel, sel_scores, out, lse
    return sel, out


def decode_no_alloc(cfg: Config, q, q_idx, k_idx, k_cache, v_cache, kv_lens, sel, out,
                    sel_scores=None, lse=None):
    """msa_decode_no_alloc: the decode step of `decode` with the library's fixed
    scratch array instead of a workspace. The outputs are the caller's (sel
    [B,1,G,K] int32, out [B,1,H,d] bf16, optional sel_scores and lse), so the
    call allocates nothing on the device."""
    dev, B, T, Nmax = _sparse_checks(cfg, q, k_cache, v_cache, kv_lens, sel, T_expected=1)
    _need(q_idx, "q_idx", _INDEX_DTYPES[cfg.index_dtype], 4, dev)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    if tuple(q_idx.shape) != (B, 1, cfg.num_kv_groups, cfg.index_dim) or \
            tuple(k_idx.shape) != (B, Nmax, cfg.index_dim):
        raise ValueError("q_idx must be [B,1,G,dI] and k_idx [B,Nmax,dI]")
    _need(out, "out", (torch.bfloat16,), 4, dev)
    if tuple(out.shape) != (B, 1, cfg.num_heads, cfg.head_dim):
        raise ValueError("out must be [B,1,H,d]")
    if sel_scores is not None:
        _need(sel_scores, "sel_scores", (torch.float32,), 4, dev)
        if sel_scores.shape != sel.shape:
            raise ValueError("sel_scores must be [B,1,G,K]")
    if lse is not None:
        _need(lse, "lse", (torch.float32,), 3, dev)
        if tuple(lse.shape) != (B, 1, cfg.num_heads):
            raise ValueError("lse must be [B,1,H]")
    with _on_device(dev):
        _check(load().msa_decode_no_alloc(ctypes.byref(cfg._c()), B, Nmax, _ptr(q), _ptr(q_idx),
                                          _ptr(k_idx), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(kv_lens), _ptr(sel), _ptr(sel_scores), _ptr(out),
                                          _ptr(lse), _stream(dev)))
    return sel, out


def decode_no_alloc_max_scratch() -> int:
    """Bytes of msa_decode_no_alloc's fixed scratch array (per GPU)."""
    return int(load().msa_decode_no_alloc_max_scratch())


def cache_append(cfg: Config, k_new, v_new, k_idx_new, pos0, k_cache, v_cache, k_idx):
    """Writes T new tokens per sequence into the caches, in place: row t of
    sequence b goes to position pos0[b] + t (rows outside [0, Nmax) are
    skipped). k_new, v_new [B,T,G,d] bf16; k_idx_new [B,T,dI] in the index
    dtype; pos0 [B] int32; k_cache, v_cache [B,G,Nmax,d]; k_idx [B,Nmax,dI]."""
    dev = k_cache.device
    _need(k_new, "k_new", (torch.bfloat16,), 4, dev)
    _need(v_new, "v_new", (torch.bfloat16,), 4, dev)
    _need(k_idx_new, "k_idx_new", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    _need(k_cache, "k_cache", (torch.bfloat16,), 4, dev)
    _need(v_cache, "v_cache", (torch.bfloat16,), 4, dev)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    B, G, Nmax, d = k_cache.shape
    T = k_new.shape[1]
    if G != cfg.num_kv_groups or d != cfg.head_dim or tuple(v_cache.shape) != (B, G, Nmax, d):
        raise ValueError("k_cache/v_cache must be [B,G,Nmax,d] for the config")
    if tuple(k_new.shape) != (B, T, G, d) or tuple(v_new.shape) != (B, T, G, d):
        raise ValueError("k_new/v_new must be [B,T,G,d]")
    if tuple(k_idx.shape) != (B, Nmax, cfg.index_dim) or \
            tuple(k_idx_new.shape) != (B, T, cfg.index_dim):
        raise ValueError("k_idx must be [B,Nmax,dI] and k_idx_new [B,T,dI]")
    _lens(pos0, "pos0", B, dev)
    with _on_device(dev):
        _check(load().msa_cache_append(ctypes.byref(cfg._c()), B, T, Nmax, _ptr(k_new),
                                       _ptr(v_new), _ptr(k_idx_new), _ptr(pos0), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(k_idx), _stream(dev)))


def index_project(cfg: Config, hidden, w, q_idx=None, k_idx=None, want_keys: bool = True):
    """Index projections (msa_index_project): hidden [..., h] bf16 (M rows in
    all) and w [(G+1)*dI, h] bf16 give q_idx [..., G, dI] and, with
    want_keys, k_idx [..., dI] (bf16). Returns (q_idx, k_idx or None)."""
    if not isinstance(hidden, torch.Tensor) or not hidden.is_cuda:
        raise ValueError("hidden must be a GPU tensor (libmsa has no CPU path)")
    dev = hidden.device
    _need(w, "w", (torch.bfloat16,), 2, dev)
    if hidden.dtype != torch.bfloat16 or not hidden.is_contiguous() or hidden.dim() < 1:
        raise ValueError("hidden must be a contiguous bf16 tensor [..., h]")
    h = hidden.shape[-1]
    lead = tuple(hidden.shape[:-1])
    M = 1
    for n in lead:
        M *= n
    G, dI = cfg.num_kv_groups, cfg.index_dim
    if tuple(w.shape) != ((G + 1) * dI, h):
        raise ValueError("w must be [(G+1)*dI, h] = %s" % (((G + 1) * dI, h),))
    if q_idx is None:
        q_idx = torch.empty(lead + (G, dI), dtype=torch.bfloat16, device=dev)
    if want_keys and k_idx is None:
        k_idx = torch.empty(lead + (dI,), dtype=torch.bfloat16, device=dev)
    if q_idx.dtype != torch.bfloat16 or not q_idx.is_contiguous() or \
            tuple(q_idx.shape) != lead + (G, dI) or q_idx.device != dev:
        raise ValueError("q_idx must be a contiguous bf16 tensor %s" % (lead + (G, dI),))
    if k_idx is not None and (k_idx.dtype != torch.bfloat16 or not k_idx.is_contiguous() or
                              tuple(k_idx.shape) != lead + (dI,) or k_idx.device != dev):
        raise ValueError("k_idx must be a contiguous bf16 tensor %s" % (lead + (dI,),))
    with _on_device(dev):
        _check(load().msa_index_project(ctypes.byref(cfg._c()), M, h, _ptr(hidden), _ptr(w),
                                        _ptr(q_idx), _ptr(k_idx), _stream(dev)))
    return q_idx, k_idx


def qblock_slots(T: int) -> int:
    """Query-block slots of a call with T rows per sequence (msa_qblock_slots)."""
    return int(load().msa_qblock_slots(T))


def index_topk_qblock(cfg: Config, q_idx, k_idx, kv_lens, q_start=None, sel=None,
                      sel_scores=None, want_scores: bool = False):
    """Query-block-shared selection: sel [B, NQ, G, K] int32 (and scores),
    NQ = qblock_slots(T); slot s is query block q_start // S + s."""
    dev = q_idx.device
    _need(q_idx, "q_idx", _INDEX_DTYPES[cfg.index_dtype], 4)
    _need(k_idx, "k_idx", _INDEX_DTYPES[cfg.index_dtype], 3, dev)
    B, T, G, dI = q_idx.shape
    Nmax = k_idx.shape[1]
    if G != cfg.num_kv_groups or dI != cfg.index_dim or k_idx.shape[0] != B or \
            k_idx.shape[2] != cfg.index_dim:
        raise ValueError("q_idx/k_idx shapes do not match the config")
    _lens(kv_lens, "kv_lens", B, dev)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    shape = (B, qblock_slots(T), G, cfg.topk)
    if sel is None:
        sel = torch.empty(shape, dtype=torch.int32, device=dev)
    _need(sel, "sel", (torch.int32,), 4, dev)
    if tuple(sel.shape) != shape:
        raise ValueError("sel must be [B, NQ, G, K]")
    if want_scores and sel_scores is None:
        sel_scores = torch.empty(shape, dtype=torch.float32, device=dev)
    if sel_scores is not None:
        _need(sel_scores, "sel_scores", (torch.float32,), 4, dev)
        if tuple(sel_scores.shape) != shape:
            raise ValueError("sel_scores must be [B, NQ, G, K]")
    with _on_device(dev):
        _check(load().msa_index_topk_qblock(ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q_idx),
                                            _ptr(k_idx), _ptr(kv_lens), _ptr(q_start), _ptr(sel),
                                            _ptr(sel_scores), _stream(dev)))
    return (sel, sel_scores) if (want_scores or sel_scores is not None) else sel


def sparse_attn_prefill_qblock(cfg: Config, q, k_cache, v_cache, kv_lens, sel, q_start=None,
                               out=None, lse=None, want_lse: bool = False):
    """Sparse branch with query-block-shared selections sel [B, NQ, G, K]."""
    dev = q.device
    _need(q, "q", (torch.bfloat16,), 4)
    _need(k_cache, "k_cache", (torch.bfloat16,), 4, dev)
    _need(v_cache, "v_cache", (torch.bfloat16,), 4, dev)
    B, T, H, d = q.shape
    Nmax = k_cache.shape[2]
    G = cfg.num_kv_groups
    if H != cfg.num_heads or d != cfg.head_dim or tuple(k_cache.shape) != (B, G, Nmax, d) or \
            tuple(v_cache.shape) != (B, G, Nmax, d):
        raise ValueError("q/k_cache/v_cache shapes do not match the config")
    _lens(kv_lens, "kv_lens", B, dev)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    _need(sel, "sel", (torch.int32,), 4, dev)
    if tuple(sel.shape) != (B, qblock_slots(T), G, cfg.topk):
        raise ValueError("sel must be [B, NQ, G, K]")
    out, lse = _outputs(cfg, dev, B, T, out, lse, want_lse)
    with _on_device(dev):
        _check(load().msa_sparse_attn_prefill_qblock(
            ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(kv_lens), _ptr(q_start), _ptr(sel), _ptr(out), _ptr(lse), _stream(dev)))
    return (out, lse) if (want_lse or lse is not None) else out


def sparse_attn_backward(cfg: Config, q, k_cache, v_cache, kv_lens, sel, out, lse, dout,
                         q_start=None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of the sparse branch for fixed selections: (dq [B,T,H,d],
    dk [B,G,Nmax,d], dv [B,G,Nmax,d]) in float32, from the forward's out and
    lse and the upstream gradient dout [B,T,H,d] bf16."""
    dev, B, T, Nmax = _sparse_checks(cfg, q, k_cache, v_cache, kv_lens, sel)
    if q_start is not None:
        _lens(q_start, "q_start", B, dev)
    H, d, G = cfg.num_heads, cfg.head_dim, cfg.num_kv_groups
    _need(out, "out", (torch.bfloat16,), 4, dev)
    _need(dout, "dout", (torch.bfloat16,), 4, dev)
    _need(lse, "lse", (torch.float32,), 3, dev)
    if tuple(out.shape) != (B, T, H, d) or tuple(dout.shape) != (B, T, H, d) or \
            tuple(lse.shape) != (B, T, H):
        raise ValueError("out/dout must be [B,T,H,d] and lse [B,T,H]")
    if dq is None:
        dq = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((B, G, Nmax, d), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, G, Nmax, d), dtype=torch.float32, device=dev)
    for t_, name, shp in ((dq, "dq", (B, T, H, d)), (dk, "dk", (B, G, Nmax, d)),
                          (dv, "dv", (B, G, Nmax, d))):
        _need(t_, name, (torch.float32,), 4, dev)
        if tuple(t_.shape) != shp:
            raise ValueError("%s must be %s" % (name, shp))
    ws, nws = _workspace(cfg, B, T, Nmax, WS_SPARSE_BACKWARD, dev, workspace)
    with _on_device(dev):
        _check(load().msa_sparse_attn_backward(
            ctypes.byref(cfg._c()), B, T, Nmax, _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(kv_lens), _ptr(q_start), _ptr(sel), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(ws), nws, _stream(dev)))
    return dq, dk, dv
