"""Seeded synthetic inputs for MiniMax Sparse Attention workloads.

Input generation only: nothing here computes any part of the attention
method. The C source ``synth.c`` holds the generator (counter-based
SplitMix64, Box-Muller normals, uniform integers); this module loads it with
ctypes and fills numpy arrays or CPU torch tensors in place.

Both the CPU oracle and the GPU library read buffers filled here, so the two
sides see identical bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

# Workload seed base ("MSA" in ASCII, shifted) plus a small config id.
SEED_BASE = 0x4D5341000

# Tensor ids used to derive one independent stream per tensor of a workload.
TENSOR_IDS = {"q": 1, "k_cache": 2, "v_cache": 3, "q_idx": 4, "k_idx": 5}


def build(force: bool = True) -> str:
    """Compiles synth.c into libsynth.so next to it (gcc, -O2, pthreads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, sz, i32, vp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [vp, sz, u64, u64, i32]
        lib.synth_int_bf16.argtypes = [vp, sz, u64, u64, i32, i32, i32]
        lib.synth_int_e4m3.argtypes = [vp, sz, u64, u64, i32, i32, i32]
        for f in (lib.synth_normal_bf16, lib.synth_int_bf16, lib.synth_int_e4m3):
            f.restype = i32
        lib.synth_stream_seed.argtypes = [u64, u64]
        lib.synth_stream_seed.restype = u64
        _lib = lib
    return _lib


def _addr_and_count(buf, itemsize):
    if isinstance(buf, np.ndarray):
        if not buf.flags["C_CONTIGUOUS"] or buf.dtype.itemsize != itemsize:
            raise ValueError("need a C-contiguous array of %d-byte elements" % itemsize)
        return buf.ctypes.data, buf.size
    # torch tensor (duck-typed so this module does not import torch)
    if getattr(buf, "is_cuda", False) or not buf.is_contiguous():
        raise ValueError("need a contiguous CPU tensor")
    if buf.element_size() != itemsize:
        raise ValueError("need %d-byte elements" % itemsize)
    return buf.data_ptr(), buf.numel()


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def stream_seed(config_id: int, tensor: str) -> int:
    """Seed of one tensor's stream in workload `config_id`."""
    return int(_load().synth_stream_seed(SEED_BASE + int(config_id), TENSOR_IDS[tensor]))


def fill_normal_bf16(buf, seed: int, offset: int = 0, threads: int | None = None):
    """Fills a 2-byte buffer with N(0,1) samples rounded to bfloat16 bits."""
    addr, n = _addr_and_count(buf, 2)
    rc = _load().synth_normal_bf16(addr, n, seed, offset, threads or default_threads())
    if rc:
        raise RuntimeError("synth_normal_bf16 failed")
    return buf


def fill_int_bf16(buf, seed: int, lo: int = -4, hi: int = 4, offset: int = 0,
                  threads: int | None = None):
    """Fills a 2-byte buffer with uniform integers in [lo, hi] as exact bfloat16 bits."""
    addr, n = _addr_and_count(buf, 2)
    rc = _load().synth_int_bf16(addr, n, seed, offset, lo, hi, threads or default_threads())
    if rc:
        raise RuntimeError("synth_int_bf16 failed")
    return buf


def fill_int_e4m3(buf, seed: int, lo: int = -4, hi: int = 4, offset: int = 0,
                  threads: int | None = None):
    """Fills a 1-byte buffer with uniform integers in [lo, hi] as exact FP8 E4M3FN bits."""
    addr, n = _addr_and_count(buf, 1)
    rc = _load().synth_int_e4m3(addr, n, seed, offset, lo, hi, threads or default_threads())
    if rc:
        raise RuntimeError("synth_int_e4m3 failed")
    return buf


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widens bfloat16 bit patterns (uint16) to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Rounds float32 values to bfloat16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
