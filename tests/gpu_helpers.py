"""Shared pieces of the GPU parity tests: moving seeded host inputs to the GPU,
running the library through its C ABI, and comparing with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_attention_30_amd as msa
import oracle
from msa_synth import workloads as wl

# Acceptance: selection bit-exact; outputs within these bounds (fp32 softmax,
# bf16 operands and bf16 output rounding against an fp64 definition).
MAX_ABS = 2e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev_index(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda().view(torch.float8_e4m3fn)
    return dev_bf16(a)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def lib_cfg(G, R, K, fp8=False, scale=0.0):
    return msa.Config(num_kv_groups=G, heads_per_group=R, topk=K, softmax_scale=scale,
                      index_dtype=msa.FP8_E4M3 if fp8 else msa.BF16)


def oracle_cfg(G, R, K, fp8=False, scale=0.0):
    return oracle.Config(groups=G, heads_per_group=R, topk=K, softmax_scale=scale,
                         index_dtype=oracle.E4M3 if fp8 else oracle.BF16)


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def compare_out(got: np.ndarray, want: np.ndarray, what: str):
    """Max-abs and relative-L2 bounds over the checked rows."""
    diff = np.abs(got - want)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say("%s: max_abs=%.3e rel_l2=%.3e" % (what, max_abs, rel))
    assert max_abs <= MAX_ABS, (what, max_abs)
    assert rel <= REL_L2, (what, rel)
    return max_abs, rel


def compare_lse(got: np.ndarray, want: np.ndarray, what: str):
    finite = np.isfinite(want)
    assert np.array_equal(finite, np.isfinite(got)), what
    d = float(np.abs(got[finite] - want[finite]).max()) if finite.any() else 0.0
    say("%s: lse max_abs=%.3e" % (what, d))
    assert d <= LSE_ABS, (what, d)


def host_problem(w: wl.Workload, row0=0, rows=None, set_id=0):
    k, v, ki = wl.gen_caches(w)
    q, qi = wl.gen_queries(w, row0=row0, rows=rows, set_id=set_id)
    return dict(k=k, v=v, ki=ki, q=q, qi=qi)


def sample_rows(B, T, picks):
    return np.array([(b, i) for b in range(B) for i in picks if 0 <= i < T], np.int32)
