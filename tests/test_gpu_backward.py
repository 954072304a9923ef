"""GPU parity of msa_sparse_attn_backward (through the C ABI) against the
oracle's fp64 gradients of the sparse branch for fixed selections: dq on
every row, dk and dv on every cached key, within the backward tolerances:
relative L2 <= 1e-2 and max-abs <= 1e-2 * max|reference| (the kernels round P
and dS to bf16 before their MFMA sums, 2^-9 relative each, round each slot's
dq partial to bf16 before the fp32 sum over the row's slots, and form
dout.out from the bf16 forward output, which dS = P (dP - dout.out) can
amplify where dP and dout.out nearly cancel)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
from gpu_helpers import dev_bf16, dev_i32, dev_index, lib_cfg, oracle_cfg, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

REL_L2 = 1e-2
MAX_REL = 1e-2


def compare(got, want, what):
    got = np.asarray(got, np.float64)
    scale = float(np.abs(want).max()) if want.size else 0.0
    err = float(np.abs(got - want).max()) if want.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say("%s: max_abs=%.3e (ref max %.3e) rel_l2=%.3e" % (what, err, scale, rel))
    assert rel <= REL_L2, (what, rel)
    assert err <= MAX_REL * max(scale, 1e-30), (what, err, scale)


def run(orc, B, T, N, G, R, K, kv_lens, q_start, seed):
    H = G * R
    q = ms.fill_normal_bf16(np.empty((B, T, H, 128), np.uint16), seed + 1)
    k = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 2)
    v = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 3)
    qi = ms.fill_int_bf16(np.empty((B, T, G, 128), np.uint16), seed + 4, -4, 4)
    ki = ms.fill_int_bf16(np.empty((B, N, 128), np.uint16), seed + 5, -4, 4)
    do = ms.fill_normal_bf16(np.empty((B, T, H, 128), np.uint16), seed + 6)
    kv_lens = np.asarray(kv_lens, np.int32)
    q_start = np.asarray(q_start, np.int32)
    cfg = lib_cfg(G, R, K)
    kv, qs = dev_i32(kv_lens), dev_i32(q_start)
    dq_, dk_, dv_ = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("forward B=%d T=%d N=%d G=%d R=%d K=%d" % (B, T, N, G, R, K))
    sel = msa.index_topk(cfg, dev_index(qi), dev_index(ki), kv, qs)
    out, lse = msa.sparse_attn_prefill(cfg, dq_, dk_, dv_, kv, sel, q_start=qs, want_lse=True)
    say("backward")
    gq, gk, gv = msa.sparse_attn_backward(cfg, dq_, dk_, dv_, kv, sel, out, lse, dev_bf16(do),
                                          q_start=qs)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    say("oracle backward")
    oq, ok_, ov = orc.sparse_attn_backward(oracle_cfg(G, R, K), q, k, v, kv_lens, q_start, sel_h,
                                           do, threads=16)
    compare(gq.cpu().numpy(), oq, "dq")
    compare(gk.cpu().numpy(), ok_, "dk")
    compare(gv.cpu().numpy(), ov, "dv")
    # Keys no row attends to, and positions past each cache, are exactly zero.
    zk = ok_ == 0
    assert not gk.cpu().numpy()[zk].any() and not gv.cpu().numpy()[ov == 0].any()


def test_backward_prefill(orc):
    run(orc, 1, 1000, 1000, 2, 4, 4, [1000], [0], seed=800)


def test_backward_chunk_ragged_and_rows_outside(orc):
    # sequence 0: chunk of a longer cache; sequence 1: cache ends inside the chunk
    run(orc, 2, 300, 1500, 2, 8, 8, [1400, 1200], [1100, 1000], seed=810)


def test_backward_two_passes(orc):
    # 16 groups x 16 heads, 32 slots: 2048 rows per pass, so two passes
    run(orc, 1, 2100, 2100, 16, 16, 32, [2100], [0], seed=820)


def test_backward_short_context_odd_heads(orc):
    run(orc, 1, 257, 257, 3, 5, 16, [257], [0], seed=830)


@pytest.mark.parametrize("G,R", [(1, 2), (3, 1)])
def test_backward_one_and_two_heads_per_group(orc, G, R):
    # one-wave dq merge workgroups (R * D / 4 <= 64 threads)
    run(orc, 1, 700, 700, G, R, 16, [700], [0], seed=840 + R)


def test_backward_bitwise_repeatable():
    # 4096 rows over 32 blocks: most lists span several tiles, so dk and dv
    # are sums over many tiles; two calls must agree bit for bit (the lists
    # keep row order, no floating-point atomics).
    B, T, N, G, R, K = 1, 4096, 4096, 2, 8, 16
    seed = 840
    H = G * R
    q = ms.fill_normal_bf16(np.empty((B, T, H, 128), np.uint16), seed + 1)
    k = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 2)
    v = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 3)
    qi = ms.fill_int_bf16(np.empty((B, T, G, 128), np.uint16), seed + 4, -4, 4)
    ki = ms.fill_int_bf16(np.empty((B, N, 128), np.uint16), seed + 5, -4, 4)
    do = ms.fill_normal_bf16(np.empty((B, T, H, 128), np.uint16), seed + 6)
    cfg = lib_cfg(G, R, K)
    kv, qs = dev_i32(np.array([N], np.int32)), dev_i32(np.array([0], np.int32))
    dq_, dk_, dv_, ddo = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    say("forward and backward twice B=%d T=%d N=%d G=%d R=%d K=%d" % (B, T, N, G, R, K))
    sel = msa.index_topk(cfg, dev_index(qi), dev_index(ki), kv, qs)
    res = []
    for _ in range(2):
        out, lse = msa.sparse_attn_prefill(cfg, dq_, dk_, dv_, kv, sel, q_start=qs, want_lse=True)
        res.append((out, lse) + tuple(msa.sparse_attn_backward(cfg, dq_, dk_, dv_, kv, sel, out,
                                                               lse, ddo, q_start=qs)))
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), res[0], res[1]):
        assert torch.equal(a, b), name
