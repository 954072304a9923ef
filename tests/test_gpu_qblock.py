"""GPU parity of the query-block-shared selection variant (msa_index_topk_qblock
and msa_sparse_attn_prefill_qblock, through the C ABI) against the oracle:
selections and their scores bit for bit, outputs and lse within the parity
tolerances, on every row, including unaligned chunk starts, rows outside the
cache, odd group counts, head counts that do not divide 16, E4M3 index data
and caller selections with repeats and invalid ids."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
import oracle
from gpu_helpers import (bf16_out_to_f64, compare_lse, compare_out, dev_bf16, dev_i32,
                         dev_index, lib_cfg, oracle_cfg, say)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

S = 128


def problem(B, T, N, G, R, seed, fp8=False):
    H = G * R
    q = ms.fill_normal_bf16(np.empty((B, T, H, 128), np.uint16), seed + 1)
    k = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 2)
    v = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 3)
    if fp8:
        qi = ms.fill_int_e4m3(np.empty((B, T, G, 128), np.uint8), seed + 4, -4, 4)
        ki = ms.fill_int_e4m3(np.empty((B, N, 128), np.uint8), seed + 5, -4, 4)
    else:
        qi = ms.fill_int_bf16(np.empty((B, T, G, 128), np.uint16), seed + 4, -4, 4)
        ki = ms.fill_int_bf16(np.empty((B, N, 128), np.uint16), seed + 5, -4, 4)
    return dict(q=q, k=k, v=v, qi=qi, ki=ki)


def check(orc, B, T, N, G, R, K, kv_lens, q_start, fp8=False, seed=700, sel_override=None):
    pr = problem(B, T, N, G, R, seed, fp8)
    kv_lens = np.asarray(kv_lens, np.int32)
    q_start = np.asarray(q_start, np.int32)
    cfg = lib_cfg(G, R, K, fp8)
    ocfg = oracle_cfg(G, R, K, fp8)
    kv, qs = dev_i32(kv_lens), dev_i32(q_start)
    say("index_topk_qblock B=%d T=%d N=%d G=%d R=%d K=%d q_start=%s fp8=%s" %
        (B, T, N, G, R, K, list(q_start), fp8))
    sel, sc = msa.index_topk_qblock(cfg, dev_index(pr["qi"]), dev_index(pr["ki"]), kv, qs,
                                    want_scores=True)
    torch.cuda.synchronize()
    nq = oracle.qblock_slots(T, S)
    assert tuple(sel.shape) == (B, nq, G, K)
    osel, osc = orc.index_topk_qblock(ocfg, pr["qi"], pr["ki"], kv_lens, q_start)
    gsel = sel.cpu().numpy().reshape(osel.shape)
    mism = int((gsel != osel).any(axis=(1, 2)).sum())
    say("qblock sel items=%d mismatching=%d" % (osel.shape[0], mism))
    assert mism == 0
    assert np.array_equal(sc.cpu().numpy().reshape(osc.shape).astype(np.float64), osc)
    use = osel.reshape(B, nq, G, K) if sel_override is None else np.asarray(sel_override,
                                                                               np.int32)
    say("sparse_attn_prefill_qblock")
    out, lse = msa.sparse_attn_prefill_qblock(cfg, dev_bf16(pr["q"]), dev_bf16(pr["k"]),
                                              dev_bf16(pr["v"]), kv, dev_i32(use), q_start=qs,
                                              want_lse=True)
    torch.cuda.synchronize()
    # Rows of the call inside the cache, with their block's selection.
    rows = np.array([(b, i) for b in range(B) for i in range(T)
                     if 0 <= q_start[b] + i < kv_lens[b]], np.int32).reshape(-1, 2)
    got_o = bf16_out_to_f64(out)
    got_l = lse.cpu().numpy().astype(np.float64)
    if rows.size:
        rsel = oracle.qblock_rows_sel(use, q_start, T, S, rows=rows)
        oout, olse = orc.sparse_attn(ocfg, pr["q"], pr["k"], pr["v"], kv_lens, q_start, rsel,
                                     rows=rows)
        compare_out(got_o[rows[:, 0], rows[:, 1]], oout, "qblock attention")
        compare_lse(got_l[rows[:, 0], rows[:, 1]], olse, "qblock attention")
    # Rows outside the cache are zero with lse = -inf.
    outside = [(b, i) for b in range(B) for i in range(T) if not 0 <= q_start[b] + i < kv_lens[b]]
    for b, i in outside:
        assert not got_o[b, i].any() and np.all(np.isneginf(got_l[b, i]))


def test_aligned_prefill(orc):
    check(orc, 1, 1024, 1024, 4, 8, 16, [1024], [0])


def test_unaligned_chunks_and_ragged_cache(orc):
    # chunk starts mid-block; sequence 1's cache ends inside the chunk
    check(orc, 2, 300, 2000, 4, 8, 16, [1900, 1500], [1600, 1300], seed=710)


def test_rows_outside_the_cache(orc):
    check(orc, 2, 200, 1000, 2, 8, 16, [150, 1000], [0, 700], seed=720)


def test_odd_groups_and_heads(orc):
    check(orc, 1, 260, 3000, 3, 5, 7, [3000], [2740], seed=730)


def test_r16_k1_and_r1(orc):
    check(orc, 1, 256, 1300, 1, 16, 1, [1300], [1044], seed=740)
    check(orc, 1, 130, 700, 2, 1, 4, [700], [570], seed=745)


def test_fp8_index_and_k32(orc):
    check(orc, 1, 384, 5000, 4, 8, 32, [5000], [4616], fp8=True, seed=750)


def test_short_contexts_keep_every_block(orc):
    # fewer causal blocks than K: every block kept, -1 padding
    check(orc, 2, 700, 700, 4, 2, 16, [700, 400], [0, 0], seed=760)


def test_caller_selection_with_repeats_and_invalid_ids(orc):
    B, T, N, G, K = 1, 256, 1024, 2, 6
    nq = oracle.qblock_slots(T, S)
    rng = np.random.default_rng(5)
    sel = rng.integers(-3, 10, size=(B, nq, G, K)).astype(np.int32)
    sel[0, 0, 0] = [3, 3, 3, -1, 99, 0]
    check(orc, B, T, N, G, 4, K, [N], [N - T], seed=770, sel_override=sel)
