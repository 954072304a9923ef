"""GPU parity: libmsa (through its C ABI) against the fp64 CPU oracle on the
same seeded inputs. Selections must match bit for bit; attention outputs to
max-abs 2e-2 and relative L2 5e-3; lse to 1e-3."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
from gpu_helpers import (bf16_out_to_f64, compare_lse, compare_out, dev_bf16, dev_i32,
                         dev_index, lib_cfg, oracle_cfg, say)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)


def random_problem(B, T, Nmax, G, R, seed, fp8=False, idx_lo=-4, idx_hi=4):
    H, d, dI = G * R, 128, 128
    q = ms.fill_normal_bf16(np.empty((B, T, H, d), np.uint16), seed + 1)
    k = ms.fill_normal_bf16(np.empty((B, G, Nmax, d), np.uint16), seed + 2)
    v = ms.fill_normal_bf16(np.empty((B, G, Nmax, d), np.uint16), seed + 3)
    if fp8:
        qi = ms.fill_int_e4m3(np.empty((B, T, G, dI), np.uint8), seed + 4, idx_lo, idx_hi)
        ki = ms.fill_int_e4m3(np.empty((B, Nmax, dI), np.uint8), seed + 5, idx_lo, idx_hi)
    else:
        qi = ms.fill_int_bf16(np.empty((B, T, G, dI), np.uint16), seed + 4, idx_lo, idx_hi)
        ki = ms.fill_int_bf16(np.empty((B, Nmax, dI), np.uint16), seed + 5, idx_lo, idx_hi)
    return dict(q=q, k=k, v=v, qi=qi, ki=ki)


def run_gpu(pr, G, R, K, kv_lens, q_start, decode=False, fp8=False, sel_override=None):
    cfg = lib_cfg(G, R, K, fp8)
    kv = dev_i32(kv_lens)
    qs = None if q_start is None else dev_i32(q_start)
    qi, ki = dev_index(pr["qi"]), dev_index(pr["ki"])
    q, k, v = dev_bf16(pr["q"]), dev_bf16(pr["k"]), dev_bf16(pr["v"])
    say("index_topk B=%d T=%d G=%d Nmax=%d K=%d" % (qi.shape[0], qi.shape[1], G, ki.shape[1], K))
    sel, scores = msa.index_topk(cfg, qi, ki, kv, qs, want_scores=True)
    torch.cuda.synchronize()
    use_sel = sel if sel_override is None else dev_i32(sel_override)
    if decode:
        say("sparse_attn_decode B=%d R=%d" % (q.shape[0], R))
        out, lse = msa.sparse_attn_decode(cfg, q, k, v, kv, use_sel, want_lse=True)
    else:
        say("sparse_attn_prefill B=%d T=%d R=%d" % (q.shape[0], q.shape[1], R))
        out, lse = msa.sparse_attn_prefill(cfg, q, k, v, kv, use_sel, q_start=qs, want_lse=True)
    torch.cuda.synchronize()
    return (sel.cpu().numpy(), scores.cpu().numpy(), bf16_out_to_f64(out),
            lse.cpu().numpy().astype(np.float64))


def check_all_rows(orc, pr, G, R, K, kv_lens, q_start, decode=False, fp8=False, what=""):
    B, T = pr["q"].shape[0], pr["q"].shape[1]
    kv_lens = np.asarray(kv_lens, np.int32)
    qs_eff = (kv_lens - T) if q_start is None else np.asarray(q_start, np.int32)
    sel, scores, out, lse = run_gpu(pr, G, R, K, kv_lens, q_start, decode, fp8)
    ocfg = oracle_cfg(G, R, K, fp8)
    osel, oscores = orc.index_topk(ocfg, pr["qi"], pr["ki"], kv_lens, qs_eff)
    n = B * T
    gsel = sel.reshape(n, G, K)
    mism = int((gsel != osel).any(axis=(1, 2)).sum())
    say("%s: sel rows=%d mismatching=%d" % (what, n, mism))
    assert mism == 0
    assert np.array_equal(scores.reshape(n, G, K).astype(np.float64), oscores)
    oout, olse = orc.sparse_attn(ocfg, pr["q"], pr["k"], pr["v"], kv_lens, qs_eff, osel)
    compare_out(out.reshape(oout.shape), oout, what)
    compare_lse(lse.reshape(olse.shape), olse, what)
    return sel, out, lse


def test_prefill_L4096_one_group_all_rows(orc):
    """The 4096-token, 1 group x 2 heads prefill on every row, then the decode
    entry points for the last token against prefill row 4095."""
    L, G, R, K = 4096, 1, 2, 16
    pr = random_problem(1, L, L, G, R, seed=100)
    sel, out, lse = check_all_rows(orc, pr, G, R, K, [L], [0], what="prefill L4096")
    last = {k_: (v_[:, L - 1:L] if k_ in ("q", "qi") else v_) for k_, v_ in pr.items()}
    dsel, _, dout, dlse = run_gpu(last, G, R, K, [L], None, decode=True)
    assert np.array_equal(dsel[0, 0], sel[0, L - 1])
    compare_out(dout[0, 0], out[0, L - 1], "decode vs prefill row")


def test_decode_ragged_lengths(orc):
    G, R, K, Nmax = 4, 8, 16, 3000
    lens = [3000, 2999, 1, 129, 2048, 128]
    pr = random_problem(len(lens), 1, Nmax, G, R, seed=200)
    check_all_rows(orc, pr, G, R, K, lens, None, decode=True, what="decode ragged")


@pytest.mark.parametrize("K", [16, 64])
def test_chunked_prefill_ragged_cache(orc, K):
    """Query rows start mid-cache; the cache stride is not a multiple of 128."""
    G, R, Nmax, T = 4, 8, 1000 if K == 16 else 9000, 300
    pr = random_problem(2, T, Nmax, G, R, seed=300 + K)
    lens = [Nmax, Nmax // 2]
    check_all_rows(orc, pr, G, R, K, lens, [Nmax - 300, 50], what="chunked ragged K%d" % K)


@pytest.mark.parametrize("G,R,K,T,N", [(1, 1, 1, 40, 300), (3, 5, 7, 5, 700), (3, 5, 7, 6, 700),
                                       (2, 16, 32, 70, 4500), (8, 4, 16, 2, 2100),
                                       (5, 3, 16, 100, 1500), (4, 8, 16, 4, 5000)])
def test_shapes(orc, G, R, K, T, N):
    pr = random_problem(2, T, N, G, R, seed=400 + G * 7 + R + K + T)
    check_all_rows(orc, pr, G, R, K, [N, N - 37], None, what="G%d R%d K%d T%d" % (G, R, K, T))


@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_register_topk_K32_sampled_rows(orc, fp8):
    """A prefill with enough row tiles (two 8192-token sequences x 4 groups:
    256 workgroups) for the index kernel's fused register top-K, at K = 32
    (its 32-slot variant), bf16 and E4M3: 640 seeded rows, bit for bit. (The
    small prefills of the other tests split their key blocks and rank the
    pooled scores instead.)"""
    G, R, K, T = 4, 8, 32, 8192
    lim = 16 if fp8 else 4
    pr = random_problem(2, T, T, G, R, seed=1400 + fp8, fp8=fp8, idx_lo=-lim, idx_hi=lim)
    cfg = lib_cfg(G, R, K, fp8)
    assert msa.workspace_size(cfg, 2, T, T, msa.WS_INDEX_TOPK) == 0  # the register path
    kv, qs = np.array([T, T - 300], np.int32), np.array([0, 0], np.int32)
    say("register top-K prefill, fp8=%s" % fp8)
    sel, sc = msa.index_topk(cfg, dev_index(pr["qi"]), dev_index(pr["ki"]), dev_i32(kv),
                             dev_i32(qs), want_scores=True)
    torch.cuda.synchronize()
    sel, sc = sel.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(1401)
    rb = rng.integers(0, 2, 640)
    rows = np.stack([rb, rng.integers(0, kv[rb])], axis=1).astype(np.int32)
    rows[:4] = [[0, 0], [0, T - 1], [1, 0], [1, T - 301]]
    osel, osc = orc.index_topk(oracle_cfg(G, R, K, fp8), pr["qi"], pr["ki"], kv, qs, rows=rows)
    gsel = sel[rows[:, 0], rows[:, 1]].reshape(osel.shape)
    assert np.array_equal(gsel, osel)
    assert np.array_equal(sc[rows[:, 0], rows[:, 1]].reshape(osc.shape), osc)
    assert (sel[1, T - 300:] == -1).all()  # rows past the second sequence's cache


def test_all_ties_select_lowest_blocks(orc):
    """Zero index queries make every pooled score 0 (including -0.0 products):
    the K lowest blocks win."""
    G, R, K, N, T = 4, 8, 16, 4096, 200
    pr = random_problem(1, T, N, G, R, seed=500)
    pr["qi"][:] = 0
    pr["qi"][0, ::2] = 0x8000  # -0.0 on every other row
    sel, out, lse = check_all_rows(orc, pr, G, R, K, [N], None, what="ties")
    assert (sel[0, :, :, :] == np.arange(K, dtype=np.int32)).all()


def test_rows_outside_the_cache_are_empty(orc):
    G, R, K, N, T = 2, 4, 8, 512, 64
    pr = random_problem(1, T, N, G, R, seed=600)
    sel, _, out, lse = run_gpu(pr, G, R, K, [300], [260])  # rows 40..63 sit at p >= 300
    assert (sel[0, 40:] == -1).all()
    assert (out[0, 40:] == 0).all()
    assert np.isneginf(lse[0, 40:]).all()
    osel, _ = orc.index_topk(oracle_cfg(G, R, K), pr["qi"][:, :40], pr["ki"], [300], [260])
    assert np.array_equal(sel[0, :40].reshape(40, G, K), osel)


def test_caller_selection_with_repeats_and_out_of_range(orc):
    G, R, K, N, T = 2, 4, 8, 2048, 32
    pr = random_problem(1, T, N, G, R, seed=700)
    rng = np.random.default_rng(7)
    sel = rng.integers(-3, 20, size=(1, T, G, K)).astype(np.int32)  # -ve, repeats, > causal
    sel[0, :, :, 1] = sel[0, :, :, 0]
    kv, qs = np.array([N], np.int32), np.array([N - T], np.int32)
    _, _, out, lse = run_gpu(pr, G, R, K, kv, qs, sel_override=sel)
    oout, olse = orc.sparse_attn(oracle_cfg(G, R, K), pr["q"], pr["k"], pr["v"], kv, qs,
                                 sel.reshape(T, G, K))
    compare_out(out.reshape(oout.shape), oout, "caller sel")
    compare_lse(lse.reshape(olse.shape), olse, "caller sel")


def test_repeat_runs_are_bitwise_identical():
    G, R, K, N = 4, 8, 16, 8192
    pr = random_problem(3, 1, N, G, R, seed=800)
    a = run_gpu(pr, G, R, K, [N, 5000, 777], None, decode=True)
    b = run_gpu(pr, G, R, K, [N, 5000, 777], None, decode=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_workspace_reuse(orc):
    """A workspace is plain scratch: calls that reuse one (starting as random
    bytes) with different batches and lengths match calls with fresh ones and
    the oracle."""
    G, R, K, N = 4, 8, 16, 6000
    cfg = lib_cfg(G, R, K)
    ws_i = msa.workspace(cfg, 4, 1, N, msa.WS_INDEX_TOPK).random_(0, 256)  # garbage scratch
    ws_d = msa.workspace(cfg, 4, 1, N, msa.WS_SPARSE_DECODE).random_(0, 256)
    for trial, lens in enumerate([[6000, 3000, 128, 1], [5000, 5000], [1, 2, 3, 4000], [6000]]):
        B = len(lens)
        pr = random_problem(B, 1, N, G, R, seed=900 + trial)
        kv = dev_i32(lens)
        qi, ki = dev_index(pr["qi"]), dev_index(pr["ki"])
        q, k, v = dev_bf16(pr["q"]), dev_bf16(pr["k"]), dev_bf16(pr["v"])
        say("workspace reuse trial %d lens=%s" % (trial, lens))
        sel = msa.index_topk(cfg, qi, ki, kv, workspace=ws_i)
        out = msa.sparse_attn_decode(cfg, q, k, v, kv, sel, workspace=ws_d)
        sel_f = msa.index_topk(cfg, qi, ki, kv)
        out_f = msa.sparse_attn_decode(cfg, q, k, v, kv, sel_f)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_f) and torch.equal(out, out_f)
        lens_np = np.array(lens, np.int32)
        osel, _ = orc.index_topk(oracle_cfg(G, R, K), pr["qi"], pr["ki"], lens_np, lens_np - 1)
        assert np.array_equal(sel.cpu().numpy().reshape(osel.shape), osel)



def run_fused_decode(pr, G, R, K, kv_lens, workspace=None, fp8=False):
    cfg = lib_cfg(G, R, K, fp8)
    kv = dev_i32(kv_lens)
    qi, ki = dev_index(pr["qi"]), dev_index(pr["ki"])
    q, k, v = dev_bf16(pr["q"]), dev_bf16(pr["k"]), dev_bf16(pr["v"])
    say("msa_decode B=%d Nmax=%d G=%d R=%d K=%d" % (q.shape[0], k.shape[2], G, R, K))
    sel, sc, out, lse = msa.decode(cfg, q, qi, ki, k, v, kv, want_scores=True, want_lse=True,
                                   workspace=workspace)
    torch.cuda.synchronize()
    return (sel.cpu().numpy(), sc.cpu().numpy(), bf16_out_to_f64(out),
            lse.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("G,R,K,lens,fp8", [
    (4, 8, 16, [3000, 2999, 1, 129, 2048, 128, 0, 5000], False), (1, 2, 16, [4096], False),
    (3, 5, 7, [700, 513], False), (2, 16, 32, [4500, 4500, 17], False),
    (4, 8, 16, [3000, 2999, 1, 129, 2048, 128, 0, 5000], True),
    # more than 16 groups: the MFMA index kernel writes the pooled scores
    (17, 1, 16, [3000, 1, 2500, 130], False),
    # K = 1 and K = 3: the ranking merges runs of 1 and 4 keys
    (2, 4, 1, [20000, 300], False), (3, 2, 3, [20000, 777, 5], False),
    # K = 40 and 64: runs of 64 keys, eight registers merged; 32 splits
    (4, 8, 64, [20000, 9000, 130, 8192], False), (2, 4, 40, [3000, 70000], True)])
def test_decode_step_matches_oracle_and_two_calls(orc, G, R, K, lens, fp8):
    Nmax = max(max(lens), 1)
    lim = 16 if fp8 else 4
    pr = random_problem(len(lens), 1, Nmax, G, R, seed=1000 + G + R + K + fp8, fp8=fp8,
                        idx_lo=-lim, idx_hi=lim)
    sel, sc, out, lse = run_fused_decode(pr, G, R, K, lens, fp8=fp8)
    kv = np.array(lens, np.int32)
    valid = kv > 0
    ocfg = oracle_cfg(G, R, K, fp8)
    rows = np.array([(b, 0) for b in range(len(lens)) if valid[b]], np.int32)
    osel, osc = orc.index_topk(ocfg, pr["qi"], pr["ki"], kv, kv - 1, rows=rows)
    assert np.array_equal(sel[valid].reshape(osel.shape), osel)
    assert np.array_equal(sc[valid].reshape(osc.shape).astype(np.float64), osc)
    assert (sel[~valid] == -1).all()
    oout, olse = orc.sparse_attn(ocfg, pr["q"], pr["k"], pr["v"], kv, kv - 1, osel, rows=rows)
    compare_out(out[valid].reshape(oout.shape), oout, "msa_decode")
    compare_lse(lse[valid].reshape(olse.shape), olse, "msa_decode")
    assert (out[~valid] == 0).all() and np.isneginf(lse[~valid]).all()
    # The same selection as msa_index_topk + msa_sparse_attn_decode; the
    # outputs agree to the tolerance (their split partials merge in a
    # different order).
    s2, _, o2, l2 = run_gpu(pr, G, R, K, lens, None, decode=True, fp8=fp8)
    assert np.array_equal(s2, sel)
    compare_out(o2[valid].reshape(oout.shape), out[valid].reshape(oout.shape), "two-call vs msa_decode")


def test_decode_step_workspace_reuse(orc):
    G, R, K, N = 4, 8, 16, 20000
    cfg = lib_cfg(G, R, K)
    ws = msa.workspace(cfg, 6, 1, N, msa.WS_DECODE).random_(0, 256)
    for trial, lens in enumerate([[20000] * 6, [1, 20000, 333], [19999, 128, 129, 4000, 5, 6]]):
        pr = random_problem(len(lens), 1, N, G, R, seed=1100 + trial)
        sel, _, out, _ = run_fused_decode(pr, G, R, K, lens, workspace=ws)
        sel2, _, out2, _ = run_fused_decode(pr, G, R, K, lens)
        assert np.array_equal(sel, sel2) and np.array_equal(out, out2)
        kv = np.array(lens, np.int32)
        osel, _ = orc.index_topk(oracle_cfg(G, R, K), pr["qi"], pr["ki"], kv, kv - 1)
        assert np.array_equal(sel.reshape(osel.shape), osel)



def test_decode_many_small_sequences(orc):
    """1030 sequences x 16 groups (16480 workgroups) of short, ragged rows."""
    G, R, K, N = 16, 1, 4, 200
    rng = np.random.default_rng(12)
    lens = rng.integers(1, N + 1, size=1030).tolist()
    pr = random_problem(len(lens), 1, N, G, R, seed=1200)
    sel, sc, out, lse = run_fused_decode(pr, G, R, K, lens)
    kv = np.array(lens, np.int32)
    ocfg = oracle_cfg(G, R, K)
    osel, _ = orc.index_topk(ocfg, pr["qi"], pr["ki"], kv, kv - 1)
    assert np.array_equal(sel.reshape(osel.shape), osel)
    oout, olse = orc.sparse_attn(ocfg, pr["q"], pr["k"], pr["v"], kv, kv - 1, osel)
    compare_out(out.reshape(oout.shape), oout, "many sequences")
    compare_lse(lse.reshape(olse.shape), olse, "many sequences")


@pytest.mark.parametrize("B,N,lens", [
    # 16 sequences x 4 groups: the 16-wave attention kernel, rows of up to
    # 128 blocks ranked by one wave
    (16, 16384, [16384] * 8 + [9000, 129, 16383, 8192, 3000, 130, 12000, 16000]),
    # rows of up to 2048 blocks: every wave ranks a share (8-wave kernel)
    (2, 262144, [262144, 140000])])
def test_decode_all_ties_take_the_general_ranking(orc, B, N, lens):
    """Zero index queries tie every pooled score at 0 (-0.0 products in every
    other sequence), so far more than 64 candidates reach the ranking's
    threshold and it takes its general path; the K lowest blocks win, in
    msa_decode and in msa_index_topk alike."""
    G, R, K = 4, 8, 16
    pr = random_problem(B, 1, N, G, R, seed=1300 + B)
    pr["qi"][:] = 0
    pr["qi"][1::2] = 0x8000
    sel, sc, out, lse = run_fused_decode(pr, G, R, K, lens)
    kv = np.array(lens, np.int32)
    ocfg = oracle_cfg(G, R, K)
    osel, _ = orc.index_topk(ocfg, pr["qi"], pr["ki"], kv, kv - 1)
    assert np.array_equal(sel.reshape(osel.shape), osel)
    full = kv >= K * 128
    assert (sel.reshape(osel.shape)[full] == np.arange(K, dtype=np.int32)).all()
    oout, olse = orc.sparse_attn(ocfg, pr["q"], pr["k"], pr["v"], kv, kv - 1, osel)
    compare_out(out.reshape(oout.shape), oout, "ties, msa_decode")
    compare_lse(lse.reshape(olse.shape), olse, "ties, msa_decode")
    s2, _, _, _ = run_gpu(pr, G, R, K, lens, None, decode=True)
    assert np.array_equal(s2, sel)


@pytest.mark.parametrize("B,T,G,N,lens,qstart", [
    (3, 1, 4, 9000, [9000, 4100, 1], None),          # streaming kernel, one row per group
    (2, 4, 4, 3000, [3000, 130], None),               # streaming kernel, 16 rows
    (2, 300, 4, 1000, [1000, 400], [700, 50]),        # MFMA kernel, chunked rows
])
def test_index_pool_matches_oracle(orc, B, T, G, N, lens, qstart):
    """msa_index_pool: every pooled block score equals the oracle's exactly;
    blocks past a row's position stay as the caller filled them (-inf)."""
    pr = random_problem(B, T, N, G, 1, seed=1300 + T)
    cfg = lib_cfg(G, 1, 16)
    kv = np.asarray(lens, np.int32)
    qs = (kv - T) if qstart is None else np.asarray(qstart, np.int32)
    say("index_pool B=%d T=%d G=%d N=%d" % (B, T, G, N))
    pooled = msa.index_pool(cfg, dev_index(pr["qi"]), dev_index(pr["ki"]), dev_i32(kv),
                            None if qstart is None else dev_i32(qs))
    torch.cuda.synchronize()
    got = pooled.cpu().numpy().astype(np.float64).reshape(B * T, G, -1)
    want = orc.index_pool(oracle_cfg(G, 1, 16), pr["qi"], pr["ki"], kv, qs)
    assert got.shape == want.shape
    assert np.array_equal(got, want), int((got != want).sum())


@pytest.mark.parametrize("B,T,N,lens,qstart,decode", [
    (2, 300, 1000, [1000, 400], [700, 50], False),     # MFMA kernel, chunked rows
    (1, 1100, 4500, [4500], None, False),               # several 256-row tiles, ragged tail
    (6, 1, 3000, [3000, 2999, 1, 129, 2048, 128], None, True),  # streaming kernel
    (2, 4, 3000, [3000, 130], None, False),             # streaming kernel, 16 rows
])
def test_fp8_index_matches_oracle(orc, B, T, N, lens, qstart, decode):
    """OCP E4M3 index queries and keys (integers in [-16, 16]): selections and
    pooled scores bit-exact, attention within tolerance."""
    G, R, K = 4, 8, 16
    pr = random_problem(B, T, N, G, R, seed=1500 + T + B, fp8=True, idx_lo=-16, idx_hi=16)
    check_all_rows(orc, pr, G, R, K, lens, qstart, decode=decode, fp8=True,
                   what="fp8 B%d T%d" % (B, T))
    kv = np.asarray(lens, np.int32)
    qs = (kv - T) if qstart is None else np.asarray(qstart, np.int32)
    pooled = msa.index_pool(lib_cfg(G, R, K, True), dev_index(pr["qi"]), dev_index(pr["ki"]),
                            dev_i32(kv), None if qstart is None else dev_i32(qs))
    torch.cuda.synchronize()
    want = orc.index_pool(oracle_cfg(G, R, K, True), pr["qi"], pr["ki"], kv, qs)
    assert np.array_equal(pooled.cpu().numpy().astype(np.float64).reshape(want.shape), want)


def test_kv_major_prefill_caller_selection_and_empty_rows(orc):
    """The KV-major sparse prefill (>= 256 (row, group) pairs) with a caller
    selection holding repeats, negative and out-of-range ids, and rows past
    the cache (empty)."""
    G, R, K, N, T = 2, 4, 8, 3000, 300
    pr = random_problem(1, T, N, G, R, seed=1700)
    rng = np.random.default_rng(17)
    sel = rng.integers(-3, 26, size=(1, T, G, K)).astype(np.int32)
    sel[0, :, :, 1] = sel[0, :, :, 0]
    kv, qs = np.array([2900], np.int32), np.array([2650], np.int32)  # rows 250.. sit at p >= 2900
    _, _, out, lse = run_gpu(pr, G, R, K, kv, qs, sel_override=sel)
    assert (out[0, 250:] == 0).all() and np.isneginf(lse[0, 250:]).all()
    rows = np.array([(0, i) for i in range(250)], np.int32)
    oout, olse = orc.sparse_attn(oracle_cfg(G, R, K), pr["q"], pr["k"], pr["v"], kv, qs,
                                 sel[0, :250].reshape(250, G, K), rows=rows)
    compare_out(out[0, :250].reshape(oout.shape), oout, "kv-major caller sel")
    compare_lse(lse[0, :250].reshape(olse.shape), olse, "kv-major caller sel")


def test_kv_major_prefill_workspace_reuse(orc):
    """Garbage-filled prefill workspace reused across calls of different
    shapes gives the same bits as fresh workspaces."""
    G, R, K, N = 4, 8, 16, 5000
    cfg = lib_cfg(G, R, K)
    ws = msa.workspace(cfg, 2, 400, N, msa.WS_SPARSE_PREFILL).random_(0, 256)
    for trial, (B, T, lens, qs) in enumerate([(2, 400, [5000, 2000], [4600, 1600]),
                                              (1, 300, [4000], [0]),
                                              (2, 128, [5000, 129], [4872, 1])]):
        pr = random_problem(B, T, N, G, R, seed=1800 + trial)
        kv, qsd = dev_i32(lens), dev_i32(qs)
        qi, ki = dev_index(pr["qi"]), dev_index(pr["ki"])
        q, k, v = dev_bf16(pr["q"]), dev_bf16(pr["k"]), dev_bf16(pr["v"])
        say("prefill workspace reuse trial %d B=%d T=%d" % (trial, B, T))
        sel = msa.index_topk(cfg, qi, ki, kv, qsd)
        out = msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qsd, workspace=ws)
        out_f = msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qsd)
        torch.cuda.synchronize()
        assert torch.equal(out, out_f)


@pytest.mark.parametrize("G,R,K,T,N,fp8", [(2, 16, 32, 300, 4500, True), (4, 16, 16, 100, 3000, False),
                                          (1, 3, 5, 700, 2000, False), (3, 1, 32, 200, 6000, True),
                                          (2, 8, 64, 300, 12000, False), (2, 4, 48, 150, 9000, True),
                                          (1, 2, 64, 40, 20000, False)])
def test_prefill_paths_more_shapes(orc, G, R, K, T, N, fp8):
    """E4M3 with K = 32 (32-slot register top-K), R = 16 (one entry per query
    tile), R = 3 (tiles of 5 entries), R = 1; all through the KV-major path;
    K = 48 and 64 (above the register top-K: pooled scores, then a ranking
    per row; list entries with slots above 31), the last one on the
    query-major path (80 (row, group) pairs)."""
    lim = 16 if fp8 else 4
    pr = random_problem(2, T, N, G, R, seed=1900 + G + R + K + T, fp8=fp8, idx_lo=-lim, idx_hi=lim)
    check_all_rows(orc, pr, G, R, K, [N, N - 300], None, fp8=fp8,
                   what="G%d R%d K%d T%d fp8=%d" % (G, R, K, T, fp8))


def _sweep_cases(n=36, seed=2024):
    """Seeded shapes for the sweep below: prefill, chunked prefill (query rows
    after a cache prefix) and decode in turn, with the group, head, top-k and
    index-type choices drawn from the supported ranges."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        mode = ("prefill", "chunked", "decode")[i % 3]
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        R = int(rng.choice([r for r in (1, 2, 3, 8, 16) if G * r <= 32]))
        K = int(rng.choice([1, 2, 5, 16, 31, 32, 33, 48, 64]))
        fp8 = bool(rng.integers(0, 2))
        cases.append((i, mode, G, R, K, fp8))
    return cases


@pytest.mark.parametrize("i,mode,G,R,K,fp8", _sweep_cases())
def test_seeded_shape_sweep(orc, i, mode, G, R, K, fp8):
    """Every row of a seeded shape against the oracle: selections bit for bit,
    outputs and lse within the tolerances (the short-prefill index split and
    the small tiles of the sparse prefill, the 8-wave decode, K on both sides
    of the register top-K)."""
    rng = np.random.default_rng(3000 + i)
    if mode == "decode":
        lens = rng.integers(1, 6000, size=int(rng.integers(1, 21))).tolist()
        test_decode_step_matches_oracle_and_two_calls(orc, G, R, K, lens, fp8)
        return
    B = int(rng.integers(1, 3))
    T = int(rng.integers(17, 200))
    qs = [0] * B if mode == "prefill" else rng.integers(1, 4000, size=B).tolist()
    kv = [q + T + int(rng.integers(0, 300)) for q in qs]  # keys past the last row exist
    lim = 16 if fp8 else 4
    pr = random_problem(B, T, max(kv), G, R, seed=3100 + i, fp8=fp8, idx_lo=-lim, idx_hi=lim)
    check_all_rows(orc, pr, G, R, K, kv, qs, fp8=fp8,
                   what="sweep %d %s G%d R%d K%d fp8=%s" % (i, mode, G, R, K, fp8))


def test_list_build_paths_for_caches_past_16384_blocks(orc):
    """A cache capacity above 16384 key blocks takes the list build's global
    atomic marking and plain scatter instead of the LDS forms: the same rows
    and keys with a small and a large capacity give bit-identical forward
    outputs and gradients, and the forward matches the oracle."""
    G, R, K, T = 1, 4, 8, 300
    kv, qs = [600], [300]
    N_small, N_big = 1024, 16386 * 128  # 8 and 16386 key blocks
    pr = random_problem(1, T, N_small, G, R, seed=2300)
    cfg = lib_cfg(G, R, K)

    def caches(N):
        k = np.zeros((1, G, N, 128), np.uint16)
        v = np.zeros((1, G, N, 128), np.uint16)
        ki = np.zeros((1, N, 128), np.uint16)
        k[:, :, :N_small], v[:, :, :N_small], ki[:, :N_small] = pr["k"], pr["v"], pr["ki"]
        return dev_bf16(k), dev_bf16(v), dev_bf16(ki)

    q, qi = dev_bf16(pr["q"]), dev_bf16(pr["qi"])
    kvd, qsd = dev_i32(kv), dev_i32(qs)
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    dout = torch.randn((1, T, G * R, 128), generator=g, device="cuda").to(torch.bfloat16)
    res = {}
    for N in (N_small, N_big):
        k, v, ki = caches(N)
        say("list build paths: Nmax=%d" % N)
        sel = msa.index_topk(cfg, qi, ki, kvd, qsd)
        out, lse = msa.sparse_attn_prefill(cfg, q, k, v, kvd, sel, q_start=qsd, want_lse=True)
        dq, dk, dv = msa.sparse_attn_backward(cfg, q, k, v, kvd, sel, out, lse, dout, q_start=qsd)
        torch.cuda.synchronize()
        assert not dk[:, :, N_small:].any() and not dv[:, :, N_small:].any()
        res[N] = (sel.cpu(), out.cpu(), lse.cpu(), dq.cpu(), dk[:, :, :N_small].cpu(),
                  dv[:, :, :N_small].cpu())
        del k, v, ki, dk, dv
        torch.cuda.empty_cache()
    for a, b in zip(res[N_small], res[N_big]):
        assert torch.equal(a, b)
    sel, lse = res[N_small][0].numpy(), res[N_small][2].numpy()
    osel, _ = orc.index_topk(oracle_cfg(G, R, K), pr["qi"], pr["ki"], kv, qs)
    assert np.array_equal(sel.reshape(osel.shape), osel)
    oout, olse = orc.sparse_attn(oracle_cfg(G, R, K), pr["q"], pr["k"], pr["v"], kv, qs, osel)
    compare_out(bf16_out_to_f64(res[N_small][1]).reshape(oout.shape), oout, "list paths")
    compare_lse(lse.astype(np.float64).reshape(olse.shape), olse, "list paths")
