"""Parity at the full sizes of the workloads, through the C ABI, in the launch
configuration the benchmark uses:
  decode, 16 sequences x 131072 tokens          every row (msa_decode and the
                                                 two-call form, each against the
                                                 oracle);
  decode, 4 sequences x 1048576 tokens           every row, uniform lengths and
                                                 mixed {256k, 512k, 768k, 1M};
  decode, 16 sequences of ragged lengths up to   every row (rows longer than
  196608 tokens                                  1024 blocks, 16-wave form);
  both decode batches with E4M3 index data       every row (uniform lengths);
  prefill, 131072 tokens (4 groups x 8 heads)    a stratified sample of 2048 rows;
  chunked prefill, 1048576 tokens in 32768-row   all 32 chunks: the first, a
  chunks, E4M3 index data                        middle and the last chunk on
                                                 1515 sampled rows, every other
                                                 chunk on its first and last
                                                 row and 17 seeded rows (2066
                                                 rows in all; the oracle's cost
                                                 per row grows with position);
  query-block-shared selections, 131072-token    24 sampled query blocks
  prefill and two chunks of the 1M chunked       (selections), 8 rows of each
  prefill                                        (attention);
  sparse backward, 131072-token prefill with     dq on about 80 sampled rows,
  seeded selections                              dk and dv on one whole block
                                                 per group.
Selections are compared bit for bit, outputs and lse within the tolerances of
the small parity tests. Inputs are the seeded synthetic workloads."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
from gpu_helpers import (bf16_out_to_f64, compare_lse, compare_out, dev_bf16, dev_i32,
                         dev_index, oracle_cfg, say)
from msa_synth import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

THREADS = 16


def lib_config(w):
    return msa.Config(num_kv_groups=w.G, heads_per_group=w.R, topk=w.topk,
                      index_dtype=msa.FP8_E4M3 if w.index_fp8 else msa.BF16)


def ora_config(w):
    return oracle_cfg(w.G, w.R, w.topk, w.index_fp8)


def check_decode_workload(orc, w):
    say("generating %s" % w.name)
    k_h, v_h, ki_h = wl.gen_caches(w)
    q_h, qi_h = wl.gen_queries(w, set_id=0)
    cfg = lib_config(w)
    kv_h = np.array(w.kv_lens, np.int32)
    k, v, ki = dev_bf16(k_h), dev_bf16(v_h), dev_index(ki_h)
    q, qi = dev_bf16(q_h), dev_index(qi_h)
    kv = dev_i32(kv_h)
    say("msa_decode %s" % w.name)
    sel, sc, out, lse = msa.decode(cfg, q, qi, ki, k, v, kv, want_scores=True, want_lse=True)
    say("msa_index_topk + msa_sparse_attn_decode %s" % w.name)
    sel2 = msa.index_topk(cfg, qi, ki, kv)
    out2 = msa.sparse_attn_decode(cfg, q, k, v, kv, sel2)
    torch.cuda.synchronize()
    del k, v, ki
    sel, sc = sel.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    out, lse = bf16_out_to_f64(out), lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(sel2.cpu().numpy(), sel)
    o2 = bf16_out_to_f64(out2)
    say("oracle %s (%d rows)" % (w.name, w.B))
    ocfg = ora_config(w)
    osel, osc = orc.index_topk(ocfg, qi_h, ki_h, kv_h, kv_h - 1, threads=THREADS)
    mism = int((sel.reshape(osel.shape) != osel).any(axis=(1, 2)).sum())
    say("%s: sel rows=%d mismatching=%d" % (w.name, w.B, mism))
    assert mism == 0
    assert np.array_equal(sc.reshape(osc.shape), osc)
    oout, olse = orc.sparse_attn(ocfg, q_h, k_h, v_h, kv_h, kv_h - 1, osel, threads=THREADS)
    compare_out(out.reshape(oout.shape), oout, w.name)
    compare_lse(lse.reshape(olse.shape), olse, w.name)
    compare_out(o2.reshape(oout.shape), oout, w.name + " (two calls)")
    torch.cuda.empty_cache()


def test_decode_B16_N131072_all_rows(orc):
    check_decode_workload(orc, wl.workload(2))


def test_decode_B4_N1M_all_rows(orc):
    check_decode_workload(orc, wl.workload(4))


def test_decode_B4_mixed_lengths_all_rows(orc):
    check_decode_workload(orc, wl.workload(4, mixed=True))


def test_decode_B16_ragged_rows_past_1024_blocks(orc):
    # Sixteen sequences of ragged lengths up to 196608 tokens: 1536 pooled
    # blocks per row, so the attention kernel runs its 16-wave form (the grid
    # fills the GPU) with every wave ranking a share of the row; the 1- and
    # 2-token sequences leave most waves' shares empty. Seeds of the c2 decode.
    lens = [196608, 150000, 140000, 131073, 131072, 100000, 70000, 1, 2, 129, 65536, 180000,
            160001, 5000, 196607, 135000]
    w = wl.Workload(2, "decode_B16_ragged_N196608", "decode", 16, 1, 196608, lens,
                    [n - 1 for n in lens])
    check_decode_workload(orc, w)


def test_decode_B16_N131072_fp8_index_all_rows(orc):
    check_decode_workload(orc, wl.workload(2, fp8_index=True))


def test_decode_B4_N1M_fp8_index_all_rows(orc):
    check_decode_workload(orc, wl.workload(4, fp8_index=True))


def stratified_rows(row0, T, C, n_random, seed):
    """Row offsets i (position row0 + i) to check: the block and top-k
    boundaries, the first and last row of every C-row chunk, then seeded
    uniform rows."""
    picks = {0, 1, 127, 128, 129, 2047, 2048, 2049, 4095, 4096}
    picks = {p - row0 for p in picks if row0 <= p < row0 + T}
    for c0 in range(0, T, C):
        picks.update((c0, min(c0 + C, T) - 1))
    rng = np.random.default_rng(seed)
    target = min(T, len(picks) + n_random)
    while len(picks) < target:
        picks.add(int(rng.integers(0, T)))
    return np.array(sorted(picks), np.int64)


def upload_caches(k_h, v_h, ki_h):
    return dict(k=dev_bf16(k_h), v=dev_bf16(v_h), ki=dev_index(ki_h))


def check_prefill_rows(orc, w, host, dev, q_h, qi_h, row0, rows_i, what):
    """msa_index_topk + msa_sparse_attn_prefill for query rows [row0, row0 + T)
    with keys [0, row0 + T) in the cache (capacity Nmax), then the listed rows
    against the oracle."""
    T = q_h.shape[1]
    cfg = lib_config(w)
    kv_h = np.array([row0 + T], np.int32)
    qs_h = np.array([row0], np.int32)
    q, qi = dev_bf16(q_h), dev_index(qi_h)
    kv, qs = dev_i32(kv_h), dev_i32(qs_h)
    say("%s: msa_index_topk T=%d q_start=%d" % (what, T, row0))
    sel, sc = msa.index_topk(cfg, qi, dev["ki"], kv, qs, want_scores=True)
    say("%s: msa_sparse_attn_prefill" % what)
    out, lse = msa.sparse_attn_prefill(cfg, q, dev["k"], dev["v"], kv, sel, q_start=qs,
                                       want_lse=True)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows_i).cuda()
    g_sel = sel[0].index_select(0, idx).cpu().numpy()
    g_sc = sc[0].index_select(0, idx).cpu().numpy().astype(np.float64)
    g_out = bf16_out_to_f64(out[0].index_select(0, idx))
    g_lse = lse[0].index_select(0, idx).cpu().numpy().astype(np.float64)
    del q, qi, sel, sc, out, lse
    torch.cuda.empty_cache()
    say("%s: oracle on %d rows" % (what, rows_i.size))
    ocfg = ora_config(w)
    rows = np.stack([np.zeros_like(rows_i), rows_i], axis=1).astype(np.int32)
    osel, osc = orc.index_topk(ocfg, qi_h, host["ki"], kv_h, qs_h, rows=rows, threads=THREADS)
    mism = int((g_sel.reshape(osel.shape) != osel).any(axis=(1, 2)).sum())
    say("%s: sel rows=%d mismatching=%d" % (what, rows_i.size, mism))
    assert mism == 0
    assert np.array_equal(g_sc.reshape(osc.shape), osc)
    oout, olse = orc.sparse_attn(ocfg, q_h, host["k"], host["v"], kv_h, qs_h, osel, rows=rows,
                                 threads=THREADS)
    compare_out(g_out.reshape(oout.shape), oout, what)
    compare_lse(g_lse.reshape(olse.shape), olse, what)


def test_prefill_L131072_sampled_rows(orc):
    w = wl.workload(3)
    say("generating %s" % w.name)
    k_h, v_h, ki_h = wl.gen_caches(w)
    q_h, qi_h = wl.gen_queries(w)
    host = dict(k=k_h, v=v_h, ki=ki_h)
    rows_i = stratified_rows(0, w.T, 32768, 2048 - 16, seed=31)
    assert rows_i.size >= 2048
    check_prefill_rows(orc, w, host, upload_caches(k_h, v_h, ki_h), q_h, qi_h, 0, rows_i,
                       w.name)


@pytest.fixture(scope="module")
def chunked_1m():
    """The 1M-token caches of the chunked prefill, on the host and the GPU."""
    w = wl.workload(5)
    say("generating %s caches" % w.name)
    k_h, v_h, ki_h = wl.gen_caches(w)
    host = dict(k=k_h, v=v_h, ki=ki_h)
    dev = upload_caches(k_h, v_h, ki_h)
    yield w, host, dev
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("chunk,n_random", [(0, 1000), (15, 300), (31, 200)])
def test_chunked_prefill_1M_fp8_sampled_rows(orc, chunked_1m, chunk, n_random):
    w, host, dev = chunked_1m
    C = w.chunk
    row0 = chunk * C
    q_h, qi_h = wl.gen_queries(w, row0=row0, rows=C)
    rows_i = stratified_rows(row0, C, C, n_random, seed=50 + chunk)
    check_prefill_rows(orc, w, host, dev, q_h, qi_h, row0, rows_i,
                       "%s chunk %d" % (w.name, chunk))


# The chunks the dense samples above leave out, in four groups of similar
# oracle cost (a row's cost grows with its position).
OTHER_CHUNKS = [c for c in range(32) if c not in (0, 15, 31)]
CHUNK_GROUPS = [OTHER_CHUNKS[0:10], OTHER_CHUNKS[10:17], OTHER_CHUNKS[17:23], OTHER_CHUNKS[23:]]


@pytest.mark.parametrize("group", range(len(CHUNK_GROUPS)))
def test_chunked_prefill_1M_fp8_every_chunk(orc, chunked_1m, group):
    """Every other chunk of the 1M chunked prefill, each run on the GPU as
    the benchmark runs it: its first and last row and 17 seeded rows against
    the oracle. With the dense samples of chunks 0, 15 and 31 (1515 rows) the
    chunked prefill is checked on 2066 rows, the first and last row of all 32
    chunks among them."""
    w, host, dev = chunked_1m
    C = w.chunk
    for chunk in CHUNK_GROUPS[group]:
        row0 = chunk * C
        q_h, qi_h = wl.gen_queries(w, row0=row0, rows=C)
        rng = np.random.default_rng(70 + chunk)
        picks = {0, C - 1}
        while len(picks) < 19:
            picks.add(int(rng.integers(1, C - 1)))
        rows_i = np.array(sorted(picks), np.int64)
        check_prefill_rows(orc, w, host, dev, q_h, qi_h, row0, rows_i,
                           "%s chunk %d" % (w.name, chunk))


def check_qblock(orc, w, host, dev, q_h, qi_h, row0, blocks, what, seed):
    """msa_index_topk_qblock + msa_sparse_attn_prefill_qblock for query rows
    [row0, row0 + T); the listed query-block slots' selections against the
    oracle, then 8 rows of each (first, last, six seeded) against the oracle
    attention with those selections."""
    import oracle
    T = q_h.shape[1]
    cfg = lib_config(w)
    kv_h = np.array([row0 + T], np.int32)
    qs_h = np.array([row0], np.int32)
    kv, qs = dev_i32(kv_h), dev_i32(qs_h)
    say("%s: msa_index_topk_qblock T=%d q_start=%d" % (what, T, row0))
    sel, sc = msa.index_topk_qblock(cfg, dev_index(qi_h), dev["ki"], kv, qs, want_scores=True)
    say("%s: msa_sparse_attn_prefill_qblock" % what)
    out, lse = msa.sparse_attn_prefill_qblock(cfg, dev_bf16(q_h), dev["k"], dev["v"], kv, sel,
                                              q_start=qs, want_lse=True)
    torch.cuda.synchronize()
    g_sel = sel[0].cpu().numpy()
    g_sc = sc[0].cpu().numpy().astype(np.float64)
    items = np.array([(0, s_) for s_ in blocks], np.int32)
    say("%s: oracle selections of %d query blocks" % (what, len(blocks)))
    ocfg = ora_config(w)
    osel, osc = orc.index_topk_qblock(ocfg, qi_h, host["ki"], kv_h, qs_h, items=items,
                                      threads=THREADS)
    mism = int((g_sel[blocks] != osel).any(axis=(1, 2)).sum())
    say("%s: qblock sel items=%d mismatching=%d" % (what, len(blocks), mism))
    assert mism == 0
    assert np.array_equal(g_sc[blocks], osc)
    rng = np.random.default_rng(seed)
    rows = []
    for s_ in blocks:
        lo = max(0, s_ * 128 - row0 % 128)
        hi = min(T, lo + 128 - (row0 % 128 if s_ == 0 else 0)) - 1
        picks = {lo, hi} | {int(x) for x in rng.integers(lo, hi + 1, size=6)}
        rows += [(0, i) for i in sorted(picks)]
    rows = np.array(rows, np.int32)
    idx = torch.from_numpy(rows[:, 1].astype(np.int64)).cuda()
    g_out = bf16_out_to_f64(out[0].index_select(0, idx))
    g_lse = lse[0].index_select(0, idx).cpu().numpy().astype(np.float64)
    rsel = oracle.qblock_rows_sel(sel.cpu().numpy(), qs_h, T, 128, rows=rows)
    oout, olse = orc.sparse_attn(ocfg, q_h, host["k"], host["v"], kv_h, qs_h, rsel, rows=rows,
                                 threads=THREADS)
    compare_out(g_out.reshape(oout.shape), oout, what)
    compare_lse(g_lse.reshape(olse.shape), olse, what)
    del sel, sc, out, lse
    torch.cuda.empty_cache()


def test_prefill_qblock_L131072_sampled_blocks(orc):
    w = wl.workload(3)
    say("generating %s" % w.name)
    k_h, v_h, ki_h = wl.gen_caches(w)
    q_h, qi_h = wl.gen_queries(w)
    host = dict(k=k_h, v=v_h, ki=ki_h)
    rng = np.random.default_rng(41)
    blocks = sorted({0, 1, 2, 15, 16, 17, 255, 256, 511, 1023} |
                    {int(x) for x in rng.integers(0, 1024, size=14)})
    check_qblock(orc, w, host, upload_caches(k_h, v_h, ki_h), q_h, qi_h, 0, blocks,
                 w.name + " qblock", seed=42)


@pytest.mark.parametrize("chunk,nblocks", [(0, 12), (5, 4)])
def test_chunked_prefill_1M_fp8_qblock_sampled_blocks(orc, chunked_1m, chunk, nblocks):
    w, host, dev = chunked_1m
    C = w.chunk
    row0 = chunk * C
    q_h, qi_h = wl.gen_queries(w, row0=row0, rows=C)
    rng = np.random.default_rng(60 + chunk)
    blocks = sorted({0, 255} | {int(x) for x in rng.integers(0, 256, size=nblocks - 2)})
    check_qblock(orc, w, host, dev, q_h, qi_h, row0, blocks,
                 "%s chunk %d qblock" % (w.name, chunk), seed=61 + chunk)


def structured_selection(T, G, K, S, seed):
    """Seeded selections [T, G, K] for a prefill whose row t sits at position
    t: every row keeps its own (diagonal) block d = t // S and K - 1 distinct
    earlier blocks, (a*k + c) mod d for k = 1 .. K-1 with a prime a above the
    block count (so the K - 1 values are distinct once d >= K - 1), or every
    earlier block when there are fewer; -1 pads. A test input of the backward,
    which takes the selections as given."""
    rng = np.random.default_rng(seed)
    diag = np.arange(T, dtype=np.int64) // S
    primes = np.array([1031, 1033, 1039, 1049, 1051, 1061, 1063, 1069], np.int64)
    assert diag[-1] < primes.min()
    sel = np.full((T, G, K), -1, np.int32)
    ks = np.arange(1, K, dtype=np.int64)
    for g in range(G):
        a = primes[rng.integers(0, primes.size, size=T)]
        c = rng.integers(0, 1 << 20, size=T)
        sel[:, g, 0] = diag
        cand = (a[:, None] * ks[None, :] + c[:, None]) % np.maximum(diag, 1)[:, None]
        full = diag >= K - 1
        sel[full, g, 1:] = cand[full]
        for t in np.flatnonzero(~full):
            sel[t, g, 1:1 + diag[t]] = np.arange(diag[t])
    return sel


def test_backward_L131072_sampled(orc):
    """msa_sparse_attn_backward on the 131072-token prefill (four passes of
    32768 rows, as the benchmark runs it) with seeded selections: dq on about
    80 sampled rows and dk, dv on every key of one block per group, whose
    attending rows span several tiles (and for one block two passes). The oracle runs on the same
    inputs with the selections of every other row removed: a row's dq depends
    on that row alone, and a key's dk and dv only on the rows that kept its
    block, so the sampled values are exact."""
    w = wl.workload(3)
    G, R, K, S, T, N = w.G, w.R, w.topk, 128, w.T, w.Nmax
    say("generating %s backward inputs" % w.name)
    k_h, v_h, _ = wl.gen_caches(w)
    q_h, _ = wl.gen_queries(w)
    dout_h = ms.fill_normal_bf16(np.empty_like(q_h), 9301)
    sel_h = structured_selection(T, G, K, S, seed=9302)[None]
    kv_h, qs_h = np.array([N], np.int32), np.array([0], np.int32)
    cfg = lib_config(w)
    q, k, v, dout = dev_bf16(q_h), dev_bf16(k_h), dev_bf16(v_h), dev_bf16(dout_h)
    kv, qs, sel = dev_i32(kv_h), dev_i32(qs_h), dev_i32(sel_h)
    say("%s: forward and backward on the GPU" % w.name)
    out, lse = msa.sparse_attn_prefill(cfg, q, k, v, kv, sel, q_start=qs, want_lse=True)
    gq, gk, gv = msa.sparse_attn_backward(cfg, q, k, v, kv, sel, out, lse, dout, q_start=qs)
    torch.cuda.synchronize()
    rows = stratified_rows(0, T, 32768, 64, seed=9303)
    # One block per group; block 760 is kept by rows of the third and the
    # fourth pass (its dk and dv add up over passes), the others by the last.
    blocks = [760, 880, 950, 1010]
    g_dq = gq[0].index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy().astype(np.float64)
    g_dk = [gk[0, g, blocks[g] * S:(blocks[g] + 1) * S].cpu().numpy().astype(np.float64)
            for g in range(G)]
    g_dv = [gv[0, g, blocks[g] * S:(blocks[g] + 1) * S].cpu().numpy().astype(np.float64)
            for g in range(G)]
    del q, k, v, dout, out, lse, gq, gk, gv, sel
    torch.cuda.empty_cache()
    keep = np.zeros((T, G), bool)
    keep[rows, :] = True
    for g in range(G):
        keep[:, g] |= (sel_h[0, :, g, :] == blocks[g]).any(axis=1)
    say("%s: oracle on %s rows per group" % (w.name, keep.sum(axis=0).tolist()))
    sel_o = np.where(keep[None, :, :, None], sel_h, -1).astype(np.int32)
    oq, ok_, ov = orc.sparse_attn_backward(oracle_cfg(G, R, K), q_h, k_h, v_h, kv_h, qs_h,
                                           sel_o, dout_h, threads=THREADS)
    compare_grad(g_dq, oq[0, rows], "dq (sampled rows)")
    compare_grad(np.concatenate(g_dk), np.concatenate(
        [ok_[0, g, blocks[g] * S:(blocks[g] + 1) * S] for g in range(G)]), "dk (one block per group)")
    compare_grad(np.concatenate(g_dv), np.concatenate(
        [ov[0, g, blocks[g] * S:(blocks[g] + 1) * S] for g in range(G)]), "dv (one block per group)")


def compare_grad(got, want, what):
    """The backward tolerances of the small parity tests: relative L2 <= 1e-2,
    max-abs <= 1e-2 * max|reference|."""
    scale = float(np.abs(want).max())
    err = float(np.abs(got - want).max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say("%s: max_abs=%.3e (ref max %.3e) rel_l2=%.3e" % (what, err, scale, rel))
    assert scale > 0.0, what
    assert rel <= 1e-2, (what, rel)
    assert err <= 1e-2 * scale, (what, err, scale)
