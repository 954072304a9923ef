"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with the hand-worked example, with brute force, with textbook dense
attention written independently in numpy, with a closed form, or with an
invariant of the method. ``test_oracle.py`` runs them on the real oracle;
``test_oracle_mutants.py`` plants mistakes in copies of the oracle's source
and checks that some pin catches each one.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from oracle import BF16, E4M3, Config
from msa_synth import float_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# helpers (independent of the oracle)

def bf16(x) -> np.ndarray:
    return float_to_bf16_bits(np.asarray(x, dtype=np.float32))


def e4m3_int(v: int) -> int:
    """E4M3FN code of a small integer, by search over the OCP format's value table."""
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        val = s * (m / 8.0) * 2.0 ** -6 if e == 0 else s * (1 + m / 8.0) * 2.0 ** (e - 7)
        if val == v and not (v == 0 and code & 0x80):
            return code
    raise ValueError(v)


def tiny_problem(rng, L, G, R, d, dI, S, K, B=1, T=None, q_start=None, kv_lens=None,
                 index_dtype=BF16, lo=-2, hi=2):
    """Random integer-valued index inputs and small-integer attention inputs."""
    T = L if T is None else T
    cfg = Config(groups=G, heads_per_group=R, head_dim=d, index_dim=dI, block_size=S, topk=K,
                 index_dtype=index_dtype)
    qi = rng.integers(lo, hi + 1, size=(B, T, G, dI))
    ki = rng.integers(lo, hi + 1, size=(B, L, dI))
    q = rng.standard_normal((B, T, G * R, d)).astype(np.float32)
    k = rng.standard_normal((B, G, L, d)).astype(np.float32)
    v = rng.standard_normal((B, G, L, d)).astype(np.float32)
    if index_dtype == E4M3:
        enc = np.vectorize(e4m3_int)
        qi_b, ki_b = enc(qi).astype(np.uint8), enc(ki).astype(np.uint8)
    else:
        qi_b, ki_b = bf16(qi), bf16(ki)
    kv_lens = np.full(B, L, np.int32) if kv_lens is None else np.asarray(kv_lens, np.int32)
    q_start = (kv_lens - T).astype(np.int32) if q_start is None else np.asarray(q_start, np.int32)
    return dict(cfg=cfg, qi=qi, ki=ki, qi_b=qi_b, ki_b=ki_b, q_b=bf16(q), k_b=bf16(k),
                v_b=bf16(v), kv_lens=kv_lens, q_start=q_start)


def as_f(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def numpy_masked_attention(q, k, v, allowed, tau):
    """Textbook softmax(tau * q k^T + mask) v for one head; allowed is a bool key mask."""
    z = tau * (k @ q)
    z = np.where(allowed, z, -np.inf)
    m = z.max()
    w = np.exp(z - m)
    w = w / w.sum()
    return w @ v, m + math.log(np.exp(z - m).sum())


def brute_force_topk(s_row, p, S, K):
    """Block choice by enumerating all subsets; the best subset has the largest
    multiset of (pooled score, -block) keys."""
    nv = p // S + 1
    pooled = [max(s_row[b * S: min(b * S + S, p + 1)]) for b in range(nv)]
    keys = [(pooled[b], -b) for b in range(nv)]
    best = None
    for subset in itertools.combinations(range(nv), min(K, nv)):
        ks = sorted((keys[b] for b in subset), reverse=True)
        if best is None or ks > best[0]:
            best = (ks, subset)
    chosen = sorted(best[1], key=lambda b: keys[b], reverse=True)
    return chosen + [-1] * (K - len(chosen))


def load_hand_example():
    with open(os.path.join(GOLDEN, "hand_example_L8.json")) as f:
        return json.load(f)


def hand_inputs(topk=2, q_start=0, kv_len=8, T=None):
    g = load_hand_example()
    L = g["config"]["L"]
    T = kv_len - q_start if T is None else T
    cfg = Config(groups=1, heads_per_group=2, head_dim=1, index_dim=1, block_size=2, topk=topk,
                 softmax_scale=1.0)
    qi = np.array(g["q_idx"], np.float32)[q_start:q_start + T].reshape(1, T, 1, 1)
    ki = np.array(g["k_idx"], np.float32).reshape(1, L, 1)
    q = np.zeros((1, T, 2, 1), np.float32)
    q[:, :, 0, 0] = 1.0
    kk = (np.arange(L) % 2).astype(np.float32).reshape(1, 1, L, 1)
    vv = np.arange(L, dtype=np.float32).reshape(1, 1, L, 1)
    return cfg, bf16(qi), bf16(ki), bf16(q), bf16(kk), bf16(vv), np.array([kv_len], np.int32), \
        np.array([q_start], np.int32)


# ---------------------------------------------------------------------------
# pins

def pin_decoders(orc):
    """bf16 and OCP E4M3FN decoding against values fixed by the formats."""
    assert orc.bf16_value(0x3F80) == 1.0
    assert orc.bf16_value(0xC000) == -2.0
    assert orc.bf16_value(0x3F81) == 1.0 + 2.0 ** -7
    assert orc.bf16_value(0x4080) == 4.0
    for code, val in ((0x38, 1.0), (0x40, 2.0), (0x44, 3.0), (0x48, 4.0), (0xB8, -1.0),
                      (0xC8, -4.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6),
                      (0x00, 0.0), (0x3C, 1.5)):
        assert orc.e4m3_value(code) == val, hex(code)
    assert math.isnan(orc.e4m3_value(0x7F))


def pin_hand_example_selection(orc):
    """Selection and pooled scores equal the hand-worked example, row by row."""
    g = load_hand_example()
    cfg, qi, ki, *_ , kv, qs = hand_inputs()
    sel, sc = orc.index_topk(cfg, qi, ki, kv, qs)
    assert sel[:, 0, :].tolist() == g["sel_topk2"], sel[:, 0, :].tolist()
    for t in range(8):
        pooled = g["pooled"][t]
        want = [pooled[b] if b >= 0 else -math.inf for b in g["sel_topk2"][t]]
        assert sc[t, 0, :].tolist() == want, (t, sc[t, 0, :].tolist(), want)
    cfg4, qi, ki, *_ , kv, qs = hand_inputs(topk=4)
    sel4, _ = orc.index_topk(cfg4, qi, ki, kv, qs)
    assert sel4[7, 0, :].tolist() == g["sel_topk4_row7"]
    pooled = orc.index_pool(cfg, qi, ki, kv, qs)
    for t in range(8):
        want = g["pooled"][t] + [-math.inf] * (4 - len(g["pooled"][t]))
        assert pooled[t, 0, :].tolist() == want, (t, pooled[t, 0, :].tolist(), want)


def pin_hand_example_attention(orc):
    """Attention outputs equal the example's closed forms (uniform and softmax heads)."""
    g = load_hand_example()
    e = math.e
    sig = e / (1 + e)
    closed_out = [0, sig, 1, 1 + sig, 1 + sig, 3 + sig, 1 + sig, 1 + sig]
    closed_lse = [0, math.log(1 + e), math.log(2 + e)] + [math.log(2 + 2 * e)] * 5
    cfg, qi, ki, q, k, v, kv, qs = hand_inputs()
    sel, _ = orc.index_topk(cfg, qi, ki, kv, qs)
    out, lse = orc.sparse_attn(cfg, q, k, v, kv, qs, sel)
    for t in range(8):
        assert abs(out[t, 0, 0] - closed_out[t]) < 1e-12, (t, out[t, 0, 0])
        assert abs(out[t, 0, 0] - g["out_head0_softmax"][t]) < 1e-9
        assert abs(lse[t, 0] - closed_lse[t]) < 1e-12, (t, lse[t, 0])
        assert abs(lse[t, 0] - g["lse_head0_softmax"][t]) < 1e-9
        assert abs(out[t, 1, 0] - g["out_head1_uniform"][t]) < 1e-12, (t, out[t, 1, 0])
        assert abs(out[t, 1, 0] - float(np.mean(g["attended_keys"][t]))) < 1e-12


def pin_hand_example_variants(orc):
    """K >= #blocks is dense causal (uniform head = t/2); decode and chunked calls
    give the same rows; a negative-zero index query ties like +0."""
    cfg4, qi, ki, q, k, v, kv, qs = hand_inputs(topk=4)
    sel, _ = orc.index_topk(cfg4, qi, ki, kv, qs)
    out, _ = orc.sparse_attn(cfg4, q, k, v, kv, qs, sel)
    for t in range(8):
        assert abs(out[t, 1, 0] - t / 2.0) < 1e-12
    cfg, qi, ki, q, k, v, kv, qs = hand_inputs()
    full_sel, _ = orc.index_topk(cfg, qi, ki, kv, qs)
    full_out, full_lse = orc.sparse_attn(cfg, q, k, v, kv, qs, full_sel)
    # decode of the last token
    _, qi1, ki1, q1, k1, v1, kv1, qs1 = hand_inputs(q_start=7)
    s1, _ = orc.index_topk(cfg, qi1, ki1, kv1, qs1)
    assert s1[0].tolist() == full_sel[7].tolist()
    o1, l1 = orc.sparse_attn(cfg, q1, k1, v1, kv1, qs1, s1)
    assert np.array_equal(o1[0], full_out[7]) and np.array_equal(l1[0], full_lse[7])
    # chunk [4, 8) against the full cache
    _, qi4, ki4, q4, k4, v4, kv4, qs4 = hand_inputs(q_start=4)
    s4, _ = orc.index_topk(cfg, qi4, ki4, kv4, qs4)
    assert s4.tolist() == full_sel[4:].tolist()
    # -0.0 as the index query of row 6 (bits 0x8000)
    qi_neg = qi.copy()
    qi_neg[0, 6, 0, 0] = 0x8000
    sn, scn = orc.index_topk(cfg, qi_neg, ki, kv, qs)
    assert sn[6, 0].tolist() == [0, 1]


def pin_brute_force_selection(orc, cases=60, seed=1):
    """Oracle selection equals exhaustive subset search on tiny random inputs."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        L = int(rng.integers(1, 17))
        S = int(rng.choice([1, 2, 4]))
        K = int(rng.integers(1, 6))
        G = int(rng.integers(1, 3))
        dI = int(rng.integers(1, 3))
        pr = tiny_problem(rng, L, G, 1, 1, dI, S, K, index_dtype=int(case % 2))
        sel, sc = orc.index_topk(pr["cfg"], pr["qi_b"], pr["ki_b"], pr["kv_lens"],
                                 pr["q_start"])
        pooled = orc.index_pool(pr["cfg"], pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
        for t in range(L):
            for g in range(G):
                s_row = [sum(int(pr["qi"][0, t, g, c]) * int(pr["ki"][0, j, c])
                             for c in range(dI)) for j in range(t + 1)]
                nb = -(-L // S)
                want_pool = [max(s_row[b * S: min(b * S + S, t + 1)]) if b * S <= t
                             else -math.inf for b in range(nb)]
                assert pooled[t, g].tolist() == want_pool, (case, t, g)
                want = brute_force_topk(s_row, t, S, K)
                assert sel[t, g].tolist() == want, (case, t, g, sel[t, g].tolist(), want)
                for kk, b in enumerate(want):
                    if b >= 0:
                        assert sc[t, g, kk] == max(s_row[b * S: min(b * S + S, t + 1)])


def pin_token_level_and_single_block(orc, seed=2):
    """S = 1 is token-level top-k (stable sort of scores); S >= L gives one block."""
    rng = np.random.default_rng(seed)
    L, K = 12, 5
    pr = tiny_problem(rng, L, 1, 1, 1, 2, 1, K)
    sel, _ = orc.index_topk(pr["cfg"], pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    for t in range(L):
        s = (pr["ki"][0, :t + 1] @ pr["qi"][0, t, 0]).astype(np.int64)
        order = sorted(range(t + 1), key=lambda j: (-s[j], j))[:K]
        assert sel[t, 0].tolist() == order + [-1] * (K - len(order))
    pr = tiny_problem(rng, L, 1, 1, 1, 2, 16, 3)
    sel, _ = orc.index_topk(pr["cfg"], pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    assert (sel[:, 0, 0] == 0).all() and (sel[:, 0, 1:] == -1).all()


def pin_selection_invariants(orc, seed=3):
    """Positive integer scaling of q_I keeps sel; permuting keys inside a block that
    lies wholly in the past keeps sel; bf16 and E4M3 storage select alike."""
    rng = np.random.default_rng(seed)
    L, S, K = 64, 8, 3
    pr = tiny_problem(rng, L, 2, 1, 1, 4, S, K)
    cfg = pr["cfg"]
    sel, _ = orc.index_topk(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    sel3, _ = orc.index_topk(cfg, bf16(3 * pr["qi"]), pr["ki_b"], pr["kv_lens"], pr["q_start"])
    assert np.array_equal(sel, sel3)
    ki_perm = pr["ki"].copy()
    ki_perm[0, 8:16] = ki_perm[0, 8:16][rng.permutation(8)]
    selp, _ = orc.index_topk(cfg, pr["qi_b"], bf16(ki_perm), pr["kv_lens"], pr["q_start"])
    assert np.array_equal(sel[16:], selp[16:])
    enc = np.vectorize(e4m3_int)
    cfg8 = Config(**{**cfg.__dict__, "index_dtype": E4M3})
    sel8, _ = orc.index_topk(cfg8, enc(pr["qi"]).astype(np.uint8),
                             enc(pr["ki"]).astype(np.uint8), pr["kv_lens"], pr["q_start"])
    assert np.array_equal(sel, sel8)


def pin_sparse_vs_numpy(orc, cases=12, seed=4):
    """Sparse attention equals an independent numpy masked-softmax attention over
    the keys of the chosen blocks; with K >= #blocks it equals dense causal."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        L = int(rng.integers(2, 40))
        S = int(rng.choice([1, 2, 4, 8]))
        G, R, d = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 9))
        K = int(rng.integers(1, 5)) if case % 3 else (L + S - 1) // S
        pr = tiny_problem(rng, L, G, R, d, 2, S, K)
        cfg = pr["cfg"]
        sel, _ = orc.index_topk(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
        out, lse = orc.sparse_attn(cfg, pr["q_b"], pr["k_b"], pr["v_b"], pr["kv_lens"],
                                   pr["q_start"], sel)
        dout, dlse = orc.dense_causal(cfg, pr["q_b"], pr["k_b"], pr["v_b"], pr["kv_lens"],
                                      pr["q_start"])
        q, k, v = as_f(pr["q_b"]), as_f(pr["k_b"]), as_f(pr["v_b"])
        tau = 1.0 / math.sqrt(d)
        for t in range(L):
            for h in range(G * R):
                g = h // R
                blocks = set(int(b) for b in sel[t, g] if b >= 0)
                allowed = np.array([(j <= t) and (j // S in blocks) for j in range(L)])
                o_ref, l_ref = numpy_masked_attention(q[0, t, h], k[0, g], v[0, g], allowed, tau)
                assert np.allclose(out[t, h], o_ref, rtol=0, atol=1e-12), (case, t, h)
                assert abs(lse[t, h] - l_ref) < 1e-12
                causal = np.arange(L) <= t
                o_d, l_d = numpy_masked_attention(q[0, t, h], k[0, g], v[0, g], causal, tau)
                assert np.allclose(dout[t, h], o_d, rtol=0, atol=1e-12)
                assert abs(dlse[t, h] - l_d) < 1e-12
                if K * S >= L:
                    assert np.allclose(out[t, h], dout[t, h], rtol=0, atol=1e-12)


def pin_attention_invariants(orc, seed=5):
    """Constant V gives that constant; q = 0 gives the mean of V over the chosen
    keys; splitting the chosen blocks in two and merging by log-sum-exp gives the
    full result; decode equals the last prefill row."""
    rng = np.random.default_rng(seed)
    L, G, R, d, S, K = 48, 2, 2, 8, 4, 4
    pr = tiny_problem(rng, L, G, R, d, 3, S, K)
    cfg = pr["cfg"]
    sel, _ = orc.index_topk(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    vc = np.full_like(pr["v_b"], bf16(np.float32(1.75)))
    out, _ = orc.sparse_attn(cfg, pr["q_b"], pr["k_b"], vc, pr["kv_lens"], pr["q_start"], sel)
    assert np.allclose(out, 1.75, rtol=0, atol=1e-12)
    q0 = np.zeros_like(pr["q_b"])
    out0, _ = orc.sparse_attn(cfg, q0, pr["k_b"], pr["v_b"], pr["kv_lens"], pr["q_start"], sel)
    v = as_f(pr["v_b"])
    for t in range(L):
        for h in range(G * R):
            g = h // R
            keys = [j for j in range(t + 1) if j // S in set(sel[t, g].tolist())]
            assert np.allclose(out0[t, h], v[0, g, keys].mean(axis=0), rtol=0, atol=1e-12)
    out, lse = orc.sparse_attn(cfg, pr["q_b"], pr["k_b"], pr["v_b"], pr["kv_lens"],
                               pr["q_start"], sel)
    half = K // 2
    sa = sel.copy()
    sa[:, :, half:] = -1
    sb = sel.copy()
    sb[:, :, :half] = -1
    oa, la = orc.sparse_attn(cfg, pr["q_b"], pr["k_b"], pr["v_b"], pr["kv_lens"], pr["q_start"], sa)
    ob, lb = orc.sparse_attn(cfg, pr["q_b"], pr["k_b"], pr["v_b"], pr["kv_lens"], pr["q_start"], sb)
    for t in range(L):
        for h in range(G * R):
            parts = [(la[t, h], oa[t, h]), (lb[t, h], ob[t, h])]
            parts = [pp for pp in parts if np.isfinite(pp[0])]
            m = max(pp[0] for pp in parts)
            ws = [math.exp(pp[0] - m) for pp in parts]
            merged = sum(w * pp[1] for w, pp in zip(ws, parts)) / sum(ws)
            assert np.allclose(merged, out[t, h], rtol=0, atol=1e-12), (t, h)
            assert abs(m + math.log(sum(ws)) - lse[t, h]) < 1e-12
    # decode: one query at position L-1 against the same caches
    qd = pr["q_b"][:, L - 1:L]
    qid = pr["qi_b"][:, L - 1:L]
    qs = np.array([L - 1], np.int32)
    sd, _ = orc.index_topk(cfg, qid, pr["ki_b"], pr["kv_lens"], qs)
    assert np.array_equal(sd[0], sel[L - 1])
    od, ld = orc.sparse_attn(cfg, qd, pr["k_b"], pr["v_b"], pr["kv_lens"], qs, sd)
    assert np.array_equal(od[0], out[L - 1]) and np.array_equal(ld[0], lse[L - 1])


def pin_mixed_lengths_and_stride(orc, seed=6):
    """Rows of a batch with per-sequence lengths inside a larger cache stride equal the
    same rows computed alone with a tight cache (keys past kv_len are never read)."""
    rng = np.random.default_rng(seed)
    G, R, d, dI, S, K = 2, 2, 4, 2, 4, 3
    lens = [37, 20, 64]
    Nmax = 64
    pr = tiny_problem(rng, Nmax, G, R, d, dI, S, K, B=3, T=1, kv_lens=lens)
    cfg = pr["cfg"]
    # garbage beyond each kv_len must not matter
    ki_b, k_b, v_b = pr["ki_b"].copy(), pr["k_b"].copy(), pr["v_b"].copy()
    for b, n in enumerate(lens):
        ki_b[b, n:] = bf16(np.float32(4.0))
        k_b[b, :, n:] = bf16(np.float32(9.0))
        v_b[b, :, n:] = bf16(np.float32(-9.0))
    sel, _ = orc.index_topk(cfg, pr["qi_b"], ki_b, pr["kv_lens"], pr["q_start"])
    out, lse = orc.sparse_attn(cfg, pr["q_b"], k_b, v_b, pr["kv_lens"], pr["q_start"], sel)
    for b, n in enumerate(lens):
        s1, _ = orc.index_topk(cfg, pr["qi_b"][b:b + 1], pr["ki_b"][b:b + 1, :n],
                               np.array([n], np.int32), np.array([n - 1], np.int32))
        assert np.array_equal(s1[0], sel[b])
        o1, l1 = orc.sparse_attn(cfg, pr["q_b"][b:b + 1], pr["k_b"][b:b + 1, :, :n],
                                 pr["v_b"][b:b + 1, :, :n], np.array([n], np.int32),
                                 np.array([n - 1], np.int32), s1)
        assert np.allclose(o1[0], out[b], rtol=0, atol=1e-12)


def pin_cache_append(orc, seed=7):
    """Appending the last T tokens of a cache (given as [B,T,G,d] rows) into a
    cache that lacks them rebuilds the full cache bit for bit, and the decode
    of the last token then equals the decode on the full cache; rows whose
    position falls outside the cache are skipped and nothing else changes."""
    import oracle
    rng = np.random.default_rng(seed)
    G, R, d, dI, S, K = 3, 2, 4, 2, 4, 3
    B, L, T = 2, 29, 3
    pr = tiny_problem(rng, L, G, R, d, dI, S, K, B=B, T=1)
    cfg = pr["cfg"]
    full_k, full_v, full_ki = pr["k_b"], pr["v_b"], pr["ki_b"]
    # The new rows in the call's layout, written out element by element.
    k_new = np.zeros((B, T, G, d), np.uint16)
    v_new = np.zeros((B, T, G, d), np.uint16)
    ki_new = np.zeros((B, T, dI), np.uint16)
    for b in range(B):
        for t in range(T):
            ki_new[b, t] = full_ki[b, L - T + t]
            for g in range(G):
                k_new[b, t, g] = full_k[b, g, L - T + t]
                v_new[b, t, g] = full_v[b, g, L - T + t]
    old_k, old_v, old_ki = full_k.copy(), full_v.copy(), full_ki.copy()
    old_k[:, :, L - T:] = 0x7F80   # +inf bits: must all be overwritten
    old_v[:, :, L - T:] = 0x7F80
    old_ki[:, L - T:] = 0x7F80
    pos0 = np.full(B, L - T, np.int32)
    nk, nv, nki = oracle.cache_append(k_new, v_new, ki_new, pos0, old_k, old_v, old_ki)
    assert np.array_equal(nk, full_k) and np.array_equal(nv, full_v)
    assert np.array_equal(nki, full_ki)
    assert np.all(old_k[:, :, L - T:] == 0x7F80)   # inputs untouched
    kv = np.full(B, L, np.int32)
    qs = kv - 1
    s_full, _ = orc.index_topk(cfg, pr["qi_b"], full_ki, kv, qs)
    s_app, _ = orc.index_topk(cfg, pr["qi_b"], nki, kv, qs)
    assert np.array_equal(s_full, s_app)
    o_full, l_full = orc.sparse_attn(cfg, pr["q_b"], full_k, full_v, kv, qs, s_full)
    o_app, l_app = orc.sparse_attn(cfg, pr["q_b"], nk, nv, kv, qs, s_app)
    assert np.array_equal(o_full, o_app) and np.array_equal(l_full, l_app)
    # Out-of-range rows are skipped: sequence 0 starts two rows before the
    # cache end (row 2 falls outside), sequence 1 two rows before position 0.
    pos0 = np.array([L - 2, -2], np.int32)
    nk, nv, nki = oracle.cache_append(k_new, v_new, ki_new, pos0, old_k, old_v, old_ki)
    assert np.array_equal(nk[0, :, L - 2:], k_new[0, :2].transpose(1, 0, 2))
    assert np.array_equal(nki[0, L - 2:], ki_new[0, :2])
    assert np.array_equal(nk[1, :, 0], k_new[1, 2]) and np.array_equal(nki[1, 0], ki_new[1, 2])
    keep = np.ones(nk.shape, bool)
    keep[0, :, L - 2:] = False
    keep[1, :, 0] = False
    assert np.array_equal(nk[keep], old_k[keep]) and np.array_equal(nv[keep], old_v[keep])


def pin_qblock_selection(orc, seed=8):
    """Query-block-shared selection against brute force (numpy scores, a max
    over the block's rows and keys, a sort), against the token-level
    selection where they must agree (one-row blocks; blocks whose rows share
    one index query select as their last row), against a split of the call
    at block boundaries; and the slot map of qblock_rows_sel by hand."""
    import oracle
    rng = np.random.default_rng(seed)
    G, R, d, dI, S, K = 2, 1, 2, 3, 4, 3
    L = 40
    for q0, T in ((5, 17), (8, 12), (0, 40), (13, 1), (36, 4)):
        pr = tiny_problem(rng, L, G, R, d, dI, S, K, B=1, T=T, q_start=[q0], kv_lens=[L])
        cfg = pr["cfg"]
        nslot = oracle.qblock_slots(T, S)
        sel, sc = orc.index_topk_qblock(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
        assert sel.shape == (nslot, G, K)
        qi, ki = pr["qi"][0].astype(np.float64), pr["ki"][0].astype(np.float64)
        for slot in range(nslot):
            qb = q0 // S + slot
            rows = [i for i in range(T) if (q0 + i) // S == qb and q0 + i < L]
            for g in range(G):
                if not rows:
                    assert (sel[slot, g] == -1).all() and np.isneginf(sc[slot, g]).all()
                    continue
                best = {}
                for i in rows:
                    p = q0 + i
                    for j in range(p + 1):
                        v = float(qi[i, g] @ ki[j])
                        best[j // S] = max(best.get(j // S, -np.inf), v)
                order = sorted(best.items(), key=lambda kv: (-kv[1], kv[0]))[:K]
                want = [b for b, _ in order] + [-1] * (K - len(order))
                assert list(sel[slot, g]) == want, (q0, T, slot, g, list(sel[slot, g]), want)
                assert np.allclose(sc[slot, g][:len(order)], [v for _, v in order], rtol=0,
                                   atol=0)
    # One-row calls select as the token-level index branch.
    pr = tiny_problem(rng, L, G, R, d, dI, S, K, B=2, T=1, kv_lens=[L, 23])
    cfg = pr["cfg"]
    sb, _ = orc.index_topk_qblock(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    st, _ = orc.index_topk(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    assert np.array_equal(sb, st)
    # Rows sharing one index query: the block selects as its last row.
    pr = tiny_problem(rng, L, G, R, d, dI, S, K, B=1, T=L, q_start=[0], kv_lens=[L])
    cfg = pr["cfg"]
    qi_b = pr["qi_b"].copy()
    for qb in range(L // S):
        qi_b[0, qb * S:qb * S + S] = qi_b[0, qb * S + 1]
    sb, _ = orc.index_topk_qblock(cfg, qi_b, pr["ki_b"], pr["kv_lens"], pr["q_start"])
    last = np.array([[0, qb * S + S - 1] for qb in range(L // S)], np.int32)
    st, _ = orc.index_topk(cfg, qi_b, pr["ki_b"], pr["kv_lens"], pr["q_start"], rows=last)
    assert np.array_equal(sb[:L // S], st)
    # Two calls split at a block boundary select as one call.
    whole, _ = orc.index_topk_qblock(cfg, pr["qi_b"], pr["ki_b"], pr["kv_lens"], pr["q_start"])
    a, _ = orc.index_topk_qblock(cfg, pr["qi_b"][:, :16], pr["ki_b"], np.array([16], np.int32),
                                 np.array([0], np.int32))
    b, _ = orc.index_topk_qblock(cfg, pr["qi_b"][:, 16:], pr["ki_b"], pr["kv_lens"],
                                 np.array([16], np.int32))
    assert np.array_equal(whole[:4], a[:4]) and np.array_equal(whole[4:10], b[:6])
    # Slot map: q_start 6, S 4 -> rows 0,1 in slot 0, rows 2..5 in slot 1, row 6 in slot 2.
    blk = np.arange(1 * 3 * 1 * 1).reshape(1, 3, 1, 1)
    rows_sel = oracle.qblock_rows_sel(blk, [6], 7, 4)
    assert list(rows_sel[:, 0, 0]) == [0, 0, 1, 1, 1, 1, 2]


def pin_backward_finite_differences(orc, seed=9):
    """Gradients of the sparse branch against central differences of the
    forward oracle: inputs are multiples of 1/8 in (-1, 1) and one element
    moves by +-1/64 (both exactly representable in bf16); the loss is
    sum(out * dout) with a fixed selection that mixes blocks, skips some and
    cuts the diagonal one."""
    rng = np.random.default_rng(seed)
    G, R, d, S, K, L = 2, 2, 4, 4, 2, 14
    cfg = Config(groups=G, heads_per_group=R, head_dim=d, index_dim=2, block_size=S, topk=K)
    H = G * R
    q = rng.integers(-7, 8, size=(1, L, H, d)) / 8.0
    k = rng.integers(-7, 8, size=(1, G, L, d)) / 8.0
    v = rng.integers(-7, 8, size=(1, G, L, d)) / 8.0
    dout = rng.integers(-7, 8, size=(1, L, H, d)) / 8.0
    kv = np.array([L], np.int32)
    qs = np.array([0], np.int32)
    sel = np.full((1, L, G, K), -1, np.int32)
    for i in range(L):
        nb = i // S + 1
        for g in range(G):
            picks = rng.choice(nb, size=min(K, nb), replace=False)
            sel[0, i, g, :len(picks)] = picks
    dq, dk, dv = orc.sparse_attn_backward(cfg, bf16(q), bf16(k), bf16(v), kv, qs, sel, bf16(dout))

    def loss(qq, kk, vv):
        out, _ = orc.sparse_attn(cfg, bf16(qq), bf16(kk), bf16(vv), kv, qs,
                                 sel.reshape(L, G, K))
        return float((out.reshape(1, L, H, d) * dout).sum())

    h = 1.0 / 64
    checks = 0
    for arr, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            if name == "q":
                num = (loss(plus, k, v) - loss(minus, k, v)) / (2 * h)
            elif name == "k":
                num = (loss(q, plus, v) - loss(q, minus, v)) / (2 * h)
            else:
                num = (loss(q, k, plus) - loss(q, k, minus)) / (2 * h)
            assert abs(num - grad[idx]) <= 2e-3 + 2e-3 * abs(num), (name, idx, num, grad[idx])
            checks += 1
    assert checks == 36
    # Keys of a block no row keeps get zero gradients.
    sel2 = np.where(sel == 1, -1, sel)
    _, dk2, dv2 = orc.sparse_attn_backward(cfg, bf16(q), bf16(k), bf16(v), kv, qs, sel2,
                                           bf16(dout))
    assert not dk2[:, :, S:2 * S].any() and not dv2[:, :, S:2 * S].any()
    assert dk2[:, :, :S].any() and dv2[:, :, :S].any()


def pin_backward_dense_autograd(orc, seed=10):
    """With every causal block kept, the sparse branch is dense causal attention:
    its gradients equal torch autograd of a float64 causal softmax attention
    (matmul, mask, softmax) on the CPU."""
    import torch
    rng = np.random.default_rng(seed)
    G, R, d, S, L = 2, 3, 8, 4, 19
    K = (L - 1) // S + 1
    cfg = Config(groups=G, heads_per_group=R, head_dim=d, index_dim=2, block_size=S, topk=K)
    H = G * R
    qb = bf16(rng.standard_normal((1, L, H, d)))
    kb = bf16(rng.standard_normal((1, G, L, d)))
    vb = bf16(rng.standard_normal((1, G, L, d)))
    db = bf16(rng.standard_normal((1, L, H, d)))
    sel = np.full((1, L, G, K), -1, np.int32)
    for i in range(L):
        sel[0, i, :, : i // S + 1] = np.arange(i // S + 1)
    dq, dk, dv = orc.sparse_attn_backward(cfg, qb, kb, vb, np.array([L], np.int32),
                                          np.array([0], np.int32), sel, db)
    q = torch.tensor(as_f(qb)[0], requires_grad=True)          # [L, H, d]
    k = torch.tensor(as_f(kb)[0], requires_grad=True)          # [G, L, d]
    v = torch.tensor(as_f(vb)[0], requires_grad=True)
    outs = []
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))
    for h in range(H):
        g = h // R
        z = (q[:, h, :] @ k[g].T) / math.sqrt(d)
        z = z.masked_fill(~mask, float("-inf"))
        outs.append(torch.softmax(z, dim=1) @ v[g])
    out = torch.stack(outs, dim=1)
    (out * torch.tensor(as_f(db)[0])).sum().backward()
    assert np.allclose(dq[0], q.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk[0], k.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv[0], v.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_index_project(orc, seed=11):
    """Index projections against values the linear map fixes: one-hot weight
    rows copy one hidden element each (so every output is a known input bit
    pattern, whatever the head), constant weights per head give h times the
    head's constant (the head order: G index queries, then the index key),
    and a sum that lies exactly halfway between two bf16 values rounds to the
    even one."""
    import oracle
    b1 = lambda x: int(np.asarray(bf16(x)).reshape(-1)[0])   # one bf16 bit pattern
    rng = np.random.default_rng(seed)
    G, dI, h, M = 3, 8, 16, 5
    hid = bf16(rng.standard_normal((M, h)))
    pick = rng.integers(0, h, size=(G + 1) * dI)
    w = np.zeros(((G + 1) * dI, h), np.uint16)
    w[np.arange((G + 1) * dI), pick] = 0x3F80               # 1.0
    q, k, qb, kb = oracle.index_project(hid, w, G, dI)
    want = hid[:, pick]                                       # [M, (G+1)*dI] bits
    assert np.array_equal(qb.reshape(M, G * dI), want[:, :G * dI])
    assert np.array_equal(kb, want[:, G * dI:])
    # Constant weights per head: head g (g = G is the index key) uses 2^-(g+1).
    ones = np.full((M, h), 0x3F80, np.uint16)
    wc = np.concatenate([np.full((dI, h), b1(2.0 ** -(g + 1)), np.uint16)
                         for g in range(G + 1)])
    q, k, qb, kb = oracle.index_project(ones, wc, G, dI)
    for g in range(G):
        assert np.all(q[:, g, :] == h * 2.0 ** -(g + 1)), g
    assert np.all(k == h * 2.0 ** -(G + 1))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: it rounds to 1.0 (even);
    # 1 + 3 * 2^-8 rounds up to 1 + 2^-6.
    hv = np.zeros((2, h), np.uint16)
    hv[0, 0], hv[0, 1] = 0x3F80, b1(2.0 ** -8)
    hv[1, 0], hv[1, 1] = 0x3F80, b1(3 * 2.0 ** -8)
    wt = np.zeros(((G + 1) * dI, h), np.uint16)
    wt[:, 0] = wt[:, 1] = 0x3F80
    q, k, qb, kb = oracle.index_project(hv, wt, G, dI)
    assert np.all(qb[0] == 0x3F80) and np.all(kb[0] == 0x3F80)
    assert np.all(qb[1] == b1(1 + 2.0 ** -6)) and np.all(q[1] == 1 + 3 * 2.0 ** -8)


ALL_PINS = [pin_decoders, pin_hand_example_selection, pin_hand_example_attention,
            pin_hand_example_variants, pin_brute_force_selection,
            pin_token_level_and_single_block, pin_selection_invariants, pin_sparse_vs_numpy,
            pin_attention_invariants, pin_mixed_lengths_and_stride, pin_cache_append,
            pin_qblock_selection, pin_backward_finite_differences, pin_backward_dense_autograd,
            pin_index_project]


def run_all(orc):
    """Runs every pin; returns {pin name: error text} for the pins that failed."""
    failures = {}
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as exc:  # a mutant may also crash or reject its inputs
            failures[pin.__name__] = "%s: %s" % (type(exc).__name__, exc)
    return failures
