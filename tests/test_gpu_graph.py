"""Graph capture: msa_decode, msa_index_topk and the sparse calls captured in
a HIP graph give the eager results on every replay, with new inputs copied
into the captured buffers and eager work between replays."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
from gpu_helpers import lib_cfg, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def rand_inputs(B, T, N, G, R, seed):
    def bf(shape, s, integer=False):
        a = np.empty(shape, np.uint16)
        (ms.fill_int_bf16 if integer else ms.fill_normal_bf16)(a, seed * 10 + s)
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return dict(q=bf((B, T, G * R, 128), 1), k=bf((B, G, N, 128), 2), v=bf((B, G, N, 128), 3),
                qi=bf((B, T, G, 128), 4, True), ki=bf((B, N, 128), 5, True))


def test_graph_replays_match_eager():
    G, R, K, N, B = 4, 8, 16, 9000, 3
    cfg = lib_cfg(G, R, K)
    kv = torch.tensor([9000, 4100, 777], dtype=torch.int32, device="cuda")
    buf = rand_inputs(B, 1, N, G, R, seed=1)
    pbuf = rand_inputs(1, 200, 1000, G, R, seed=2)
    pkv = torch.tensor([1000], dtype=torch.int32, device="cuda")
    sel = torch.empty((B, 1, G, K), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 1, G * R, 128), dtype=torch.bfloat16, device="cuda")
    sel2 = torch.empty_like(sel)
    out2 = torch.empty_like(out)
    psel = torch.empty((1, 200, G, K), dtype=torch.int32, device="cuda")
    pout = torch.empty((1, 200, G * R, 128), dtype=torch.bfloat16, device="cuda")
    ws_dec = msa.workspace(cfg, B, 1, N, msa.WS_DECODE)
    ws_i = msa.workspace(cfg, B, 1, N, msa.WS_INDEX_TOPK)
    ws_s = msa.workspace(cfg, B, 1, N, msa.WS_SPARSE_DECODE)
    ws_p = msa.workspace(cfg, 1, 200, 1000, msa.WS_INDEX_TOPK)

    def calls():
        msa.decode(cfg, buf["q"], buf["qi"], buf["ki"], buf["k"], buf["v"], kv, sel=sel, out=out,
                   workspace=ws_dec)
        msa.index_topk(cfg, buf["qi"], buf["ki"], kv, sel=sel2, workspace=ws_i)
        msa.sparse_attn_decode(cfg, buf["q"], buf["k"], buf["v"], kv, sel2, out=out2,
                               workspace=ws_s)
        msa.index_topk(cfg, pbuf["qi"], pbuf["ki"], pkv, sel=psel, workspace=ws_p)
        msa.sparse_attn_prefill(cfg, pbuf["q"], pbuf["k"], pbuf["v"], pkv, psel, out=pout)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        new = rand_inputs(B, 1, N, G, R, seed=10 + rep)
        newp = rand_inputs(1, 200, 1000, G, R, seed=20 + rep)
        for k_ in buf:
            buf[k_].copy_(new[k_])
            pbuf[k_].copy_(newp[k_])
        torch.cuda.synchronize()
        say("graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (sel, out, sel2, out2, psel, pout)]
        _ = torch.ones(1000, device="cuda").sum().item()  # eager work between replays
        calls()  # eager on the same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, (sel, out, sel2, out2, psel, pout)):
            assert torch.equal(a, b), rep
        # msa_decode and the two-call form select the same blocks; their split
        # partials merge in a different order.
        assert torch.equal(sel, sel2)
        assert (out.float() - out2.float()).abs().max().item() <= 2e-2


def test_graph_backward_and_qblock_match_eager():
    """msa_sparse_attn_backward (list build, tile kernel, reductions),
    msa_index_topk_qblock and msa_sparse_attn_prefill_qblock captured in one
    graph: every replay equals the eager calls on the same inputs, bit for
    bit."""
    G, R, K, T = 2, 8, 8, 700
    cfg = lib_cfg(G, R, K)
    kv = torch.tensor([T], dtype=torch.int32, device="cuda")
    qs = torch.tensor([0], dtype=torch.int32, device="cuda")
    buf = rand_inputs(1, T, T, G, R, seed=3)
    dout = rand_inputs(1, T, T, G, R, seed=4)["q"]
    sel = msa.index_topk(cfg, buf["qi"], buf["ki"], kv, qs)
    out, lse = msa.sparse_attn_prefill(cfg, buf["q"], buf["k"], buf["v"], kv, sel, q_start=qs,
                                       want_lse=True)
    ws_b = msa.workspace(cfg, 1, T, T, msa.WS_SPARSE_BACKWARD)
    dq, dk, dv = msa.sparse_attn_backward(cfg, buf["q"], buf["k"], buf["v"], kv, sel, out, lse,
                                          dout, q_start=qs, workspace=ws_b)
    nq = msa.qblock_slots(T)
    qsel = torch.empty((1, nq, G, K), dtype=torch.int32, device="cuda")
    qout = torch.empty((1, T, G * R, 128), dtype=torch.bfloat16, device="cuda")
    qlse = torch.empty((1, T, G * R), dtype=torch.float32, device="cuda")

    def calls():
        msa.sparse_attn_backward(cfg, buf["q"], buf["k"], buf["v"], kv, sel, out, lse, dout,
                                 q_start=qs, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        msa.index_topk_qblock(cfg, buf["qi"], buf["ki"], kv, qs, sel=qsel)
        msa.sparse_attn_prefill_qblock(cfg, buf["q"], buf["k"], buf["v"], kv, qsel, q_start=qs,
                                       out=qout, lse=qlse)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        new = rand_inputs(1, T, T, G, R, seed=30 + rep)
        for k_ in buf:
            buf[k_].copy_(new[k_])
        dout.copy_(rand_inputs(1, T, T, G, R, seed=40 + rep)["q"])
        torch.cuda.synchronize()
        say("graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dq, dk, dv, qsel, qout, qlse)]
        _ = torch.ones(1000, device="cuda").sum().item()  # eager work between replays
        calls()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "qsel", "qout", "qlse"), got,
                              (dq, dk, dv, qsel, qout, qlse)):
            assert torch.equal(a, b), (rep, name)
