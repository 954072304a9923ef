"""msa_decode_no_alloc (the decode step with the library's fixed scratch
array) against msa_decode (caller workspace) through the C ABI: two calls in
a row on one GPU, the second with a smaller batch and cache, so the second
runs on scratch the first left behind. The two entry points run the same
kernels in the same order, so selections, scores, outputs and lse must agree
bit for bit (stricter than the parity tolerances); the selections are also
checked against the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
from gpu_helpers import dev_bf16, dev_i32, lib_cfg, oracle_cfg, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def problem(B, N, G, R, seed):
    H = G * R
    q = ms.fill_normal_bf16(np.empty((B, 1, H, 128), np.uint16), seed + 1)
    k = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 2)
    v = ms.fill_normal_bf16(np.empty((B, G, N, 128), np.uint16), seed + 3)
    qi = ms.fill_int_bf16(np.empty((B, 1, G, 128), np.uint16), seed + 4, -4, 4)
    ki = ms.fill_int_bf16(np.empty((B, N, 128), np.uint16), seed + 5, -4, 4)
    return dict(q=q, k=k, v=v, qi=qi, ki=ki)


def run_both(orc, G, R, K, lens, N, seed):
    B = len(lens)
    pr = problem(B, N, G, R, seed)
    cfg = lib_cfg(G, R, K)
    d = {n: dev_bf16(a) for n, a in pr.items()}
    kv = dev_i32(lens)
    need = msa.workspace_size(cfg, B, 1, N, msa.WS_DECODE)
    assert need <= msa.decode_no_alloc_max_scratch()
    say("msa_decode_no_alloc B=%d N=%d G=%d R=%d K=%d (scratch %d bytes)" % (B, N, G, R, K, need))
    sel = torch.full((B, 1, G, K), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty((B, 1, G, K), dtype=torch.float32, device="cuda")
    out = torch.empty((B, 1, G * R, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, G * R), dtype=torch.float32, device="cuda")
    msa.decode_no_alloc(cfg, d["q"], d["qi"], d["ki"], d["k"], d["v"], kv, sel, out,
                        sel_scores=sc, lse=lse)
    torch.cuda.synchronize()
    say("msa_decode (workspace) on the same inputs")
    sel2, sc2, out2, lse2 = msa.decode(cfg, d["q"], d["qi"], d["ki"], d["k"], d["v"], kv,
                                       want_scores=True, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    assert torch.equal(sc, sc2)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)
    kvh = np.array(lens, np.int32)
    osel, _ = orc.index_topk(oracle_cfg(G, R, K), pr["qi"], pr["ki"], kvh, kvh - 1)
    assert np.array_equal(sel.cpu().numpy().reshape(osel.shape), osel)


def test_no_alloc_decode_matches_workspace_decode_twice(orc):
    # First call: 16 ragged sequences of up to 20000 tokens (about 2.3 MiB of
    # scratch); second call: 3 shorter sequences on the scratch it left.
    run_both(orc, 4, 8, 16, [20000, 19999, 1, 129, 2048, 128, 5000, 20000, 17, 333, 4096, 4097,
                             12000, 8191, 8192, 8193], 20000, seed=7100)
    run_both(orc, 4, 8, 16, [3000, 1, 2900], 3000, seed=7200)


def test_no_alloc_decode_rejects_oversized_shapes():
    cfg = lib_cfg(4, 8, 16)
    B, N = 256, 1 << 20  # far more scratch than the fixed array holds
    assert msa.workspace_size(cfg, B, 1, N, msa.WS_DECODE) > msa.decode_no_alloc_max_scratch()
    lib = msa.load()
    import ctypes
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: rejected before any launch
    st = lib.msa_decode_no_alloc(ctypes.byref(cfg._c()), B, N, fake, fake, fake, fake, fake,
                                 fake, fake, None, fake, None, None)
    assert st == 3  # MSA_ERR_WORKSPACE
    assert b"scratch" in lib.msa_last_error()
