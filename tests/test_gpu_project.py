"""GPU parity of msa_index_project (through the C ABI) against the oracle's
exact float64 sums of the same bf16 inputs. The kernel sums in fp32 (MFMA
order) and rounds once to bf16, so an output may differ from the exact sum by
half a bf16 ulp (2^-8 relative) plus the fp32 summation error, bounded by
h * 2^-24 * sum_k |hidden_k * w_k| (generous); outputs away from a bf16
rounding boundary equal the oracle's rounded value, which the test also
requires of almost all of them (>= 99%)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_30_amd as msa
import msa_synth as ms
import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def inputs(M, h, G, seed, w_scale=None):
    hid = ms.fill_normal_bf16(np.empty((M, h), np.uint16), seed)
    w = np.empty(((G + 1) * 128, h), np.uint16)
    ms.fill_normal_bf16(w, seed + 1)
    scale = w_scale if w_scale is not None else 1.0 / np.sqrt(h)
    wf = (w.astype(np.uint32) << 16).view(np.float32) * np.float32(scale)
    w = ms.float_to_bf16_bits(wf)
    return hid, w


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check(got_bits, exact, absbound, what):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - exact)
    bound = 2.0 ** -8 * np.abs(exact) + absbound
    worst = float((err / np.maximum(bound, 1e-300)).max())
    say("%s: max err / bound = %.3f" % (what, worst))
    assert worst <= 1.0, what


def run(M, h, G, seed, rows=None, keys=True):
    hid, w = inputs(M, h, G, seed)
    cfg = msa.Config(num_kv_groups=G, heads_per_group=8, topk=16)
    say("index projection M=%d h=%d G=%d keys=%s" % (M, h, G, keys))
    q, k = msa.index_project(cfg, dev(hid), dev(w), want_keys=keys)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    gq = q.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    oq, ok_, oqb, okb = oracle.index_project(hid[rows], w, G)
    hf = (hid[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    absb = h * 2.0 ** -23 * (np.abs(hf) @ np.abs(wf).T)          # [rows, (G+1)*dI]
    check(gq, oq, absb[:, :G * 128].reshape(oq.shape), "q_idx")
    same = float((gq == oqb).mean())
    if keys:
        gk = k.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
        check(gk, ok_, absb[:, G * 128:], "k_idx")
        same = min(same, float((gk == okb).mean()))
    else:
        assert k is None
    say("bit-equal to the oracle's rounding: %.4f" % same)
    assert same >= 0.99
    return gq


def test_project_ragged_rows():
    run(300, 256, 3, seed=501)


def test_project_several_tiles_ragged_tail_two_k_steps():
    # Nine 512-token tiles and a ragged tenth (the grid rounds tiles up to a
    # multiple of eight), hidden size 64: two K steps, the fewest.
    run(512 * 9 + 77, 64, 5, seed=506)


def test_project_ragged_tail_six_k_steps_eight_groups():
    run(1100, 192, 8, seed=507)


def test_project_one_row_one_group_no_keys():
    run(1, 64, 1, seed=502, keys=False)


def test_project_queries_alone_equal_queries_with_keys():
    hid, w = inputs(200, 128, 2, 503)
    cfg = msa.Config(num_kv_groups=2, heads_per_group=8, topk=16)
    q1, k1 = msa.index_project(cfg, dev(hid), dev(w))
    q2, k2 = msa.index_project(cfg, dev(hid), dev(w), want_keys=False)
    assert k2 is None and torch.equal(q1, q2)


def test_project_prefill_L131072_sampled_rows():
    # 131072 tokens, hidden size 6144 (the pages give none), 4 groups: every
    # row computed on the GPU, 512 seeded rows checked.
    rows = np.sort(np.random.default_rng(504).choice(131072, 512, replace=False))
    run(131072, 6144, 4, seed=505, rows=rows)
