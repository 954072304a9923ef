"""GPU parity of msa_cache_append (through the C ABI) against the oracle's
cache_append, bit for bit, and a decode step whose new token was appended by
the library against the oracle on the complete cache."""
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


def host_bits(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().contiguous()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.view(torch.uint8).numpy()


def caches(B, G, Nmax, seed, fp8):
    k = ms.fill_normal_bf16(np.empty((B, G, Nmax, 128), np.uint16), seed)
    v = ms.fill_normal_bf16(np.empty((B, G, Nmax, 128), np.uint16), seed + 1)
    if fp8:
        ki = ms.fill_int_e4m3(np.empty((B, Nmax, 128), np.uint8), seed + 2, -4, 4)
    else:
        ki = ms.fill_int_bf16(np.empty((B, Nmax, 128), np.uint16), seed + 2, -4, 4)
    return k, v, ki


@pytest.mark.parametrize("B,T,G,Nmax,pos0,fp8", [
    (3, 1, 4, 300, [0, 129, 299], False),          # decode appends, first and last slot
    (2, 5, 3, 257, [250, -3], True),               # rows past the end / before 0 skipped
    (4, 37, 1, 1000, [0, 500, 963, 990], False),   # several rows, a ragged last row set
    (1, 300, 2, 640, [128], True),                 # a prefill chunk
    (2, 2, 4, 64, [64, -2], False),                # every row outside the cache
])
def test_cache_append_matches_oracle(B, T, G, Nmax, pos0, fp8):
    k, v, ki = caches(B, G, Nmax, 900 + T, fp8)
    kn = ms.fill_normal_bf16(np.empty((B, T, G, 128), np.uint16), 950)
    vn = ms.fill_normal_bf16(np.empty((B, T, G, 128), np.uint16), 951)
    if fp8:
        kin = ms.fill_int_e4m3(np.empty((B, T, 128), np.uint8), 952, -4, 4)
    else:
        kin = ms.fill_int_bf16(np.empty((B, T, 128), np.uint16), 952, -4, 4)
    pos = np.array(pos0, np.int32)
    want_k, want_v, want_ki = oracle.cache_append(kn, vn, kin, pos, k, v, ki)
    dk, dv, dki = dev_bf16(k), dev_bf16(v), dev_index(ki)
    say("cache_append B=%d T=%d G=%d Nmax=%d pos0=%s fp8=%s" % (B, T, G, Nmax, pos0, fp8))
    msa.cache_append(lib_cfg(G, 2, 16, fp8), dev_bf16(kn), dev_bf16(vn), dev_index(kin),
                     dev_i32(pos), dk, dv, dki)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dk), want_k)
    assert np.array_equal(host_bits(dv), want_v)
    assert np.array_equal(host_bits(dki), want_ki)


@pytest.mark.parametrize("fp8", [False, True])
def test_append_then_decode_equals_decode_on_full_cache(orc, fp8):
    """Decode of a token whose K, V and index key the library appended equals
    the oracle's decode on the cache that held the token from the start."""
    B, G, R, K, Nmax = 3, 4, 8, 16, 4500
    lens = np.array([4500, 2049, 130], np.int32)
    k, v, ki = caches(B, G, Nmax, 960, fp8)
    q = ms.fill_normal_bf16(np.empty((B, 1, G * R, 128), np.uint16), 965)
    if fp8:
        qi = ms.fill_int_e4m3(np.empty((B, 1, G, 128), np.uint8), 966, -4, 4)
    else:
        qi = ms.fill_int_bf16(np.empty((B, 1, G, 128), np.uint16), 966, -4, 4)
    # The new token of sequence b is at position lens[b] - 1: lift it out in
    # the append layout and overwrite it in the device caches with +inf bits.
    pos = lens - 1
    kn = np.stack([k[b, :, pos[b]] for b in range(B)])[:, None]
    vn = np.stack([v[b, :, pos[b]] for b in range(B)])[:, None]
    kin = np.stack([ki[b, pos[b]] for b in range(B)])[:, None]
    k_old, v_old, ki_old = k.copy(), v.copy(), ki.copy()
    for b in range(B):
        k_old[b, :, pos[b]] = 0x7F80
        v_old[b, :, pos[b]] = 0x7F80
        ki_old[b, pos[b]] = 0x7F if fp8 else 0x7F80
    dk, dv, dki = dev_bf16(k_old), dev_bf16(v_old), dev_index(ki_old)
    cfg = lib_cfg(G, R, K, fp8)
    say("append + decode fp8=%s" % fp8)
    msa.cache_append(cfg, dev_bf16(np.ascontiguousarray(kn)), dev_bf16(np.ascontiguousarray(vn)),
                     dev_index(np.ascontiguousarray(kin)), dev_i32(pos), dk, dv, dki)
    sel, out = msa.decode(cfg, dev_bf16(q), dev_index(qi), dki, dk, dv, dev_i32(lens))
    torch.cuda.synchronize()
    ocfg = oracle_cfg(G, R, K, fp8)
    osel, _ = orc.index_topk(ocfg, qi, ki, lens, pos)
    assert np.array_equal(sel.cpu().numpy().reshape(osel.shape), osel)
    oout, olse = orc.sparse_attn(ocfg, q, k, v, lens, pos, osel)
    compare_out(bf16_out_to_f64(out).reshape(oout.shape), oout, "append+decode fp8=%s" % fp8)
