"""C ABI of libmsa on the CPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_30_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msa.library_path()):
        pytest.skip("libmsa.so not built")
    return msa.load()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("msa_index_topk", "msa_index_pool", "msa_sparse_attn_prefill",
              "msa_sparse_attn_decode", "msa_decode", "msa_cache_append",
              "msa_index_topk_qblock", "msa_sparse_attn_prefill_qblock", "msa_qblock_slots",
              "msa_sparse_attn_backward", "msa_index_project", "msa_decode_no_alloc",
              "msa_decode_no_alloc_max_scratch",
              "msa_workspace_size", "msa_status_string", "msa_last_error", "msa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", msa.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)  # resolvable through the dynamic loader too


def test_status_strings_and_version(lib):
    assert lib.msa_status_string(0) == b"MSA_OK"
    assert lib.msa_status_string(3) == b"MSA_ERR_WORKSPACE"
    assert lib.msa_version() >= 100


def cfg(**kw):
    return msa.Config(**kw)._c()


FAKE = ctypes.c_void_p(0x100000)      # aligned, never dereferenced: calls fail before launch
FAKE_MIS = ctypes.c_void_p(0x100002)  # misaligned


def index_call(lib, c, B=2, T=1, N=1024, q_idx=FAKE, k_idx=FAKE, kv=FAKE, qs=None, sel=FAKE,
               ws=FAKE, nws=0):
    return lib.msa_index_topk(ctypes.byref(c), B, T, N, q_idx, k_idx, kv, qs, sel, None, ws,
                              nws, None)


def test_index_validation(lib):
    c = cfg()
    assert index_call(lib, c, B=0) == OK            # empty batch: nothing to do
    assert index_call(lib, c, T=0) == OK
    assert index_call(lib, c, q_idx=None) == INVALID
    assert index_call(lib, c, sel=None) == INVALID
    assert index_call(lib, c, k_idx=FAKE_MIS) == INVALID
    assert index_call(lib, c, B=-1) == INVALID
    assert index_call(lib, c, N=0) == INVALID
    assert index_call(lib, c, B=70000) == UNSUPPORTED
    assert index_call(lib, cfg(head_dim=64)) == UNSUPPORTED
    assert index_call(lib, cfg(index_dim=64)) == UNSUPPORTED
    assert index_call(lib, cfg(block_size=64)) == UNSUPPORTED
    assert index_call(lib, cfg(topk=65)) == UNSUPPORTED
    assert index_call(lib, cfg(topk=0)) == INVALID
    assert index_call(lib, cfg(heads_per_group=17)) == UNSUPPORTED
    assert index_call(lib, cfg(index_dtype=7)) == INVALID
    assert index_call(lib, cfg(softmax_scale=-1.0)) == INVALID
    assert lib.msa_index_topk(None, 1, 1, 128, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 0,
                              None) == INVALID
    # workspace: missing, misaligned, too small
    need = lib.msa_workspace_size(ctypes.byref(c), 2, 1, 1024, 0)
    assert need >= 2 * 4 * 8 * 4
    assert index_call(lib, c, ws=None, nws=need) == WORKSPACE
    assert index_call(lib, c, ws=ctypes.c_void_p(0x100010), nws=need) == WORKSPACE
    assert index_call(lib, c, nws=need - 1) == WORKSPACE
    assert b"workspace" in lib.msa_last_error()


def test_pool_validation(lib):
    c = cfg()

    def call(B=2, T=1, N=1024, qi=FAKE, ki=FAKE, kv=FAKE, pooled=FAKE, c=c):
        return lib.msa_index_pool(ctypes.byref(c), B, T, N, qi, ki, kv, None, pooled, None)

    assert call(B=0) == OK
    assert call(pooled=None) == INVALID
    assert call(pooled=ctypes.c_void_p(0x100002)) == INVALID
    assert call(ki=FAKE_MIS) == INVALID
    assert call(N=0) == INVALID
    assert call(c=cfg(block_size=64)) == UNSUPPORTED


def test_sparse_validation(lib):
    c = cfg()
    args = dict(q=FAKE, k=FAKE, v=FAKE, kv=FAKE, qs=None, sel=FAKE, out=FAKE, lse=None)

    def prefill(**kw):
        a = {**args, **kw}
        return lib.msa_sparse_attn_prefill(ctypes.byref(kw.get("c", c)), 1, 32, 1024, a["q"],
                                           a["k"], a["v"], a["kv"], a["qs"], a["sel"],
                                           a["out"], a["lse"], None, 0, None)

    def decode(**kw):
        a = {**args, **kw}
        return lib.msa_sparse_attn_decode(ctypes.byref(c), 2, 1024, a["q"], a["k"], a["v"],
                                          a["kv"], a["sel"], a["out"], a["lse"], None, 0, None)

    assert prefill(q=None) == INVALID
    assert prefill(out=FAKE_MIS) == INVALID
    assert prefill(lse=ctypes.c_void_p(0x100001)) == INVALID
    assert prefill(c=cfg(heads_per_group=32)) == UNSUPPORTED
    # 64 rows x 4 groups takes the KV-major path, which needs a workspace.
    assert lib.msa_sparse_attn_prefill(ctypes.byref(c), 1, 64, 1024, FAKE, FAKE, FAKE, FAKE,
                                       None, FAKE, FAKE, None, None, 0, None) == WORKSPACE
    assert decode(sel=None) == INVALID
    assert decode(v=FAKE_MIS) == INVALID
    assert decode() == WORKSPACE  # split partials need a workspace
    assert lib.msa_workspace_size(ctypes.byref(c), 2, 1, 1024, 9) == ctypes.c_size_t(-1).value
    assert lib.msa_workspace_size(None, 2, 1, 1024, 0) == ctypes.c_size_t(-1).value


def test_decode_step_validation(lib):
    c = cfg()

    def call(ws=FAKE, nws=0, **kw):
        a = dict(q=FAKE, qi=FAKE, ki=FAKE, k=FAKE, v=FAKE, kv=FAKE, sel=FAKE, out=FAKE)
        a.update(kw)
        return lib.msa_decode(ctypes.byref(c), 2, 1024, a["q"], a["qi"], a["ki"], a["k"], a["v"],
                              a["kv"], a["sel"], None, a["out"], None, ws, nws, None)

    need = lib.msa_workspace_size(ctypes.byref(c), 2, 1, 1024, 3)
    assert need >= 2 * 4 * 8 * 4
    assert call(qi=None, nws=need) == INVALID
    assert call(ki=FAKE_MIS, nws=need) == INVALID
    assert call(nws=need - 1) == WORKSPACE
    assert call(ws=None, nws=need) == WORKSPACE


def test_decode_no_alloc_validation(lib):
    """msa_decode_no_alloc rejects bad arguments and shapes whose scratch
    exceeds its fixed array on the host, before any HIP call."""
    c = cfg()
    cap = lib.msa_decode_no_alloc_max_scratch()
    assert cap == 32 << 20

    def call(B=2, N=1024, **kw):
        a = dict(q=FAKE, qi=FAKE, ki=FAKE, k=FAKE, v=FAKE, kv=FAKE, sel=FAKE, out=FAKE)
        a.update(kw)
        return lib.msa_decode_no_alloc(ctypes.byref(c), B, N, a["q"], a["qi"], a["ki"], a["k"],
                                       a["v"], a["kv"], a["sel"], None, a["out"], None, None)

    assert call(B=0) == OK
    assert call(qi=None) == INVALID
    assert call(k=FAKE_MIS) == INVALID
    big = (256, 1 << 20)
    assert lib.msa_workspace_size(ctypes.byref(c), big[0], 1, big[1], 3) > cap
    assert call(B=big[0], N=big[1]) == WORKSPACE
    assert b"scratch" in lib.msa_last_error()


def test_cache_append_validation(lib):
    c = cfg()

    def call(B=2, T=1, N=1024, **kw):
        a = dict(kn=FAKE, vn=FAKE, kin=FAKE, pos=FAKE, k=FAKE, v=FAKE, ki=FAKE)
        a.update(kw)
        return lib.msa_cache_append(ctypes.byref(c), B, T, N, a["kn"], a["vn"], a["kin"],
                                    a["pos"], a["k"], a["v"], a["ki"], None)

    assert call(B=0) == OK and call(T=0) == OK        # nothing to write
    for name in ("kn", "vn", "kin", "pos", "k", "v", "ki"):
        assert call(**{name: None}) == INVALID, name
    for name in ("kn", "vn", "kin", "k", "v", "ki"):
        assert call(**{name: FAKE_MIS}) == INVALID, name
    assert call(pos=ctypes.c_void_p(0x100002)) == INVALID
    assert call(B=-1) == INVALID and call(N=0) == INVALID
    assert call(B=70000) == UNSUPPORTED
    assert lib.msa_cache_append(ctypes.byref(cfg(head_dim=64)), 1, 1, 128, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert b"NULL" in lib.msa_last_error() or b"aligned" in lib.msa_last_error() or \
        b"head_dim" in lib.msa_last_error()


def test_qblock_slots_and_validation(lib):
    # 128-token query blocks that T consecutive positions can touch.
    for T, want in ((0, 0), (-3, 0), (1, 1), (2, 2), (128, 2), (129, 2), (130, 3), (256, 3),
                    (32768, 257)):
        assert lib.msa_qblock_slots(T) == want, T
    assert msa.qblock_slots(131072) == 1025
    c = cfg()

    def idx(B=2, T=300, N=1024, **kw):
        a = dict(qi=FAKE, ki=FAKE, kv=FAKE, qs=None, sel=FAKE, sc=None)
        a.update(kw)
        return lib.msa_index_topk_qblock(ctypes.byref(c), B, T, N, a["qi"], a["ki"], a["kv"],
                                         a["qs"], a["sel"], a["sc"], None)

    assert idx(B=0) == OK and idx(T=0) == OK
    assert idx(qi=None) == INVALID and idx(sel=None) == INVALID and idx(kv=None) == INVALID
    assert idx(ki=FAKE_MIS) == INVALID and idx(sc=ctypes.c_void_p(0x100002)) == INVALID
    assert idx(B=70000) == UNSUPPORTED
    assert lib.msa_index_topk_qblock(ctypes.byref(cfg(topk=33)), 1, 8, 128, FAKE, FAKE, FAKE,
                                     None, FAKE, None, None) == UNSUPPORTED

    def att(B=2, T=300, N=1024, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kv=FAKE, qs=None, sel=FAKE, out=FAKE, lse=None)
        a.update(kw)
        return lib.msa_sparse_attn_prefill_qblock(ctypes.byref(c), B, T, N, a["q"], a["k"],
                                                  a["v"], a["kv"], a["qs"], a["sel"], a["out"],
                                                  a["lse"], None)

    assert att(B=0) == OK
    for name in ("q", "k", "v", "kv", "sel", "out"):
        assert att(**{name: None}) == INVALID, name
    assert att(v=FAKE_MIS) == INVALID and att(out=FAKE_MIS) == INVALID
    assert lib.msa_sparse_attn_prefill_qblock(ctypes.byref(cfg(heads_per_group=17)), 1, 8, 128,
                                              FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                                              None) == UNSUPPORTED


def test_backward_validation(lib):
    c = cfg()
    need = lib.msa_workspace_size(ctypes.byref(c), 1, 300, 1024, 4)
    assert need >= 300 * 32 * 4 and need % 256 == 0   # at least delta per (row, head)

    def call(B=1, T=300, N=1024, ws=FAKE, nws=None, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kv=FAKE, sel=FAKE, out=FAKE, lse=FAKE, do=FAKE,
                 dq=FAKE, dk=FAKE, dv=FAKE)
        a.update(kw)
        return lib.msa_sparse_attn_backward(ctypes.byref(c), B, T, N, a["q"], a["k"], a["v"],
                                            a["kv"], None, a["sel"], a["out"], a["lse"],
                                            a["do"], a["dq"], a["dk"], a["dv"], ws,
                                            need if nws is None else nws, None)

    assert call(B=0) == OK and call(T=0) == OK
    for name in ("q", "k", "v", "kv", "sel", "out", "lse", "do", "dq", "dk", "dv"):
        assert call(**{name: None}) == INVALID, name
    for name in ("q", "out", "do", "dq", "dk"):
        assert call(**{name: FAKE_MIS}) == INVALID, name
    assert call(lse=ctypes.c_void_p(0x100002)) == INVALID
    assert call(nws=need - 1) == WORKSPACE and call(ws=None) == WORKSPACE
    assert call(B=70000) == UNSUPPORTED


def test_workspace_sizes_follow_shapes(lib):
    c = cfg()
    a = lib.msa_workspace_size(ctypes.byref(c), 16, 1, 131072, 0)
    assert a >= 16 * 4 * 1024 * 4 and a % 256 == 0          # pooled block scores
    assert lib.msa_workspace_size(ctypes.byref(c), 1, 63, 1024, 1) == 0   # query-major: none
    pf = lib.msa_workspace_size(ctypes.byref(c), 1, 64, 1024, 1)           # KV-major lists
    assert pf >= 64 * 4 * 16 * 8 * 128 * 2 and pf % 256 == 0
    d = lib.msa_workspace_size(ctypes.byref(c), 16, 1, 131072, 2)  # split partials
    assert d >= 16 * 4 * 2 * 8 * 130 * 4 and d % 256 == 0
    # msa_decode: pooled scores, split partials, one arrival counter per
    # (sequence, group)
    dd = lib.msa_workspace_size(ctypes.byref(c), 16, 1, 131072, 3)
    assert a + d <= dd <= a + d + 16 * 4 * 4 + 256 and dd % 256 == 0


def test_topk_limits_and_prefill_workspace_above_32(lib):
    """K up to 64; the prefill index path keeps its top-K in registers up to
    K = 32 (no workspace) and above that ranks pooled scores from the
    workspace; the query-block variant keeps K <= 32."""
    B, T, N = 1, 4096, 8192
    assert lib.msa_workspace_size(ctypes.byref(cfg(topk=32)), B, T, N, 0) == 0
    w64 = lib.msa_workspace_size(ctypes.byref(cfg(topk=64)), B, T, N, 0)
    assert w64 >= B * T * 4 * (N // 128) * 4 and w64 % 256 == 0
    assert lib.msa_workspace_size(ctypes.byref(cfg(topk=65)), B, T, N, 0) == ctypes.c_size_t(-1).value
    c = cfg(topk=64)
    need = lib.msa_workspace_size(ctypes.byref(c), 2, 64, 1024, 0)
    assert need >= 2 * 64 * 4 * 8 * 4
    assert index_call(lib, c, T=64, nws=need - 1) == WORKSPACE  # rejected before any launch
    assert index_call(lib, c, T=64, ws=None, nws=need) == WORKSPACE
    c33 = cfg(topk=33)
    st = lib.msa_index_topk_qblock(ctypes.byref(c33), 1, 256, 1024, FAKE, FAKE, FAKE, None, FAKE,
                                   None, None)
    assert st == UNSUPPORTED
    assert b"topk" in lib.msa_last_error()


def test_decode_workspace_holds_pooled_scores_above_16_groups(lib):
    """msa_decode with more than 16 groups takes the MFMA index kernel, which
    writes the pooled scores of all B*G rows into the same workspace: the size
    must hold them (plus the split partials and counters) for every G."""
    for G in (16, 17, 64):
        c = cfg(num_kv_groups=G, heads_per_group=1)
        B, N = 1, 1 << 20
        nb = N // 128
        pooled = B * G * nb * 4
        parts = lib.msa_workspace_size(ctypes.byref(c), B, 1, N, 2)
        dd = lib.msa_workspace_size(ctypes.byref(c), B, 1, N, 3)
        assert dd >= pooled + parts + B * G * 4, (G, dd)
        assert dd % 256 == 0


def test_index_project_validation(lib):
    c = cfg()

    def call(M=300, h=256, **kw):
        a = dict(hid=FAKE, w=FAKE, q=FAKE, k=FAKE)
        a.update(kw)
        return lib.msa_index_project(ctypes.byref(c), M, h, a["hid"], a["w"], a["q"], a["k"],
                                     None)

    assert call(M=0) == OK                                # nothing to compute
    for name in ("hid", "w", "q"):
        assert call(**{name: None}) == INVALID, name
    for name in ("hid", "w", "q", "k"):
        assert call(**{name: FAKE_MIS}) == INVALID, name
    assert call(M=-1) == INVALID
    assert call(h=0) == UNSUPPORTED and call(h=100) == UNSUPPORTED
    assert lib.msa_index_project(ctypes.byref(cfg(index_dtype=msa.FP8_E4M3)), 8, 64, FAKE, FAKE, FAKE,
                                 FAKE, None) == UNSUPPORTED
    assert b"bf16" in lib.msa_last_error()
    assert lib.msa_index_project(ctypes.byref(cfg(index_dim=64)), 8, 64, FAKE, FAKE, FAKE,
                                 FAKE, None) == UNSUPPORTED


def test_python_binding_rejects_cpu_tensors():
    import torch
    c = msa.Config()
    q = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        msa.index_topk(c, q, torch.zeros(1, 128, 128, dtype=torch.bfloat16),
                       torch.ones(1, dtype=torch.int32))


def test_read_probe_loads_and_rejects_bad_arguments():
    """The benchmark's streaming-read probe (a separate object) loads, and its
    argument checks run before any launch."""
    path = os.path.join(os.path.dirname(msa.__file__), "libmsa_probe.so")
    probe = ctypes.CDLL(path)
    fn = probe.msa_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    dummy = ctypes.c_void_p(0x1000)
    for nt in (0, 1):
        assert fn(None, 1 << 20, 64, nt, dummy, None) == -1
        assert fn(dummy, 1 << 20, 64, nt, None, None) == -1
        assert fn(dummy, 1 << 20, 0, nt, dummy, None) == -1
        assert fn(dummy, (1 << 20) + 16, 64, nt, dummy, None) == -1   # not a multiple of 16 * wgs
