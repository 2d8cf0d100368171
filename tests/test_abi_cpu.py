"""C-ABI checks that need no GPU: the library loads, exports every function
include/dustin.h declares, and rejects bad arguments on the host before any
HIP call."""
import ctypes
import os
import re

import pytest
import torch

import sparse_kv_verification_amd as dk
from sparse_kv_verification_amd._lib import DustinKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, HIPERR = 1, 2, 3
FAKE = 0x1000   # never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "dustin.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dustin_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return dk.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(dk.EXPORTS)


def test_version_and_strings(L):
    assert L.dustin_abi_version() == 7
    assert L.dustin_status_string(0) == b"DUSTIN_OK"
    assert L.dustin_status_string(2) == b"DUSTIN_ERR_UNSUPPORTED"


def kv(**kw):
    d = dict(k=FAKE, v=FAKE, dtype=1, B=2, H_kv=8, head_dim=128, N_max=4096, seq_lens=FAKE,
             page_size=0, page_table=None, max_pages=0, num_pages=0)
    d.update(kw)
    return DustinKV(**d)


def attn(L, desc, q=FAKE, w=4, Hq=64, idx=FAKE, count=FAKE, k=2048, ws=FAKE, ws_bytes=1 << 40, scale=0.0, out=FAKE):
    return L.dustin_sparse_verify_attn(q, w, Hq, ctypes.byref(desc), idx, count, k, scale, out, None, ws, ws_bytes, None)


def test_attention_argument_errors(L):
    assert attn(L, kv(k=None)) == INVALID
    assert attn(L, kv(v=None)) == INVALID
    assert attn(L, kv(), q=None) == INVALID
    assert attn(L, kv(), out=None) == INVALID
    assert attn(L, kv(dtype=7)) == UNSUPPORTED
    assert attn(L, kv(head_dim=96)) == UNSUPPORTED
    assert attn(L, kv(), Hq=60) == INVALID                            # not a multiple of H_kv
    assert attn(L, kv(), w=9) == UNSUPPORTED                          # w * G = 72 > 64
    assert attn(L, kv(), k=0) == INVALID
    assert attn(L, kv(), count=None) == INVALID
    assert attn(L, kv(), idx=None, k=5) == INVALID                    # dense form takes k = 0
    assert attn(L, kv(seq_lens=None)) == INVALID
    assert attn(L, kv(page_size=8)) == UNSUPPORTED
    assert attn(L, kv(page_size=16, page_table=None, max_pages=256, num_pages=10)) == INVALID
    assert attn(L, kv(page_size=16, page_table=FAKE, max_pages=10, num_pages=10)) == INVALID
    assert attn(L, kv(), scale=float("nan")) == INVALID
    assert attn(L, kv(B=4096, H_kv=8)) == UNSUPPORTED                 # more groups than counter slots
    need = L.dustin_attn_workspace_bytes(2, 4, 64, 8, 128, 2048)
    assert need > 0
    assert attn(L, kv(), ws_bytes=need - 1) == INVALID
    assert attn(L, kv(), ws=None) == INVALID
    assert b"workspace" in L.dustin_last_error()


def test_topk_argument_errors(L):
    f = lambda **kw: L.dustin_topk(kw.get("sd", FAKE), kw.get("st", FAKE), kw.get("lens", FAKE), kw.get("B", 2),
                                   kw.get("N", 1000), kw.get("k", 64), kw.get("m", 10), kw.get("ns", 4),
                                   kw.get("nw", 8), kw.get("idx", FAKE), kw.get("cnt", FAKE), None, FAKE,
                                   kw.get("ws", 1 << 30), None)
    assert f(sd=None, st=None) == INVALID
    assert f(k=0) == INVALID
    assert f(m=-1) == INVALID
    assert f(ns=40, nw=40) == INVALID           # protected tokens exceed k
    assert f(idx=None) == INVALID
    assert f(lens=None) == INVALID
    assert f(ws=L.dustin_topk_workspace_bytes(2, 1000, 64) - 1) == INVALID


def test_score_argument_errors(L):
    d = (DustinKV * 2)(kv(H_kv=2, head_dim=64), kv(H_kv=2, head_dim=64))
    t = (DustinKV * 1)(kv())
    heads = (ctypes.c_int32 * 4)(0, 0, 0, 8)
    def f(**kw):
        return L.dustin_score(kw.get("d", d), kw.get("L_d", 2), kw.get("qd", FAKE), kw.get("H_d", 14),
                              kw.get("gamma", 4), kw.get("t", t), kw.get("L_t", 1), kw.get("qh", FAKE),
                              kw.get("heads", heads), kw.get("S", 2), kw.get("H_t", 64), 0.0, 0.0,
                              kw.get("lse", None), kw.get("sd", FAKE), kw.get("st", FAKE), FAKE,
                              kw.get("ws", 1 << 40), None)
    assert f(qd=None) == INVALID
    assert f(H_d=13) == INVALID                                   # not a multiple of draft H_kv
    assert f(gamma=20) == UNSUPPORTED                             # gamma * G_d = 140 > 64
    bad = (DustinKV * 2)(kv(H_kv=2, head_dim=64), kv(H_kv=2, head_dim=128))
    assert f(d=bad) == INVALID                                    # layers differ in geometry
    assert f(heads=(ctypes.c_int32 * 4)(0, 0, 1, 8)) == INVALID   # layer out of range
    assert f(heads=(ctypes.c_int32 * 4)(0, 0, 0, 64)) == INVALID  # head out of range
    assert f(H_t=60) == INVALID                                   # H_t not a multiple of H_kv
    assert f(qh=None) == INVALID
    assert f(S=65, heads=(ctypes.c_int32 * 130)()) == UNSUPPORTED
    assert f(ws=10) == INVALID
    # nothing requested: a no-op that succeeds without touching the GPU
    assert f(sd=None, st=None) == 0
    # the row-normaliser query checks the draft side the same way
    def g(**kw):
        return L.dustin_draft_row_lse(kw.get("d", d), kw.get("L_d", 2), kw.get("qd", FAKE), kw.get("H_d", 14),
                                      kw.get("gamma", 4), 0.0, kw.get("out", FAKE), FAKE, kw.get("ws", 1 << 40), None)
    assert g(out=None) == INVALID
    assert g(L_d=0) == INVALID
    assert g(qd=None) == INVALID
    assert g(H_d=13) == INVALID
    assert g(gamma=20) == UNSUPPORTED
    assert g(d=bad) == INVALID
    assert g(ws=10) == INVALID


def test_arr_and_window_argument_errors(L):
    assert L.dustin_arr(None, FAKE, 2, 4, 100, FAKE, FAKE, 8, FAKE, FAKE, None) == INVALID
    assert L.dustin_arr(FAKE, FAKE, 2, 65, 100, FAKE, FAKE, 8, FAKE, FAKE, None) == UNSUPPORTED
    assert L.dustin_arr(FAKE, FAKE, 2, 4, 100, FAKE, FAKE, 0, FAKE, FAKE, None) == INVALID
    desc = kv()
    assert L.dustin_window_attn(FAKE, 17, 8, ctypes.byref(desc), 0.0, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED
    assert L.dustin_window_attn(FAKE, 4, 64, ctypes.byref(desc), 0.0, None, FAKE, 1 << 40, None) == INVALID
    assert L.dustin_window_attn(FAKE, 4, 64, ctypes.byref(desc), 0.0, FAKE, FAKE, 16, None) == INVALID
    # bfloat16 takes long windows in slices (at most 64 rows per KV head per slice), float32 does not
    assert L.dustin_window_attn(FAKE, 4, 60, ctypes.byref(desc), 0.0, FAKE, FAKE, 1 << 40, None) == INVALID
    h2 = kv(H_kv=1)
    assert L.dustin_window_attn(FAKE, 2, 65, ctypes.byref(h2), 0.0, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED
    f32 = kv(dtype=0)
    assert L.dustin_window_attn(FAKE, 16, 64, ctypes.byref(f32), 0.0, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED
    assert L.dustin_window_attn(FAKE, 9, 64, ctypes.byref(f32), 0.0, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED


def test_verify_window_argument_errors(L):
    def va(desc, **kw):
        return L.dustin_verify_attn(kw.get("q", FAKE), kw.get("w", 4), kw.get("Hq", 64), ctypes.byref(desc),
                                    kw.get("idx", FAKE), kw.get("count", FAKE), kw.get("k", 2048), 0.0,
                                    kw.get("out", FAKE), None, FAKE, kw.get("ws_bytes", 1 << 40), None)
    assert va(kv(v=None)) == INVALID
    assert va(kv(), out=None) == INVALID
    assert va(kv(), w=9) == UNSUPPORTED
    assert va(kv(), idx=None, k=5) == INVALID
    assert va(kv(), count=None) == INVALID
    need = L.dustin_verify_attn_workspace_bytes(2, 4, 64, 8, 128, 2048)
    assert need > 0
    assert va(kv(), ws_bytes=need - 1) == INVALID
    assert b"verify_attn" in L.dustin_last_error()
    assert L.dustin_verify_attn_workspace_bytes(2, 0, 64, 8, 128, 2048) == 0

    def vaa(desc, **kw):
        return L.dustin_verify_attn_append(kw.get("q", FAKE), kw.get("w", 4), kw.get("Hq", 64), ctypes.byref(desc),
                                           kw.get("kw", FAKE), kw.get("vw", FAKE), kw.get("idx", FAKE),
                                           kw.get("count", FAKE), kw.get("k", 2048), 0.0, kw.get("out", FAKE), None,
                                           FAKE, kw.get("ws_bytes", 1 << 40), None)
    assert vaa(kv(), kw=None) == INVALID and vaa(kv(), vw=None) == INVALID
    assert vaa(kv(), kw=FAKE + 8) == INVALID                      # not 16-byte aligned
    assert b"aligned" in L.dustin_last_error()
    assert vaa(kv(v=None)) == INVALID
    assert vaa(kv(), w=9) == UNSUPPORTED
    assert vaa(kv(), count=None) == INVALID
    assert vaa(kv(), ws_bytes=need - 1) == INVALID
    assert vaa(kv(dtype=0), out=None) == INVALID                 # float32: every check before the append
    assert b"verify_attn_append" in L.dustin_last_error()

    def ap(desc, kw_=FAKE, vw=FAKE, w=4):
        return L.dustin_append_window_kv(ctypes.byref(desc), kw_, vw, w, None)
    assert ap(kv(), kw_=None) == INVALID
    assert ap(kv(), vw=None) == INVALID
    assert ap(kv(v=None)) == INVALID
    assert ap(kv(), w=0) == INVALID
    assert ap(kv(), kw_=FAKE + 8) == INVALID                       # not 16-byte aligned
    assert b"aligned" in L.dustin_last_error()
    assert ap(kv(dtype=7)) == UNSUPPORTED
    assert L.dustin_commit_window(None, FAKE, 2, 4, None) == INVALID
    assert L.dustin_commit_window(FAKE, None, 2, 4, None) == INVALID
    assert L.dustin_commit_window(FAKE, FAKE, 0, 4, None) == INVALID
    assert L.dustin_commit_window(FAKE, FAKE, 2, 0, None) == INVALID


def test_sweep_argument_errors(L):
    desc = kv()
    ks = (ctypes.c_int32 * 3)(128, 512, 2048)
    ms = (ctypes.c_int32 * 3)(46, 238, 1006)
    def f(**kw):
        return L.dustin_policy_sweep(kw.get("qw", FAKE), kw.get("w", 4), kw.get("qp", FAKE), kw.get("P", 4),
                                     kw.get("Hq", 64), ctypes.byref(kw.get("desc", desc)), kw.get("sd", FAKE),
                                     kw.get("st", FAKE), kw.get("ks", ks), kw.get("ms", ms), kw.get("nk", 3),
                                     kw.get("ns", 4), kw.get("nw", 32), 0.0, kw.get("arr", FAKE), FAKE,
                                     kw.get("ws", 1 << 40), None)
    assert f(qw=None) == INVALID
    assert f(qp=None) == INVALID                          # n_past > 0 needs q_past
    assert f(sd=None) == INVALID and f(st=None) == INVALID and f(arr=None) == INVALID
    assert f(ks=None) == INVALID and f(nk=0) == INVALID
    assert f(w=17) == UNSUPPORTED
    assert f(P=65) == UNSUPPORTED
    assert f(ks=(ctypes.c_int32 * 3)(16, 512, 2048)) == INVALID              # k < n_sink + n_window
    assert f(ms=(ctypes.c_int32 * 3)(200, 238, 1006)) == INVALID             # m_hybrid > k
    need = L.dustin_policy_sweep_workspace_bytes(2, 4, 4, 64, 8, 128, 4096, 2048)
    assert need > L.dustin_window_attn_workspace_bytes(2, 4, 64, 8, 128, 4096)
    assert f(ws=need - 1) == INVALID
    assert b"workspace" in L.dustin_last_error()
    assert L.dustin_window_mean(None, 2, 4, 10, FAKE, None) == INVALID
    assert L.dustin_window_mean(FAKE, 2, 0, 10, FAKE, None) == INVALID


def test_page_estimator_argument_errors(L):
    desc = kv()
    assert L.dustin_page_bounds(ctypes.byref(desc), None, FAKE, None) == INVALID
    assert L.dustin_page_bounds(ctypes.byref(desc), FAKE + 4, FAKE, None) == INVALID     # misaligned
    assert L.dustin_page_bounds(ctypes.byref(kv(k=None)), FAKE, FAKE, None) == INVALID
    need = L.dustin_page_scores_workspace_bytes(2, 8, 128)
    assert need == 2 * 2 * 8 * 128 * 4
    f = lambda **k: L.dustin_page_scores(k.get("q", FAKE), k.get("w", 4), k.get("Hq", 64), ctypes.byref(desc),
                                         FAKE, FAKE, k.get("scale", 0.0), k.get("out", FAKE), k.get("ws", FAKE),
                                         k.get("ws_bytes", need), None)
    assert f(q=None) == INVALID and f(out=None) == INVALID
    assert f(Hq=60) == INVALID
    assert f(q=FAKE + 2) == INVALID                      # misaligned
    assert f(ws=None) == INVALID and f(ws_bytes=need - 1) == INVALID
    assert L.dustin_page_scores(FAKE, 4, 512, ctypes.byref(kv(H_kv=64)), FAKE, FAKE, 0.0, FAKE, FAKE, 1 << 30,
                                None) == UNSUPPORTED     # H_kv * head_dim beyond 4096
    assert f(scale=float("inf")) == INVALID


def test_search_argument_errors(L):
    I32 = ctypes.c_int32
    ids_bad = (I32 * 2)(0, 5)
    cand = lambda **k: L.dustin_candidate_arr(k.get("sd"), k.get("du"), k.get("st", FAKE), k.get("tu"), k.get("U", 4),
                                              k.get("ids"), k.get("C", 2), k.get("mc"), FAKE, 2, 1024, k.get("abar", FAKE),
                                              k.get("k", 64), 0, k.get("ns", 4), 32, FAKE, None, FAKE, 1 << 40, None)
    assert cand(st=None) == INVALID                          # no score side at all
    assert cand(du=FAKE, tu=FAKE) == INVALID                 # units on both sides
    assert cand(abar=None) == INVALID
    assert cand(k=0) == INVALID and cand(ns=64) == INVALID   # protected tokens exceed k
    assert cand(tu=FAKE, ids=ids_bad, U=4) == INVALID        # unit id out of range
    assert cand(tu=FAKE, U=1, C=2) == INVALID                # C > U without ids
    assert cand(mc=(I32 * 2)(0, -1)) == INVALID              # negative per-candidate m
    assert L.dustin_candidate_arr(None, None, FAKE, None, 0, None, 1, None, FAKE, 2, 1024, FAKE, 64, 0, 4, 32, FAKE,
                                  None, FAKE, 0, None) == INVALID   # workspace too small
    ch, cu, n = (I32 * 4)(), (ctypes.c_float * 4)(), I32(0)
    g = lambda **k: L.dustin_greedy_select(k.get("units", FAKE), 4, None, 4, k.get("side", 0), k.get("fixed"), FAKE, 2,
                                           1024, FAKE, 64, 10, 4, 32, 2, ch, cu, ctypes.byref(n), k.get("out", FAKE),
                                           FAKE, 1 << 40, None)
    assert g(side=2) == INVALID and g(units=None) == INVALID and g(out=None) == INVALID
    assert g(side=1) == INVALID                              # the draft side needs the fixed S_Target
    assert g(side=0, fixed=FAKE) == INVALID                  # the target side takes none
    assert L.dustin_greedy_select_workspace_bytes(4, 2, 1024, 64) >= L.dustin_candidate_arr_workspace_bytes(4, 2, 1024, 64, 1)
    heads = (I32 * 2)(0, 3)
    assert L.dustin_head_scores(ctypes.byref(kv()), 1, FAKE, heads, 1, 64, 0.0, None, FAKE, 1 << 40, None) == INVALID
    assert L.dustin_head_scores(ctypes.byref(kv()), 1, FAKE, heads, 0, 64, 0.0, FAKE, FAKE, 1 << 40, None) == INVALID
    bad = (I32 * 2)(0, 64)
    assert L.dustin_head_scores(ctypes.byref(kv()), 1, FAKE, bad, 1, 64, 0.0, FAKE, FAKE, 1 << 40, None) == INVALID


def test_workspace_sizes_are_shape_only(L):
    # c4 shapes: the attention plan merges partials from several splits
    a = L.dustin_attn_workspace_bytes(16, 4, 64, 8, 128, 2048)
    b = L.dustin_attn_workspace_bytes(16, 4, 64, 8, 128, 32768)
    assert 0 < a < b
    assert L.dustin_attn_workspace_bytes(0, 4, 64, 8, 128, 2048) == 0
    assert L.dustin_score_workspace_bytes(16, 32768, 24, 14, 4, 8) > 16 * 8 * 32768 * 4
    # rows up to 32768 positions: register-resident select, no workspace beyond the minimum;
    # 32769 .. 262144: per-chunk histograms (4096-position chunks, 2048 bins of 4 bytes);
    # longer: one tier byte per position
    assert L.dustin_topk_workspace_bytes(16, 32768, 2048) == 256
    assert L.dustin_topk_workspace_bytes(8, 131072, 4096) >= 8 * 32 * 2048 * 4
    assert L.dustin_topk_workspace_bytes(2, 300000, 4096) >= 2 * 300000


def test_attention_head_dims(L):
    """Every attention entry point serves head_dim 32, 64 and 128 in bfloat16
    and float32 (validation passes, then a device is needed); other head dims
    are refused on the host with DUSTIN_ERR_UNSUPPORTED."""
    if not torch.cuda.is_available():
        for d in (32, 64, 128):
            for dt in (0, 1):
                assert attn(L, kv(head_dim=d, dtype=dt)) == HIPERR, (d, dt)
        d32 = kv(head_dim=32, dtype=1)
        assert L.dustin_verify_attn(FAKE, 4, 64, ctypes.byref(d32), FAKE, FAKE, 2048, 0.0, FAKE, None, FAKE,
                                    1 << 40, None) == HIPERR
        assert L.dustin_sparse_verify_attn_noalloc(FAKE, 4, 64, ctypes.byref(d32), FAKE, FAKE, 2048, 0.0, FAKE,
                                                   None, None) == HIPERR
    assert attn(L, kv(head_dim=48, dtype=1)) == UNSUPPORTED
    assert b"head_dim" in L.dustin_last_error()


def test_probe_argument_errors(L):
    """The measurement kernels check their arguments on the host."""
    assert L.dustin_probe_stream_read(None, 4096, 1, FAKE, None) == INVALID
    assert L.dustin_probe_stream_read(FAKE, 4096, 1, None, None) == INVALID
    assert L.dustin_probe_stream_read(FAKE, 4100, 1, FAKE, None) == INVALID
    assert L.dustin_probe_stream_read(FAKE, 0, 1, FAKE, None) == INVALID
    g = L.dustin_probe_gather_rows
    assert g(FAKE, None, 256, 100, FAKE, 10, 96, None) == INVALID          # row size
    assert g(FAKE, None, 128, 100, FAKE, 10, 256, None) == INVALID         # stride below the row
    assert g(FAKE, None, 264, 100, FAKE, 10, 256, None) == INVALID         # stride not a multiple of 16
    assert g(FAKE, None, 256, 100, FAKE, 0, 256, None) == INVALID          # no rows
    assert g(FAKE, None, 256, 100, FAKE, 256 * 4096 + 1, 256, None) == INVALID
    assert g(FAKE, None, 256, 0, FAKE, 10, 256, None) == INVALID
    assert g(None, None, 256, 100, FAKE, 10, 256, None) == INVALID


def test_noalloc_attention_limits(L):
    """The allocation-free attention checks its arguments like the workspace
    form and refuses, on the host, a shape whose split state exceeds its
    static scratch (the dense form over 131072 positions at B = 64)."""
    def call(desc, **kw):
        a = dict(q=FAKE, w=4, Hq=64, idx=FAKE, count=FAKE, k=2048, out=FAKE)
        a.update(kw)
        return L.dustin_sparse_verify_attn_noalloc(a["q"], a["w"], a["Hq"], ctypes.byref(desc), a["idx"],
                                                   a["count"], a["k"], 0.0, a["out"], None, None)
    assert call(kv(k=None)) == INVALID
    assert call(kv(), out=None) == INVALID
    assert call(kv(), Hq=60) == INVALID
    big = kv(B=64, N_max=131072)
    assert L.dustin_attn_workspace_bytes(64, 4, 64, 8, 128, 131072) > (32 << 20)
    assert call(big, idx=None, count=None, k=0) == UNSUPPORTED
    assert b"scratch" in L.dustin_last_error()
    assert L.dustin_attn_workspace_bytes(16, 4, 64, 8, 128, 2048) <= (32 << 20)   # the headline shape fits


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_valid_call_without_device_reports_hip_error(L):
    # Validation passes; the first HIP call then fails because there is no device.
    desc = kv()
    st = attn(L, desc)
    assert st == HIPERR
    assert L.dustin_last_error() != b""
    st = L.dustin_sparse_verify_attn_noalloc(FAKE, 4, 64, ctypes.byref(desc), FAKE, FAKE, 2048, 0.0, FAKE, None,
                                             None)
    assert st == HIPERR


def test_binding_refuses_host_tensors():
    """A host (CPU) tensor handed to a kernel would be dereferenced as a
    device address; the binding refuses it before any call."""
    import torch
    import sparse_kv_verification_amd as dk
    lens = torch.full((2,), 8, dtype=torch.int32)
    with pytest.raises(TypeError):
        dk.KV(torch.zeros((2, 8, 1, 32), dtype=torch.bfloat16), None, lens)
    with pytest.raises(TypeError):
        dk.dustin_window_mean(torch.zeros((2, 3, 8)))


def test_missing_library_fails_loudly():
    """No fallback: with the library absent, every entry point raises
    instead of computing anything elsewhere (run in a fresh interpreter so
    the already-loaded library of this process is not involved)."""
    import subprocess
    import sys
    code = (
        "import torch, sparse_kv_verification_amd._lib as L\n"
        "L.LIB_PATH = '/nonexistent/libdustin.so'\n"
        "L._lib = None\n"
        "try:\n"
        "    L.dustin_topk(torch.zeros(1, 8), torch.zeros(1, 8), torch.full((1,), 8, dtype=torch.int32), 4, 1, 0, 0)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', 'is missing' in str(e))\n"
        "else:\n"
        "    print('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert "raised: True" in r.stdout, r.stdout + r.stderr
