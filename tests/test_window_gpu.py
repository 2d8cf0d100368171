"""GPU parity of the verification-window calls (blog, Fig. 5, Stage 2): the
window's keys/values are appended to the cache, the window queries attend the
selected history rows plus the window causally, and the accepted tokens are
committed.  Each is compared with the oracle on the same seeded inputs.

Tolerances as for the history-only attention: output max-abs 2e-2 (bf16) /
1e-4 (float32), lse abs 2e-3 / 1e-5; cache rows and lengths bit-exact.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import f64, make_idx, oracle_kv, say, valid_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(name, over, room=True):
    """Seeded inputs with every history shortened so the window fits behind
    it, plus the window's keys and values [B][w][H_kv][d].  The window keys
    lean towards the window queries so the causal block carries real weight."""
    over = dict(over)
    base = over.pop("base", "c4")
    sh = synth.preset(base).replace(**over)
    x = synth.make(sh, device=DEV)
    lens = x.seq_lens.cpu().numpy().astype(np.int64)
    if room:
        lens = np.maximum(lens - sh.w - (np.arange(sh.B) * 13) % 50, 0)
        x.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    g = torch.Generator(device=DEV)
    g.manual_seed(zlib.crc32(name.encode()))
    store = x.K.dtype
    shp = (sh.B, sh.w, sh.Hkv, sh.d)
    lead = x.q[:, :, ::sh.G, :].float()                     # first query head of each KV group
    k_win = (torch.randn(shp, generator=g, device=DEV) + 0.5 * lead).to(store).contiguous()
    v_win = torch.randn(shp, generator=g, device=DEV).to(store).contiguous()
    return sh, x, k_win, v_win


def _phys_rows(x, b, positions):
    """Storage row (in the flattened [rows][H_kv][d] view) of logical positions."""
    pos = np.asarray(positions, dtype=np.int64)
    if x.page_table is None:
        return b * x.K.shape[1] + pos
    ps = x.shape.page_size
    pages = x.page_table[b].cpu().numpy().astype(np.int64)
    return pages[pos // ps] * ps + pos % ps


def _check_append(x, k_before, v_before, k_win, v_win):
    """Rows n_b .. n_b + w - 1 now hold the window; nothing else changed."""
    sh = x.shape
    lens = x.seq_lens.cpu().numpy()
    flat = lambda t: t.reshape(-1, sh.Hkv, sh.d)
    changed = np.zeros(flat(x.K).shape[0], dtype=bool)
    for b in range(sh.B):
        n = int(lens[b])
        rows = _phys_rows(x, b, np.arange(n, n + sh.w))
        changed[rows] = True
        for name, cache, win in (("K", x.K, k_win), ("V", x.V, v_win)):
            got = flat(cache)[torch.from_numpy(rows).to(DEV)]
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               win[b].view(torch.int16) if win.dtype == torch.bfloat16 else win[b]), \
                f"{name} rows of b={b} differ from the window"
        # the oracle's append on the logical view agrees with the cache
        K0 = f64(flat(k_before)[torch.from_numpy(_phys_rows(x, b, np.arange(n + sh.w))).to(DEV)])
        V0 = f64(flat(v_before)[torch.from_numpy(_phys_rows(x, b, np.arange(n + sh.w))).to(DEV)])
        K1, V1 = oracle.append_window_kv(K0, V0, n, f64(k_win[b]), f64(v_win[b]))
        rows_all = torch.from_numpy(_phys_rows(x, b, np.arange(n + sh.w))).to(DEV)
        assert np.array_equal(f64(flat(x.K)[rows_all]), K1) and np.array_equal(f64(flat(x.V)[rows_all]), V1)
    # bit patterns: unused slots of a paged pool hold NaN
    keep = torch.from_numpy(~changed).to(DEV)
    assert _equal(flat(x.K)[keep], flat(k_before)[keep]), "rows outside the window changed"
    assert _equal(flat(x.V)[keep], flat(v_before)[keep]), "rows outside the window changed"


def _equal(a, b):
    """Bitwise equality (NaN payloads included)."""
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


CASES = [
    # name, shape overrides, k (None = dense form), idx options
    ("qwen72b-rows32", dict(B=2, n=5000, Hq=64, Hkv=8, k=1000, L_d=1), 1000, dict(frac_invalid=0.05, short=7)),
    ("qwen32b-rows20", dict(B=2, n=3000, Hq=40, Hkv=8, k=300, L_d=1), 300, dict()),
    ("window-own-split", dict(B=2, n=3000, Hq=64, Hkv=8, k=512, L_d=1), 512, dict()),
    ("qwen7b-rows28-tail", dict(B=3, n=2333, Hq=28, Hkv=4, k=517, L_d=1), 517, dict(shuffle=False)),
    ("paged-ragged-rows64", dict(base="c5", B=3, n=4000, n_lo=700, k=700, L_d=1), 700, dict(frac_invalid=0.02)),
    ("d64-rows16", dict(B=2, n=2000, Hq=8, Hkv=2, d=64, k=257, L_d=1), 257, dict()),
    ("d32-rows16", dict(B=2, n=2000, Hq=8, Hkv=2, d=32, k=257, L_d=1), 257, dict()),
    ("d32-dense-rows32", dict(B=2, n=120, Hq=16, Hkv=2, d=32, L_d=1), None, dict()),   # short: the mask matters
    ("w1-rows8", dict(B=2, n=3000, Hq=64, Hkv=8, w=1, k=200, L_d=1), 200, dict()),
    ("dense-qwen72b", dict(B=2, n=4100, Hq=64, Hkv=8, L_d=1), None, dict()),
    ("dense-paged", dict(base="c5", B=2, n=3000, n_lo=900, L_d=1), None, dict()),
    ("tiny-f32", dict(base="c1"), 128, dict()),
    ("tiny-f32-dense", dict(base="c1"), None, dict()),
]


@pytest.mark.parametrize("name,over,k,iopt", CASES, ids=[c[0] for c in CASES])
def test_verify_step_matches_oracle(name, over, k, iopt):
    say("verify step", name)
    sh, x, k_win, v_win = _setup(name, over)
    f32 = sh.dtype == "f32"
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    k_before, v_before = x.K.clone(), x.V.clone()
    dk.dustin_append_window_kv(kv, k_win, v_win)
    torch.cuda.synchronize()
    _check_append(x, k_before, v_before, k_win, v_win)

    if k is None:
        idx = cnt = None
    else:
        idx, cnt = make_idx(x.seq_lens, k, seed=zlib.crc32(name.encode()) % 1000, device=DEV, **iopt)
    lse = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    out = dk.dustin_verify_attn(x.q, kv, idx, cnt, lse=lse)
    out2 = dk.dustin_verify_attn(x.q, kv, idx, cnt)
    torch.cuda.synchronize()
    assert _equal(out, out2), "not deterministic"
    lens = x.seq_lens.cpu().numpy()
    for b in range(sh.B):
        n = int(lens[b])
        I = np.arange(n) if idx is None else valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        K, V = oracle_kv(x, "K", b), oracle_kv(x, "V", b)
        O, L = oracle.verify_attention(f64(x.q[b]), K, V, f64(k_win[b]), f64(v_win[b]), I)
        err = np.abs(f64(out[b]) - O).max()
        lerr = np.abs(f64(lse[b]) - L).max()
        # the causal block matters: attending the whole window differs by far more than the tolerance
        Ofull, _ = oracle.sparse_attention(f64(x.q[b]), np.concatenate([K, f64(k_win[b])]),
                                           np.concatenate([V, f64(v_win[b])]),
                                           np.concatenate([I, n + np.arange(sh.w)]))
        gap = np.abs(Ofull - O).max()
        say(f"  b={b} n={n} |I|={len(I)} max|dO|={err:.2e} max|dlse|={lerr:.2e} (mask effect {gap:.2e})")
        assert err <= (1e-4 if f32 else 2e-2)
        assert lerr <= (1e-5 if f32 else 2e-3)
        if sh.w > 1:
            assert gap > 10 * (1e-4 if f32 else 2e-2)

    # commit: the accepted rows become history
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    accepted = rng.integers(-1, sh.w + 2, sh.B).astype(np.int32)
    dk.dustin_commit_window(x.seq_lens, torch.from_numpy(accepted).to(DEV), sh.w)
    torch.cuda.synchronize()
    got = x.seq_lens.cpu().numpy()
    for b in range(sh.B):
        assert int(got[b]) == oracle.commit_window(int(lens[b]), int(accepted[b]), sh.w)


def test_two_verification_steps():
    """Append, verify, commit, then a second step whose window overwrites the
    rejected rows and whose set includes just-accepted positions."""
    say("two verification steps")
    sh, x, kw1, vw1 = _setup("two-steps", dict(B=3, n=3000, Hq=64, Hkv=8, k=400, L_d=1))
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    n0 = x.seq_lens.cpu().numpy().astype(np.int64)
    Kh = [oracle_kv(x, "K", b) for b in range(sh.B)]
    Vh = [oracle_kv(x, "V", b) for b in range(sh.B)]
    dk.dustin_append_window_kv(kv, kw1, vw1)
    accepted = np.array([0, 2, sh.w], dtype=np.int32)
    dk.dustin_commit_window(x.seq_lens, torch.from_numpy(accepted).to(DEV), sh.w)
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    kw2 = torch.randn(kw1.shape, generator=g, device=DEV).to(kw1.dtype)
    vw2 = torch.randn(vw1.shape, generator=g, device=DEV).to(vw1.dtype)
    q2 = torch.randn(x.q.shape, generator=g, device=DEV).to(x.q.dtype)
    dk.dustin_append_window_kv(kv, kw2, vw2)
    n1 = x.seq_lens.cpu().numpy().astype(np.int64)
    B, k = sh.B, 400
    idx = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        recent = np.arange(n0[b], n1[b])                          # the accepted rows of step 1
        rest = np.random.default_rng(b).choice(int(n0[b]), k - len(recent), replace=False)
        idx[b] = np.concatenate([rest, recent])
    cnt = torch.full((B,), k, dtype=torch.int32, device=DEV)
    lse = torch.empty((B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    out = dk.dustin_verify_attn(q2, kv, torch.from_numpy(idx).to(DEV), cnt, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        assert n1[b] == oracle.commit_window(int(n0[b]), int(accepted[b]), sh.w)
        pad = np.zeros((2 * sh.w, sh.Hkv, sh.d))
        K1, V1 = oracle.append_window_kv(np.concatenate([Kh[b], pad]), np.concatenate([Vh[b], pad]), int(n0[b]),
                                         f64(kw1[b]), f64(vw1[b]))
        K2, V2 = oracle.append_window_kv(K1, V1, int(n1[b]), f64(kw2[b]), f64(vw2[b]))
        O, L = oracle.verify_attention(f64(q2[b]), K2[:n1[b]], V2[:n1[b]], f64(kw2[b]), f64(vw2[b]), idx[b])
        err = np.abs(f64(out[b]) - O).max()
        lerr = np.abs(f64(lse[b]) - L).max()
        say(f"  b={b} n0={n0[b]} n1={n1[b]} max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 2e-3


def test_verify_edge_cases():
    """Empty set (only the causal window), an empty history, and a window
    that runs past the cache end (the rows beyond N_max are left out)."""
    say("verify edge cases")
    sh, x, k_win, v_win = _setup("verify-edges", dict(B=4, n=600, Hq=64, Hkv=8, k=64, L_d=1), room=False)
    N = x.K.shape[1]
    lens = np.array([300, 0, N - 2, 450], dtype=np.int32)
    x.seq_lens.copy_(torch.from_numpy(lens))
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    dk.dustin_append_window_kv(kv, k_win, v_win)
    idx = torch.full((4, 64), -1, dtype=torch.int32, device=DEV)
    idx[2, :10] = torch.arange(0, 100, 10, dtype=torch.int32)
    idx[2, 10:13] = torch.tensor([N - 2, N - 1, N + 3], dtype=torch.int32)   # window / past-end: ignored
    idx[3, :64] = torch.arange(64, dtype=torch.int32) * 7
    cnt = torch.tensor([0, 64, 13, 64], dtype=torch.int32, device=DEV)       # b=1: entries are all >= n_b = 0
    lse = torch.empty((4, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    out = dk.dustin_verify_attn(x.q, kv, idx, cnt, lse=lse)
    torch.cuda.synchronize()
    flat_k = x.K.reshape(-1, sh.Hkv, sh.d)
    for b in range(4):
        n = int(lens[b])
        I = valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        K, V = oracle_kv(x, "K", b), oracle_kv(x, "V", b)
        fit = min(sh.w, N - n)                                   # window rows inside the cache
        if fit == sh.w:
            O, L = oracle.verify_attention(f64(x.q[b]), K, V, f64(k_win[b]), f64(v_win[b]), I)
        else:
            # per query: the set I plus the window rows t <= s that lie inside the cache
            Kc = np.concatenate([K, f64(k_win[b, :fit])])
            Vc = np.concatenate([V, f64(v_win[b, :fit])])
            O = np.zeros((sh.w, sh.Hq, sh.d))
            L = np.zeros((sh.w, sh.Hq))
            for s in range(sh.w):
                J = np.concatenate([I, n + np.arange(min(s + 1, fit))])
                Os, Ls = oracle.sparse_attention(f64(x.q[b, s:s + 1]), Kc, Vc, J)
                O[s], L[s] = Os[0], Ls[0]
            assert torch.equal(flat_k[b * N + n: b * N + N].float(), k_win[b, :fit].float())
        err = np.abs(f64(out[b]) - O).max()
        lerr = np.abs(f64(lse[b]) - L).max()
        say(f"  b={b} n={n} |I|={len(I)} window rows {fit} max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 2e-3


FUSED_CASES = CASES + [
    ("full-history-qwen72b", dict(B=2, n=3000, Hq=64, Hkv=8, k=600, L_d=1), 600, dict(), False),
    ("full-history-paged", dict(base="c5", B=3, n=3000, n_lo=800, k=500, L_d=1), 500, dict(), False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_append_matches_separate_calls(case):
    """dustin_verify_attn_append (one launch for bf16) against
    dustin_append_window_kv + dustin_verify_attn on identical seeded inputs:
    out, lse and both caches bit-identical (the unused cache rows hold NaN, so
    the caches are compared as bit patterns); the fused output also against
    the oracle.  The full-history cases put some windows past N_max."""
    name, over, k, iopt = case[:4]
    room = case[4] if len(case) > 4 else True
    say("fused append + verify", name)
    sh, x1, k_win, v_win = _setup(name, over, room=room)
    _, x2, k_win2, v_win2 = _setup(name, over, room=room)
    assert torch.equal(k_win, k_win2) and torch.equal(v_win, v_win2)
    f32 = sh.dtype == "f32"
    kv1 = dk.KV(x1.K, x1.V, x1.seq_lens, x1.page_table)
    kv2 = dk.KV(x2.K, x2.V, x2.seq_lens, x2.page_table)
    if k is None:
        idx = cnt = None
    else:
        idx, cnt = make_idx(x1.seq_lens, k, seed=zlib.crc32(name.encode()) % 1000, device=DEV, **iopt)
    lse1 = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    lse2 = torch.empty_like(lse1)
    dk.dustin_append_window_kv(kv1, k_win, v_win)
    out1 = dk.dustin_verify_attn(x1.q, kv1, idx, cnt, lse=lse1)
    out2 = dk.dustin_verify_attn_append(x2.q, kv2, k_win, v_win, idx, cnt, lse=lse2)
    torch.cuda.synchronize()
    bits = torch.int32 if f32 else torch.int16
    assert torch.equal(x1.K.view(bits), x2.K.view(bits)), "K cache differs"
    assert torch.equal(x1.V.view(bits), x2.V.view(bits)), "V cache differs"
    assert torch.equal(out1.view(bits), out2.view(bits)), "output differs"
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32)), "lse differs"
    lens = x2.seq_lens.cpu().numpy()
    for b in range(sh.B):
        n = int(lens[b])
        I = np.arange(n) if idx is None else valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        K, V = oracle_kv(x2, "K", b), oracle_kv(x2, "V", b)
        # window rows present in the cache: positions below N_max whose page
        # (paged caches) is allocated; they form a prefix of the window
        nw = 0
        while nw < sh.w and n + nw < kv2.desc.N_max:
            if x2.page_table is not None:
                pg = int(x2.page_table[b, (n + nw) // sh.page_size])
                if not 0 <= pg < x2.K.shape[0]:
                    break
            nw += 1
        say(f"  b={b} n={n} |I|={len(I)} window rows in the cache {nw}")
        if len(I) == 0 and nw == 0:
            continue
        O, L = oracle.verify_attention(f64(x2.q[b]), K, V, f64(k_win[b, :nw]), f64(v_win[b, :nw]), I)
        assert np.abs(f64(out2[b]) - O).max() <= (1e-4 if f32 else 2e-2)
        assert np.abs(f64(lse2[b]) - L).max() <= (1e-5 if f32 else 2e-3)
