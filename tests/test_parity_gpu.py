"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Tolerances (from the benchmark spec and the arithmetic):
  attention output   max-abs 2e-2 (bf16 storage, fp32 accumulation, P
                     rounded to bf16 for the PV MFMA); 1e-4 for float32
  attention lse      abs 2e-3 (bf16) / 1e-5 (float32)
  index sets         bit-exact when the oracle's tier rule runs on the GPU's
                     own scores; against the fp64 oracle scores, differences
                     only within 1e-5 relative of a tier threshold
  scores             |d| <= 1e-5 * S + 1e-9 per position: fp32 accumulation
                     of bf16 products and an fp32 log-sum-exp over up to
                     131072 positions, against fp64
  window weights A   abs 1e-5 (each weight <= 1); ARR abs 1e-4
"""
import zlib

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import assert_scores_close, check_set_tieband, f64, make_idx, max_rel_err, oracle_kv, say, valid_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(base, **kw):
    return synth.preset(base).replace(**kw)


ATTN_CASES = [
    # name, shape overrides, k, idx options
    ("qwen32b-rows20", dict(B=2, n=3000, Hq=40, Hkv=8, k=300, L_d=1), 300, dict()),
    ("qwen72b-rows32", dict(B=2, n=5000, Hq=64, Hkv=8, k=1000, L_d=1), 1000, dict(frac_invalid=0.05, short=7)),
    ("qwen7b-rows28-tail", dict(B=3, n=2333, Hq=28, Hkv=4, k=517, L_d=1), 517, dict(shuffle=False)),
    ("paged-ragged-rows64", dict(base="c5", B=3, n=4000, n_lo=700, k=700, L_d=1), 700, dict(frac_invalid=0.02)),
    ("d64-rows16", dict(B=2, n=2000, Hq=8, Hkv=2, d=64, k=257, L_d=1), 257, dict()),
    # head_dim 32: 16 rows padded to two row blocks; 64 rows in four
    ("d32-rows16", dict(B=2, n=2000, Hq=8, Hkv=2, d=32, k=257, L_d=1), 257, dict(frac_invalid=0.05)),
    ("d32-rows64", dict(B=2, n=2600, Hq=32, Hkv=2, d=32, k=700, L_d=1), 700, dict(short=5)),
    ("k1", dict(B=2, n=500, Hq=64, Hkv=8, k=1, L_d=1), 1, dict()),
    ("tiny-f32", dict(base="c1"), 128, dict()),
]


def _make(name, over):
    over = dict(over)
    base = over.pop("base", "c4" if name != "tiny-f32" else "c1")
    return synth.make(_shape(base, **over), device=DEV)


@pytest.mark.parametrize("name,over,k,iopt", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_sparse_attention_matches_oracle(name, over, k, iopt):
    say("sparse attention", name)
    x = _make(name, over)
    sh = x.shape
    idx, cnt = make_idx(x.seq_lens, k, seed=zlib.crc32(name.encode()) % 1000, device=DEV, **iopt)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    lse = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    out = dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt, lse=lse)
    out2 = dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8) if out.dtype != torch.float32 else out, out2.view(torch.uint8) if out2.dtype != torch.float32 else out2), "not deterministic"
    f32 = sh.dtype == "f32"
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        I = valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        O, L = oracle.sparse_attention(f64(x.q[b]), oracle_kv(x, "K", b), oracle_kv(x, "V", b), I)
        err = np.abs(f64(out[b]) - O).max()
        lerr = np.abs(f64(lse[b]) - L).max()
        say(f"  b={b} n={n} |I|={len(I)} max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= (1e-4 if f32 else 2e-2)
        assert lerr <= (1e-5 if f32 else 2e-3)


@pytest.mark.parametrize("name,over", [
    ("dense-qwen72b", dict(B=2, n=4100, Hq=64, Hkv=8, L_d=1)),
    ("dense-paged", dict(base="c5", B=2, n=3000, n_lo=900, L_d=1)),
    ("dense-d32", dict(B=2, n=2100, Hq=16, Hkv=4, d=32, L_d=1)),
    ("dense-f32", dict(base="c1")),
])
def test_dense_attention_matches_oracle(name, over):
    say("dense attention", name)
    x = _make(name, over)
    sh = x.shape
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    out = dk.dustin_sparse_verify_attn(x.q, kv)
    torch.cuda.synchronize()
    for b in range(sh.B):
        O = oracle.dense_attention(f64(x.q[b]), oracle_kv(x, "K", b), oracle_kv(x, "V", b))
        err = np.abs(f64(out[b]) - O).max()
        say(f"  b={b} max|dO|={err:.2e}")
        assert err <= (1e-4 if sh.dtype == "f32" else 2e-2)


def test_attention_edge_cases():
    say("attention edge cases")
    x = _make("edge", dict(B=3, n=300, Hq=64, Hkv=8, k=64, L_d=1))
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    idx = torch.full((3, 64), -1, dtype=torch.int32, device=DEV)
    idx[1, :5] = torch.tensor([7, 300, -5, 299, 1000], dtype=torch.int32)   # mixed valid / invalid
    idx[2, :64] = torch.arange(64, dtype=torch.int32)
    cnt = torch.tensor([0, 5, 3], dtype=torch.int32, device=DEV)            # b=0: empty set
    lse = torch.empty((3, 4, 64), dtype=torch.float32, device=DEV)
    out = dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out[0].float() == 0) and torch.all(torch.isneginf(lse[0]))
    for b, I in ((1, [7, 299]), (2, [0, 1, 2])):
        O, L = oracle.sparse_attention(f64(x.q[b]), oracle_kv(x, "K", b), oracle_kv(x, "V", b), I)
        assert np.abs(f64(out[b]) - O).max() <= 2e-2
        assert np.abs(f64(lse[b]) - L).max() <= 2e-3


def test_attention_workspace_reused_across_shapes():
    """One workspace serves a dense call with few (b, KV head) groups and many
    splits, then a sparse call with 128 groups: the second call's arrival
    counters must not land on the partials the first one stored."""
    say("attention workspace reused across shapes")
    ws = dk.Workspace()
    x1 = _make("ws-dense", dict(B=2, n=8000, Hq=64, Hkv=8, L_d=1))
    kv1 = dk.KV(x1.K, x1.V, x1.seq_lens, x1.page_table)
    d1 = kv1.desc
    n1 = dk.lib().dustin_attn_workspace_bytes(d1.B, 4, 64, 8, 128, d1.N_max)
    dk.dustin_sparse_verify_attn(x1.q, kv1, ws=ws)
    x2 = _make("ws-sparse", dict(B=16, n=1000, Hq=64, Hkv=8, k=256, L_d=1))
    kv2 = dk.KV(x2.K, x2.V, x2.seq_lens, x2.page_table)
    n2 = dk.lib().dustin_attn_workspace_bytes(16, 4, 64, 8, 128, 256)
    assert n2 <= n1, "the second call must reuse the first call's workspace"
    idx, cnt = make_idx(x2.seq_lens, 256, seed=11, device=DEV)
    out = dk.dustin_sparse_verify_attn(x2.q, kv2, idx, cnt, ws=ws)
    torch.cuda.synchronize()
    for b in (0, 9, 15):
        n = int(x2.seq_lens[b])
        I = valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        O, _ = oracle.sparse_attention(f64(x2.q[b]), oracle_kv(x2, "K", b), oracle_kv(x2, "V", b), I)
        err = np.abs(f64(out[b]) - O).max()
        say(f"  b={b} max|dO|={err:.2e}")
        assert err <= 2e-2


SELECT_CASES = [
    (dict(B=3, N=5000, k=512, m=200, ns=4, nw=32, ties=True), "ties"),
    (dict(B=2, N=3000, k=700, m=0, ns=0, nw=0, ties=False), "target-only"),
    (dict(B=2, N=3000, k=700, m=700, ns=0, nw=0, ties=False), "draft-only"),
    (dict(B=4, N=1000, k=2048, m=100, ns=4, nw=32, ties=True), "k>=n"),
    (dict(B=1, N=131072, k=4096, m=2030, ns=4, nw=32, ties=False), "long"),
    (dict(B=2, N=140000, k=1000, m=400, ns=4, nw=32, ties=True), "longer-than-registers"),
    (dict(B=2, N=2500, k=333, m=50, ns=8, nw=8, ties=True, no_draft=True), "no-draft"),
    (dict(B=2, N=2500, k=333, m=50, ns=8, nw=8, ties=True, no_target=True), "no-target"),
    (dict(B=3, N=65536, k=2048, m=1006, ns=4, nw=32, ties=True), "two-words-ties"),
    (dict(B=2, N=32768, k=2048, m=1006, ns=4, nw=32, ties=False, equal=True), "all-equal"),
    (dict(B=2, N=98304, k=4096, m=2030, ns=4, nw=32, ties=False, narrow=True), "narrow-range"),
    # rows of 32769 .. 262144 positions go through the chunked (multi-work-group) select
    (dict(B=3, N=50000, k=1500, m=600, ns=4, nw=32, ties=True, empty_last=True), "chunked-ties-empty"),
    (dict(B=2, N=65536, k=2048, m=1006, ns=4, nw=32, ties=False, equal=True), "chunked-all-equal"),
    (dict(B=2, N=70000, k=900, m=50, ns=8, nw=8, ties=True, no_draft=True), "chunked-no-draft"),
    (dict(B=2, N=70000, k=900, m=50, ns=8, nw=8, ties=True, no_target=True), "chunked-no-target"),
    (dict(B=2, N=40000, k=50000, m=100, ns=4, nw=32, ties=True), "chunked-k>=n"),
    (dict(B=2, N=262144, k=8192, m=4000, ns=4, nw=32, ties=True), "chunked-max"),
    (dict(B=2, N=300000, k=4096, m=2000, ns=4, nw=32, ties=True), "beyond-chunked"),
]


@pytest.mark.parametrize("cfg,name", SELECT_CASES, ids=[c[1] for c in SELECT_CASES])
def test_select_is_bit_exact(cfg, name):
    say("select", name)
    rng = np.random.default_rng(len(name))
    B, N, k = cfg["B"], cfg["N"], cfg["k"]
    lens = rng.integers(max(1, N // 3), N + 1, size=B).astype(np.int32)
    lens[0] = N
    if B > 2:
        lens[-1] = 0 if (name == "ties" or cfg.get("empty_last")) else lens[-1]
    if cfg.get("equal"):     # one key value: every selection is decided by position alone
        sd = np.full((B, N), 0.25, dtype=np.float32)
        st = np.full((B, N), 3.0, dtype=np.float32)
    elif cfg.get("narrow"):  # keys within one binade, a few patterns apart at the top
        sd = (1.0 + rng.integers(0, 1 << 12, size=(B, N)) * 2.0 ** -23).astype(np.float32)
        st = (1.0 + rng.integers(0, 300, size=(B, N)) * 2.0 ** -23).astype(np.float32)
    elif cfg["ties"]:
        sd = rng.integers(0, 50, size=(B, N)).astype(np.float32) / 7.0
        st = rng.integers(0, 50, size=(B, N)).astype(np.float32) / 3.0
    else:
        sd = rng.random((B, N), dtype=np.float32)
        st = rng.random((B, N), dtype=np.float32) * 1e-3
    sdt = None if cfg.get("no_draft") else torch.from_numpy(sd).to(DEV)
    stt = None if cfg.get("no_target") else torch.from_numpy(st).to(DEV)
    lt = torch.from_numpy(lens).to(DEV)
    idx, cnt, tier = dk.dustin_topk(sdt, stt, lt, k, cfg["m"], cfg["ns"], cfg["nw"])
    torch.cuda.synchronize()
    for b in range(B):
        n = int(lens[b])
        I, T = oracle.select_verify_set(None if sdt is None else sd[b, :n], None if stt is None else st[b, :n],
                                        n, k, cfg["m"], cfg["ns"], cfg["nw"])
        c = int(cnt[b])
        assert c == len(I) == min(k, n)
        assert (idx[b, :c].cpu().numpy() == I).all()
        assert (tier[b, :c].cpu().numpy() == T).all()
        assert (idx[b, c:] == -1).all() and (tier[b, c:] == -1).all()


SCORE_CASES = [
    ("qwen7b-ragged", dict(base="c2", B=3, n=2100, L_d=3, n_lo=900)),
    ("paged-drift", dict(base="c5", B=2, n=3000, n_lo=1200, L_d=2)),
    ("qwen72b-packed", dict(base="c4", B=2, n=1700, L_d=2, S=8)),
    ("stream-ragged", dict(base="c2", B=3, n=5000, L_d=4, n_lo=700)),
    ("stream-layer-groups", dict(base="c2", B=2, n=3000, L_d=6, n_lo=1000)),
    ("stream-paged", dict(base="c5", B=3, n=5000, n_lo=1200, L_d=4, w=4)),
    ("stream-many-groups", dict(base="c2", B=1, n=2048, L_d=24)),          # 12 layer groups
    ("stream-one-head-rb4", dict(base="c4", B=2, n=3000, L_d=2, w=8)),      # 56 rows: one KV head per item
    # 12 draft heads over 2 KV heads, 6 steps: 36 rows, one KV head per item, ragged
    ("stream-one-head-rb3", dict(base="c2", B=2, n=2500, n_lo=900, L_d=4, H_d=12, w=6)),
    # 56 rows, one KV head per item, 8 layers in 4 groups: 8 (group, head) partials
    ("stream-one-head-groups", dict(base="c4", B=1, n=2048, L_d=8, w=8)),
    ("stream-odd-layers", dict(base="c2", B=2, n=3000, n_lo=1100, L_d=5)),     # 28 rows, five layers
    ("stream-one-head-odd-layers", dict(base="c4", B=2, n=2500, L_d=3, w=8)),  # 56 rows, three layers
    # draft head_dim 128: the register-staged passes at two, three and four row blocks
    ("mfma-d128-rb2", dict(base="c2", B=2, n=2300, n_lo=800, L_d=2, d_d=128)),
    ("mfma-d128-rb3", dict(base="c2", B=2, n=2000, L_d=3, d_d=128, H_d=12, w=6)),
    ("mfma-d128-rb4-paged", dict(base="c5", B=2, n=2600, n_lo=900, L_d=2, d_d=128)),
    # 140000 positions: 547 target chunks of 256, past the 512 per-chunk pairs
    # the row normaliser holds in registers (its loop form)
    ("long-row-normaliser-loop", dict(base="c2", B=1, n=140000, L_d=1)),
    ("tiny-f32", dict(base="c1")),
]


@pytest.mark.parametrize("name,over", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_scores_match_oracle(name, over):
    say("scores", name)
    over = dict(over)
    base = over.pop("base")
    sh = synth.preset(base).replace(**over)
    x = synth.make(sh, device=DEV)
    sub = x.sub_heads
    q_hist = x.q_hist
    if name == "qwen72b-packed":   # all scored heads in one KV group
        sub = [(0, h) for h in range(sh.S)]
        q_hist = x.q[:, 0, :sh.S].contiguous()
    kvs = [dk.KV(x.K, None, x.seq_lens, x.page_table)]
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
    s_d, s_t = dk.dustin_score(dkv, x.q_draft, kvs, q_hist, sub, sh.Hq)
    s_d2, s_t2 = dk.dustin_score(dkv, x.q_draft, kvs, q_hist, sub, sh.Hq)
    torch.cuda.synchronize()
    assert torch.equal(s_d, s_d2) and torch.equal(s_t, s_t2), "not deterministic"
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        K = oracle_kv(x, "K", b)
        st = oracle.score_target(f64(q_hist[b]), {0: K}, sub, sh.Hq)
        sd = oracle.score_draft(f64(x.q_draft[b]), oracle_kv(x, "Kd", b))
        gt, gd = f64(s_t[b, :n]), f64(s_d[b, :n])
        rt, rd = max_rel_err(gt, st), max_rel_err(gd, sd)
        say(f"  b={b} n={n} max rel|dS_T|={rt:.2e} rel|dS_D|={rd:.2e} (S >= 1e-6) "
            f"sums {gt.sum():.5f}/{len(sub)} {gd.sum():.4f}/{sh.L_d*sh.H_d*sh.w}")
        assert_scores_close(gt, st, "S_Target")
        assert_scores_close(gd, sd, "S_Draft")
        assert abs(gt.sum() - len(sub)) < 1e-3 * len(sub)
        assert abs(gd.sum() - sh.L_d * sh.H_d * sh.w) < 1e-3 * sh.L_d * sh.H_d * sh.w
        assert (f64(s_t[b, n:]) == 0).all() and (f64(s_d[b, n:]) == 0).all()


@pytest.mark.parametrize("layout,paged", [("two-rows-per-kv-head", False), ("two-rows-per-kv-head", True),
                                           ("split-units", False)],
                         ids=["rows-2-per-head", "rows-2-per-head-paged", "units-not-one-per-head"])
def test_target_scores_whole_row_form(layout, paged):
    """S_Target when the scored rows of one layer use every KV head (the
    whole-row statistics pass) with two rows per KV head, contiguous and
    paged; and with rows of one KV head that are not adjacent (two units for
    that head: the per-unit pass).  The oracle scores the same pairs."""
    say("target scores", layout, "paged" if paged else "contiguous")
    sh = synth.preset("c5" if paged else "c2").replace(B=2, n=3000, n_lo=1100, L_d=1, Hq=28, Hkv=4, S=8)
    x = synth.make(sh, device=DEV)
    G = sh.Hq // sh.Hkv
    if layout == "two-rows-per-kv-head":
        heads = [0, 1, G, G + 3, 2 * G + 1, 2 * G + 6, 3 * G, 3 * G + 2]
    else:
        heads = [0, G, 1, 2 * G, 3 * G, 2 * G + 1, 3 * G + 4, G + 5]
    sub = [(0, h) for h in heads]
    qh = x.q[:, -1][:, heads].contiguous()
    kvs = [dk.KV(x.K, None, x.seq_lens, x.page_table)]
    _, s_t = dk.dustin_score([], None, kvs, qh, sub, sh.Hq, want_draft=False)
    torch.cuda.synchronize()
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        st = oracle.score_target(f64(qh[b]), {0: oracle_kv(x, "K", b)}, sub, sh.Hq)
        say(f"  b={b} n={n} max rel|dS_T|={max_rel_err(f64(s_t[b, :n]), st):.2e}")
        assert_scores_close(f64(s_t[b, :n]), st, "S_Target")
        assert (f64(s_t[b, n:]) == 0).all()


# Every head of a layer scored (five to eight rows per KV head: the matrix-
# core whole-row pass).  The shapes pick how the KV heads are split over
# work-groups: one head per group with four waves sharing its subtiles (few
# chunks), two heads, four heads, all eight heads per group (two per wave).
ALL_HEADS_CASES = [
    ("g7-hkv4-one-head-per-group", dict(base="c2", B=2, n=3000, n_lo=1100), None, False),
    ("g8-paged-ragged-empty", dict(base="c5", B=3, n=2600, n_lo=700), None, True),
    ("g8-two-heads-per-group", dict(base="c4", B=2, n=40000), None, False),
    ("g8-four-heads-per-group", dict(base="c4", B=4, n=40000), [0, 3], False),
    ("g8-eight-heads-per-group", dict(base="c4", B=8, n=32768), [1, 6], False),
]


@pytest.mark.parametrize("name,over,check,empty_last", ALL_HEADS_CASES, ids=[c[0] for c in ALL_HEADS_CASES])
def test_target_scores_all_heads(name, over, check, empty_last):
    """S_Target over every head of one layer, and the per-head softmax rows
    (dustin_head_scores), against the oracle on the same heads: contiguous
    and paged caches, ragged lengths that end inside a chunk, an empty
    sequence, and each split of the KV heads over work-groups."""
    say("all-heads target scores", name)
    over = dict(over)
    sh = synth.preset(over.pop("base")).replace(L_d=1, **over)
    x = synth.make(sh, device=DEV)
    lens = x.seq_lens.clone()
    if empty_last:
        lens[-1] = 0
    heads = [(0, h) for h in range(sh.Hq)]
    qh = x.q[:, -1].contiguous()
    kvs = [dk.KV(x.K, None, lens, x.page_table)]
    _, s_t = dk.dustin_score([], None, kvs, qh, heads, sh.Hq, want_draft=False)
    rows = dk.dustin_head_scores(kvs, qh, heads, sh.Hq)
    _, s_t2 = dk.dustin_score([], None, kvs, qh, heads, sh.Hq, want_draft=False)
    torch.cuda.synchronize()
    assert torch.equal(s_t, s_t2), "not deterministic"
    for b in (check if check is not None else range(sh.B)):
        n = int(lens[b])
        if n == 0:
            assert (f64(s_t[b]) == 0).all() and (f64(rows[:, b]) == 0).all()
            continue
        K = oracle_kv(x, "K", b)[:n]
        st = oracle.score_target(f64(qh[b]), {0: K}, heads, sh.Hq)
        hp = oracle.head_probs(f64(qh[b])[None], K)[:, 0]
        say(f"  b={b} n={n} max rel|dS_T|={max_rel_err(f64(s_t[b, :n]), st):.2e} "
            f"rows {max_rel_err(f64(rows[:, b, :n]).ravel(), hp.ravel()):.2e}")
        assert_scores_close(f64(s_t[b, :n]), st, "S_Target")
        assert_scores_close(f64(rows[:, b, :n]).ravel(), hp.ravel(), "head rows")
        assert (f64(s_t[b, n:]) == 0).all() and (f64(rows[:, b, n:]) == 0).all()
        assert abs(f64(s_t[b, :n]).sum() - sh.Hq) < 1e-3 * sh.Hq


LSE_CASES = [
    ("stream-ragged-empty", dict(base="c2", B=3, n=3000, L_d=3, n_lo=900), True),   # last sequence empty
    ("stream-one-head-paged", dict(base="c5", B=2, n=3000, n_lo=1200, L_d=2, w=8), False),
    ("stream-layer-groups", dict(base="c2", B=1, n=2048, L_d=24), False),
    ("mfma-one-kv-head", dict(base="c2", B=2, n=2100, L_d=2, Hkv_d=1, H_d=8), False),
    ("tiny-f32", dict(base="c1"), False),
]


@pytest.mark.parametrize("name,over,empty_last", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_draft_row_lse_and_supplied_normalisers(name, over, empty_last):
    """The row normalisers of S_Draft's softmaxes (dustin_draft_row_lse)
    against the oracle's, and S_Draft computed from normalisers the caller
    supplies (one read of the draft keys) against the oracle's S_Draft given
    the same normalisers: the oracle's own, then the same with one row's
    raised by ln 2 in each sequence (that row's terms halve)."""
    say("draft row normalisers", name)
    over = dict(over)
    base = over.pop("base")
    sh = synth.preset(base).replace(**over)
    x = synth.make(sh, device=DEV)
    lens = x.seq_lens.clone()
    if empty_last:
        lens[-1] = 0
    dkv = [dk.KV(x.Kd[l], None, lens, x.page_table) for l in range(sh.L_d)]
    lse = dk.dustin_draft_row_lse(dkv, x.q_draft)
    torch.cuda.synchronize()
    lse_ref = np.empty((sh.B, sh.L_d, sh.w, sh.H_d))
    for b in range(sh.B):
        n = int(lens[b])
        Kd = oracle_kv(x, "Kd", b)[:, :n] if n else np.zeros((sh.L_d, 0, sh.Hkv_d, sh.d_d))
        lse_ref[b] = oracle.draft_row_lse(f64(x.q_draft[b]), Kd)
    got = f64(lse)
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(got) == ~fin).all(), "empty rows must read -inf"
    err = np.abs(got[fin] - lse_ref[fin]).max()
    say(f"  max |d lse| = {err:.2e}")
    assert err <= 2e-5 + 2e-6 * np.abs(lse_ref[fin]).max()
    shifted = lse_ref.copy()
    for b in range(sh.B):
        shifted[b, sh.L_d - 1, 0, sh.H_d - 1] += math.log(2.0)
    for given in (lse_ref, shifted):
        given32 = given.astype(np.float32)
        s_d, _ = dk.dustin_score(dkv, x.q_draft, [], None, None, sh.Hq, want_target=False,
                                 draft_lse=torch.from_numpy(given32).to(DEV))
        torch.cuda.synchronize()
        for b in range(sh.B):
            n = int(lens[b])
            assert (f64(s_d[b, n:]) == 0).all()
            if n == 0:
                continue
            ref = oracle.score_draft_given_lse(f64(x.q_draft[b]), oracle_kv(x, "Kd", b)[:, :n], given32[b].astype(np.float64))
            say(f"  b={b} n={n} max rel|dS_D| = {max_rel_err(f64(s_d[b, :n]), ref):.2e}")
            assert_scores_close(f64(s_d[b, :n]), ref, "S_Draft from supplied normalisers")


def test_scores_on_searched_subsets():
    """Dustin-H restricted to a searched configuration (blog section 2.4,
    Fig. 6; section 3 Fig. 8): S_Draft over a subset of the draft layers (not
    contiguous, in the caller's order) and S_Target over heads that sit in
    three different target layers, each layer its own cache.  The oracle
    scores the same subsets from the same layers."""
    say("scores on a draft-layer subset and target heads over three layers")
    sh = synth.preset("c4").replace(B=2, n=3000, L_d=6)
    x = synth.make(sh, device=DEV)
    layers = [1, 4, 5, 2, 0]                     # the searched draft layers, in the caller's order
    qd = x.q_draft[:, layers].contiguous()
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens) for l in layers]
    # three target layers: the generated cache and two position-rotated copies of it
    Kt = [x.K, torch.roll(x.K, 7, dims=1).contiguous(), torch.roll(x.K, -123, dims=1).contiguous()]
    kvs = [dk.KV(K, None, x.seq_lens) for K in Kt]
    sub = [(2, 9), (0, 40), (1, 17), (2, 63), (1, 0)]    # (layer, head): heads of KV groups 1, 5, 2, 7, 0
    qh = x.q[:, -1][:, [h for _, h in sub]].contiguous()
    s_d, s_t = dk.dustin_score(dkv, qd, kvs, qh, sub, sh.Hq)
    torch.cuda.synchronize()
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        Ko = {l: f64(Kt[l][b, :n]) for l in range(3)}
        st = oracle.score_target(f64(qh[b]), Ko, sub, sh.Hq)
        sd = oracle.score_draft(f64(qd[b]), f64(x.Kd[layers, b, :n]))
        say(f"  b={b} n={n} max rel|dS_T|={max_rel_err(f64(s_t[b, :n]), st):.2e} "
            f"rel|dS_D|={max_rel_err(f64(s_d[b, :n]), sd):.2e}")
        assert_scores_close(f64(s_t[b, :n]), st, "S_Target")
        assert_scores_close(f64(s_d[b, :n]), sd, "S_Draft")
        assert abs(float(s_d[b, :n].double().sum()) - len(layers) * sh.H_d * sh.w) < 1e-3 * len(layers) * sh.H_d * sh.w


@pytest.mark.parametrize("w", [4, 8], ids=["both-heads-per-item-w4", "one-head-per-item-w8"])
def test_scores_treat_absent_pages_as_zero_keys(w):
    """Page ids outside [0, num_pages) inside a sequence: both scores treat
    those positions as all-zero keys (the documented convention), on the
    streaming draft passes with both KV heads per item (28 rows) and with
    one KV head per item (56 rows).
    The oracle gets the logical keys with exactly those rows zeroed."""
    say("scores with absent pages, w", w)
    sh = synth.preset("c5").replace(B=2, n=3000, n_lo=1200, L_d=2, w=w)
    x = synth.make(sh, device=DEV)
    rng = np.random.default_rng(w)
    pt = x.page_table.clone()
    gone = {}
    for b in range(sh.B):
        npg = (int(x.seq_lens[b]) + 15) // 16
        gone[b] = rng.choice(npg - 1, 2, replace=False)
        pt[b, int(gone[b][0])] = -1
        pt[b, int(gone[b][1])] = x.K.shape[0] + 7          # past num_pages
    kvs = [dk.KV(x.K, None, x.seq_lens, pt)]
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, pt) for l in range(sh.L_d)]
    s_d, s_t = dk.dustin_score(dkv, x.q_draft, kvs, x.q_hist, x.sub_heads, sh.Hq)
    torch.cuda.synchronize()
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        K, Kd = oracle_kv(x, "K", b).copy(), oracle_kv(x, "Kd", b).copy()
        for pg in gone[b]:
            K[pg * 16:(pg + 1) * 16] = 0.0
            Kd[:, pg * 16:(pg + 1) * 16] = 0.0
        st = oracle.score_target(f64(x.q_hist[b]), {0: K}, x.sub_heads, sh.Hq)
        sd = oracle.score_draft(f64(x.q_draft[b]), Kd)
        assert_scores_close(f64(s_t[b, :n]), st, "S_Target")
        assert_scores_close(f64(s_d[b, :n]), sd, "S_Draft")


@pytest.mark.parametrize("name,over", [
    ("qwen72b", dict(base="c4", B=2, n=3000, L_d=1)),                       # 32 rows per KV head
    ("qwen7b-rows28", dict(base="c2", B=2, n=2600, n_lo=900, L_d=1)),        # 7 rows per step
    ("d64-one-step", dict(base="c4", B=2, n=2100, Hq=8, Hkv=2, d=64, w=1, L_d=1)),
    ("paged-one-step", dict(base="c5", B=2, n=2000, n_lo=800, w=1, L_d=1)),
    ("paged", dict(base="c5", B=2, n=2000, n_lo=800, L_d=1)),                # w = 8: two slices of 4 steps
    ("w6-slices-4-2", dict(base="c4", B=2, n=2300, w=6, L_d=1)),
    ("w5-g16", dict(base="c4", B=2, n=2200, Hq=64, Hkv=4, w=5, L_d=1)),      # 64 rows per slice of 4
    ("w3-g32-d64", dict(base="c4", B=2, n=1900, Hq=64, Hkv=2, d=64, w=3, L_d=1)),   # slices of 2 steps
    ("w16-g7", dict(base="c2", B=1, n=2000, w=16, L_d=1)),                   # four slices
    ("d32-bf16", dict(base="c4", B=2, n=2000, Hq=8, Hkv=2, d=32, L_d=1)),    # head_dim 32
    ("tiny-f32", dict(base="c1")),                                           # float32: the dense-pass form
])
def test_window_attention_and_arr(name, over):
    say("window attention + ARR", name)
    over = dict(over)
    sh = synth.preset(over.pop("base")).replace(**over)
    x = synth.make(sh, device=DEV)
    kv = dk.KV(x.K, None, x.seq_lens, x.page_table)
    A = dk.dustin_window_attn(x.q, kv)
    idx, cnt = make_idx(x.seq_lens, min(sh.k, 512), seed=3, device=DEV)
    arr_s, arr_w = dk.dustin_arr(A, x.seq_lens, idx, cnt)
    # SD oracle through the select call on the window-mean weights
    Abar = A.mean(dim=1).contiguous()
    oi, oc, _ = dk.dustin_topk(None, Abar, x.seq_lens, 64, 0, 0, 0)
    torch.cuda.synchronize()
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        Aref = oracle.window_attention(f64(x.q[b]), oracle_kv(x, "K", b))
        err = np.abs(f64(A[b, :, :n]) - Aref).max()
        I = valid_set(idx[b].cpu().numpy(), int(cnt[b]), n)
        say(f"  b={b} max|dA|={err:.2e} arr={float(arr_w[b]):.5f}/{oracle.arr_window(Aref, I):.5f}")
        assert err < 1e-5
        assert (f64(A[b, :, n:]) == 0).all()
        np.testing.assert_allclose(f64(arr_s[b]), oracle.arr_step(Aref, I), atol=1e-4)
        assert abs(float(arr_w[b]) - oracle.arr_window(Aref, I)) < 1e-4
        # SD oracle (Eq. 3-4): the GPU's TopK of its own Abar against the
        # oracle's set, equal except at ties within 1e-5 of the 64-th score
        sel, arr_orc, Abar_ref = oracle.sd_oracle(Aref, 64)
        g = oi[b, :int(oc[b])].cpu().numpy()
        nd = check_set_tieband(g, np.full(len(g), 2), sel, np.full(len(sel), 2), None, Abar_ref)
        assert abs(Abar_ref[g].sum() - arr_orc) < 1e-5
        say(f"    SD-oracle set: {len(g)} positions, {nd} differ (tie band)")


def test_window_attention_paths_share_a_workspace():
    """The statistics form (bf16; w = 8 in two slices) and the dense-pass
    form (float32) of the window attention run on one workspace in both
    orders; the statistics form must leave the attention arrival counters at
    the workspace's start untouched (zero)."""
    say("window attention: both forms on one workspace")
    ws = dk.Workspace()
    buf = ws.get(1 << 28, torch.device("cuda", torch.cuda.current_device()))   # large enough for all three calls
    ptr = buf.data_ptr()
    for base, over in (("c4", dict(B=2, n=1500, L_d=1)), ("c1", dict(n=1500)),
                       ("c5", dict(B=2, n=1500, n_lo=700, L_d=1)), ("c1", dict(n=1300, seed=9)),
                       ("c4", dict(B=2, n=1500, L_d=1, seed=9))):
        sh = synth.preset(base).replace(**over)
        x = synth.make(sh, device=DEV)
        kv = dk.KV(x.K, None, x.seq_lens, x.page_table)
        A = dk.dustin_window_attn(x.q, kv, ws=ws)
        torch.cuda.synchronize()
        b = 0
        n = int(x.seq_lens[b])
        Aref = oracle.window_attention(f64(x.q[b]), oracle_kv(x, "K", b))
        err = np.abs(f64(A[b, :, :n]) - Aref).max()
        say(f"  {base} w={sh.w}: max|dA|={err:.2e}")
        assert err < 1e-5
        assert ws.buf.data_ptr() == ptr              # the same (never re-zeroed) buffer throughout
