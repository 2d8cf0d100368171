"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: score -> select -> sparse attention (and the dense baseline) on the
real shapes, checked against the oracle on sampled sequences (the oracle
computes those one by one) and, for every sequence, through properties that
hold at any size (score sums; the set's tier invariants on the GPU's own
scores, checked directly, not through the oracle).  The oracle only ever
sees the seeded inputs: its own scores, its own set and its own attention.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import assert_scores_close, check_set_tieband, check_sweep_rows, check_tier_rule, f64, max_rel_err, oracle_kv, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_step(sh, x, k):
    """The bench step's calls (layer 0) with the library's own planning."""
    n_sink, n_window, m = synth.tier_defaults(k)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
    s_d, s_t = dk.dustin_score(dkv, x.q_draft, [kv], x.q_hist, x.sub_heads, sh.Hq)
    idx, cnt, tier = dk.dustin_topk(s_d, s_t, x.seq_lens, k, m, n_sink, n_window)
    out = dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt)
    torch.cuda.synchronize()
    return (n_sink, n_window, m), kv, s_d, s_t, idx, cnt, tier, out


def _check(sh, x, k, sample):
    (n_sink, n_window, m), kv, s_d, s_t, idx, cnt, tier, out = _run_step(sh, x, k)
    lens = x.seq_lens.cpu().numpy()
    S, rows_d = len(x.sub_heads), sh.L_d * sh.H_d * sh.w
    # every sequence: score sums and the set's tier invariants on the GPU's own scores
    sd_all, st_all = s_d.cpu().numpy(), s_t.cpu().numpy()
    idx_all, tier_all, cnt_all = idx.cpu().numpy(), tier.cpu().numpy(), cnt.cpu().numpy()
    for b in range(sh.B):
        n = int(lens[b])
        assert abs(st_all[b, :n].astype(np.float64).sum() - S) < 1e-3 * S
        assert abs(sd_all[b, :n].astype(np.float64).sum() - rows_d) < 1e-3 * rows_d
        assert (st_all[b, n:] == 0).all() and (sd_all[b, n:] == 0).all()
        check_tier_rule(idx_all[b], tier_all[b], int(cnt_all[b]), sd_all[b, :n], st_all[b, :n], n, k, m,
                        n_sink, n_window)
    # sampled sequences: scores, end-to-end set and attention against the oracle
    for b in sample:
        n = int(lens[b])
        K = oracle_kv(x, "K", b)
        st = oracle.score_target(f64(x.q_hist[b]), {0: K}, x.sub_heads, sh.Hq)
        sd = oracle.score_draft(f64(x.q_draft[b]), oracle_kv(x, "Kd", b))
        assert_scores_close(f64(s_t[b, :n]), st, "S_Target")
        assert_scores_close(f64(s_d[b, :n]), sd, "S_Draft")
        say(f"  b={b} max rel|dS_T|={max_rel_err(f64(s_t[b, :n]), st):.2e} "
            f"rel|dS_D|={max_rel_err(f64(s_d[b, :n]), sd):.2e} (S >= 1e-6)")
        oi, ot = oracle.select_verify_set(sd, st, n, k, m, n_sink, n_window)
        c = int(cnt[b])
        nd = check_set_tieband(idx[b, :c].cpu().numpy(), tier[b, :c].cpu().numpy(), oi, ot, sd, st)
        O, _ = oracle.sparse_attention(f64(x.q[b]), K, oracle_kv(x, "V", b), oi)
        got = out[b]
        if nd:   # the sets differ at near-ties: attend the oracle's set on the GPU as well
            oidx = torch.full((sh.B, k), -1, dtype=torch.int32, device=DEV)
            ocnt = torch.zeros((sh.B,), dtype=torch.int32, device=DEV)
            oidx[b, :len(oi)] = torch.from_numpy(np.asarray(oi, dtype=np.int32)).to(DEV)
            ocnt[b] = len(oi)
            got = dk.dustin_sparse_verify_attn(x.q, kv, oidx, ocnt)[b]
            torch.cuda.synchronize()
        err = np.abs(f64(got) - O).max()
        say(f"  b={b} n={n} k={k}: set diff {nd} (tie band), attention max|dO|={err:.2e}")
        assert err <= 2e-2
    return kv


@pytest.mark.parametrize("k", [512, 1024, 2048])
def test_c4_headline_step(k):
    """72B-shaped headline workload (B=16, 32k, 64/8 heads) at each swept k."""
    say("full-size c4 step, k =", k)
    sh = synth.preset("c4").replace(k=k, layers=1)
    x = synth.make(sh, device=DEV)
    _check(sh, x, k, sample=[0, sh.B - 1])


def test_c3_step_and_dense_baseline():
    """32B-shaped workload, with the dense full-KV baseline on the same inputs."""
    say("full-size c3 step + dense")
    sh = synth.preset("c3")
    x = synth.make(sh, device=DEV)
    kv = _check(sh, x, sh.k, sample=[5])
    lse = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    dense = dk.dustin_sparse_verify_attn(x.q, kv, None, None, lse=lse)
    torch.cuda.synchronize()
    for b in (0, 11):
        n = int(x.seq_lens[b])
        K, V = oracle_kv(x, "K", b), oracle_kv(x, "V", b)
        O = oracle.dense_attention(f64(x.q[b]), K, V)
        _, L = oracle.sparse_attention(f64(x.q[b]), K, V, np.arange(n))   # k = n: the dense LSE
        err = np.abs(f64(dense[b]) - O).max()
        lerr = np.abs(f64(lse[b]) - L).max()
        say(f"  dense b={b}: max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 2e-3


def test_c2_step():
    """7B-shaped workload, every sequence sampled."""
    say("full-size c2 step")
    sh = synth.preset("c2")
    x = synth.make(sh, device=DEV)
    _check(sh, x, sh.k, sample=list(range(sh.B)))


def test_c5_ragged_paged_step():
    """Ragged paged stress (B=8, n in [8192, 131072], 16-token pages, w=8, k=4096)."""
    say("full-size c5 step")
    sh = synth.preset("c5")
    x = synth.make(sh, device=DEV)
    lens = x.seq_lens.cpu().numpy()
    _check(sh, x, sh.k, sample=[int(np.argmin(lens)), int(np.argmax(lens))])


def test_c4_verify_step_with_window():
    """The headline shape with the window: score, select, then the causal
    verification attention that appends the window rows to the cache in the
    same launch (as the bench times it), on histories shortened by w so the
    window fits; sampled sequences against the oracle, and the appended rows
    checked in the cache."""
    say("full-size c4 verify step with the window")
    sh = synth.preset("c4").replace(layers=1)
    x = synth.make(sh, device=DEV)
    x.seq_lens.sub_(sh.w)
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    shp = (sh.B, sh.w, sh.Hkv, sh.d)
    k_win = torch.randn(shp, generator=g, device=DEV).to(x.K.dtype)
    v_win = torch.randn(shp, generator=g, device=DEV).to(x.K.dtype)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    sample = [3, sh.B - 2]
    hist = {b: (oracle_kv(x, "K", b), oracle_kv(x, "V", b)) for b in sample}
    n_sink, n_window, m = synth.tier_defaults(sh.k)
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
    s_d, s_t = dk.dustin_score(dkv, x.q_draft, [kv], x.q_hist, x.sub_heads, sh.Hq)
    idx, cnt, tier = dk.dustin_topk(s_d, s_t, x.seq_lens, sh.k, m, n_sink, n_window)
    lse = torch.empty((sh.B, sh.w, sh.Hq), dtype=torch.float32, device=DEV)
    out = dk.dustin_verify_attn_append(x.q, kv, k_win, v_win, idx, cnt, lse=lse)
    torch.cuda.synchronize()
    for b in sample:
        n = int(x.seq_lens[b])
        assert torch.equal(x.K[b, n:n + sh.w], k_win[b]) and torch.equal(x.V[b, n:n + sh.w], v_win[b])
        K, V = hist[b]
        n = int(x.seq_lens[b])
        c = int(cnt[b])
        assert int(idx[b, :c].max()) < n
        # the oracle's own scores, set and attention
        st = oracle.score_target(f64(x.q_hist[b]), {0: K}, x.sub_heads, sh.Hq)
        sd = oracle.score_draft(f64(x.q_draft[b]), oracle_kv(x, "Kd", b))
        oi, ot = oracle.select_verify_set(sd, st, n, sh.k, m, n_sink, n_window)
        nd = check_set_tieband(idx[b, :c].cpu().numpy(), tier[b, :c].cpu().numpy(), oi, ot, sd, st)
        O, L = oracle.verify_attention(f64(x.q[b]), K, V, f64(k_win[b]), f64(v_win[b]), oi)
        got_o, got_l = out[b], lse[b]
        if nd:   # near-tie differences: the GPU attends the oracle's set too
            oidx = torch.full((sh.B, sh.k), -1, dtype=torch.int32, device=DEV)
            ocnt = torch.zeros((sh.B,), dtype=torch.int32, device=DEV)
            oidx[b, :len(oi)] = torch.from_numpy(np.asarray(oi, dtype=np.int32)).to(DEV)
            ocnt[b] = len(oi)
            l2 = torch.empty_like(lse)
            got_o = dk.dustin_verify_attn(x.q, kv, oidx, ocnt, lse=l2)[b]
            got_l = l2[b]
            torch.cuda.synchronize()
        err, lerr = np.abs(f64(got_o) - O).max(), np.abs(f64(got_l) - L).max()
        say(f"  b={b} |I|={c} set diff {nd} (tie band) max|dO|={err:.2e} max|dlse|={lerr:.2e}")
        assert err <= 2e-2 and lerr <= 2e-3


def test_c4_policy_sweep():
    """The policy sweep on the 72B-shaped workload (B=16, 32k) with the
    look-back distances of Fig. 2 and the budgets of the k sweep; two sampled
    sequences against the oracle.  Scores: seeded synthetic [B][N_max]."""
    say("full-size c4 policy sweep")
    sh = synth.preset("c4").replace(layers=1, L_d=1)
    x = synth.make(sh, device=DEV)
    deltas, ks = [1, 4, 16, 64], [128, 512, 2048]
    qpast = synth.history_trajectory(x, deltas)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    sd = (torch.rand((sh.B, sh.n), generator=g, device=DEV) ** 4).contiguous()
    st = (torch.rand((sh.B, sh.n), generator=g, device=DEV) ** 4).contiguous()
    ms = [synth.tier_defaults(k)[2] for k in ks]
    arr = dk.dustin_policy_sweep(x.q, qpast, kv, sd, st, ks, ms, 4, 32).cpu().numpy()
    P = len(deltas)
    for b in (2, sh.B - 1):
        K = oracle_kv(x, "K", b)
        want = oracle.policy_sweep(f64(x.q[b]), f64(qpast[:, b]), K, f64(sd[b]), f64(st[b]), ks, ms, 4, 32)
        A = oracle.window_attention(f64(x.q[b]), K)
        e, t = check_sweep_rows(arr[:, :, b], want, A, f64(qpast[:, b]), K, ks)
        say(f"  b={b} k=2048: oracle {want[0, -1]:.4f} history {np.round(want[1:P + 1, -1], 4)}; "
            f"entries with one correct set {e}, with ties inside the 1e-5 band {t}")
