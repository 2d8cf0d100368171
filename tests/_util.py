"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_idx(seq_lens, k, seed, frac_invalid=0.0, short=0, shuffle=True, device="cuda"):
    """Random distinct positions per sequence (count = min(k, n_b) - short),
    optionally with some invalid entries (-1 or >= n_b) mixed in."""
    rng = np.random.default_rng(seed)
    lens = seq_lens.cpu().numpy()
    B = len(lens)
    idx = np.full((B, k), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b, n in enumerate(lens):
        c = max(0, min(k, int(n)) - short)
        sel = rng.choice(int(n), c, replace=False) if c else np.zeros(0, np.int64)
        if not shuffle:
            sel = np.sort(sel)
        sel = sel.astype(np.int32)
        if frac_invalid > 0 and c > 0:
            bad = rng.random(c) < frac_invalid
            sel[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, int(n) + rng.integers(0, 1000, bad.sum()))
        idx[b, :c] = sel
        cnt[b] = c
    return torch.from_numpy(idx).to(device), torch.from_numpy(cnt).to(device)


def assert_scores_close(got, want, what="scores", rel=1e-5, abs_=1e-9):
    """Score parity bar: |got - want| <= rel * want + abs_ elementwise (fp32
    accumulation of bf16 products and an fp32 log-sum-exp against fp64)."""
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    excess = np.abs(got - want) - (rel * np.abs(want) + abs_)
    if excess.size and excess.max() > 0:
        j = int(np.argmax(excess))
        raise AssertionError(f"{what}: position {j} got {got[j]!r} want {want[j]!r} "
                             f"(|d| = {abs(got[j] - want[j]):.3e} > {rel:g} * want + {abs_:g}); "
                             f"{int((excess > 0).sum())} positions outside the bar")


def max_rel_err(got, want, floor=1e-6):
    """Largest |got - want| / want over positions with want >= floor (report only)."""
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    sel = want >= floor
    return float((np.abs(got - want)[sel] / want[sel]).max()) if sel.any() else 0.0


def tieband_range(rank, value, k, rel=1e-5):
    """Range of sum(value[I]) over every size-min(k, n) set I that a TopK of
    `rank` may return when ties within `rel` (relative) of the k-th largest
    rank may fall either way: the positions ranked strictly above the band
    are in every such set, the rest come from the band.  Returns (lo, hi,
    number of band positions beyond the ones needed)."""
    rank, value = np.asarray(rank, dtype=np.float64), np.asarray(value, dtype=np.float64)
    n = rank.size
    if k >= n:
        v = float(value.sum())
        return v, v, 0
    th = np.sort(rank)[::-1][k - 1]
    sure = rank > th + rel * abs(th)
    band = np.abs(rank - th) <= rel * abs(th)
    need = k - int(sure.sum())
    bv = np.sort(value[band])
    base = float(value[sure].sum())
    return base + float(bv[:need].sum()), base + float(bv[::-1][:need].sum()), int(band.sum()) - need


def check_sweep_rows(got, want, A, q_past, K, ks, tol=1e-4):
    """Policy-sweep rows (oracle.policy_sweep's layout) of one sequence:
    rows ranked by score vectors both sides share must match the oracle within
    tol; the SD-oracle and history rows, ranked by attention each side computes
    itself, must lie within tol of the windowed-ARR range of the sets that the
    1e-5 tie band allows.  got, want [P + 5][len(ks)]; A the oracle's window
    attention (Eq. 1), q_past [P][Hq][d].  Returns (entries checked against
    the oracle's value, entries checked against a tie-band range)."""
    P = q_past.shape[0]
    Abar = A.mean(axis=0)
    rank = [Abar] + [oracle.window_attention(q_past[p][None], K)[0] for p in range(P)]
    exact = banded = 0
    for row in range(P + 5):
        for ki, k in enumerate(ks):
            v = got[row, ki]
            assert 0.0 <= v <= 1.0 + 1e-5
            lo = hi = want[row, ki]
            spare = 0
            if row <= P:        # ranked by attention each side computes itself
                lo, hi, spare = tieband_range(rank[row], Abar, k)
                assert lo - 1e-12 <= want[row, ki] <= hi + 1e-12
            if spare:
                banded += 1
            else:
                exact += 1
            assert lo - tol <= v <= hi + tol, (row, k, v, want[row, ki], lo, hi)
    return exact, banded


def valid_set(idx_row, cnt, n):
    s = idx_row[:cnt]
    return s[(s >= 0) & (s < n)]


def check_set_tieband(gi, gt, oi, ot, sd, st, rel=1e-5):
    """End-to-end index-set parity: the GPU set equals the oracle set except
    for positions whose oracle score lies within `rel` (relative) of the
    oracle's threshold in the draft or target tier."""
    gi, oi = np.asarray(gi), np.asarray(oi)
    assert len(gi) == len(oi), f"set sizes differ: {len(gi)} vs {len(oi)}"
    assert set(gi[np.asarray(gt) == 0]) == set(oi[np.asarray(ot) == 0]), "protected tier differs"
    diff = set(gi) ^ set(oi)
    if not diff:
        return 0
    od = oi[np.asarray(ot) == 1]
    otg = oi[np.asarray(ot) == 2]
    th_d = sd[od].min() if (sd is not None and len(od)) else None
    th_t = st[otg].min() if (st is not None and len(otg)) else None
    for j in diff:
        ok = False
        if th_d is not None and abs(sd[j] - th_d) <= rel * th_d:
            ok = True
        if th_t is not None and abs(st[j] - th_t) <= rel * th_t:
            ok = True
        assert ok, f"position {j} differs outside the tie band (sd={None if sd is None else sd[j]}, " \
                   f"st={None if st is None else st[j]}, th_d={th_d}, th_t={th_t})"
    return len(diff)


def oracle_kv(x, name, b):
    return f64(x.logical(name, b))


def check_tier_rule(idx_row, tier_row, cnt, sd, st, n, k, m, n_sink, n_window):
    """Invariants of the verification set (blog section 2.3) on any size,
    checked directly (not through the oracle): the count, ascending unique
    positions below n, the protected tier exactly the sinks and the recent
    window, the draft tier of size min(m, k - |P|, n - |P|) holding the top
    S_Draft keys (score, then lower position) outside P, and the target tier
    holding the top S_Target keys of the rest."""
    idx_row, tier_row = np.asarray(idx_row[:cnt]), np.asarray(tier_row[:cnt])
    assert cnt == min(k, n)
    assert (np.diff(idx_row) > 0).all() and (idx_row.size == 0 or (idx_row[0] >= 0 and idx_row[-1] < n))
    P = set(range(min(n_sink, n))) | set(range(max(0, n - n_window), n))
    got_p = set(idx_row[tier_row == 0].tolist())
    assert got_p == P, "protected tier"
    D = idx_row[tier_row == 1]
    T = idx_row[tier_row == 2]
    rest = np.setdiff1d(np.arange(n), np.array(sorted(P), dtype=np.int64))
    budget = k - len(P)
    m_eff = 0 if sd is None else (budget if st is None else m)
    m_eff = max(0, min(m_eff, budget, rest.size))
    assert D.size == m_eff, "draft tier size"
    assert T.size == max(0, min(budget - m_eff, rest.size - m_eff)), "target tier size"

    def top_by(score, chosen, pool):
        """Every chosen position outranks every unchosen one of the pool."""
        if chosen.size == 0 or chosen.size == pool.size:
            return
        others = np.setdiff1d(pool, chosen)
        worst = min(chosen.tolist(), key=lambda j: (score[j], -j))
        best = max(others.tolist(), key=lambda j: (score[j], -j))
        assert (score[worst], -worst) > (score[best], -best), "tier is not the top of its pool"

    if D.size:
        top_by(sd, D, rest)
    if T.size:
        top_by(st, T, np.setdiff1d(rest, D))

