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

