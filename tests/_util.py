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
