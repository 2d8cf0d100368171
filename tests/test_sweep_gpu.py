"""GPU parity of the policy sweep (translation sections 3.2-3.3, Figs. 2-3;
blog Table 3): windowed ARR of the SD oracle, the history policy at several
look-back distances, the draft lookahead and the Dustin-T/D/H sets, against
the oracle's policy_sweep on the same seeded inputs.

S_Draft / S_Target are seeded synthetic scores (rounded to float32, the
precision the GPU selects in), so both sides select those rows from identical
values and must agree within the ARR bar, 1e-4.  The oracle and history rows
rank positions by attention each side computes itself (float32 vs float64):
the index-set rule lets positions whose rank score lies within 1e-5 (relative)
of the k-th score fall either way, so those entries must lie within 1e-4 of
the range of windowed ARRs that such sets reach (computed exactly from the
oracle's values); every other entry within 1e-4 of the oracle's value.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import check_sweep_rows, f64, oracle_kv, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _scores(sh, x, kv, seed):
    """[B][N_max] score vectors (N_max of the cache descriptor: a paged cache
    rounds it up to whole pages), zero at positions >= n_b."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    lens = x.seq_lens.cpu().numpy()
    N = kv.desc.N_max
    sd = torch.rand((sh.B, N), generator=g, device=DEV) ** 4     # skewed, like attention mass
    st = torch.rand((sh.B, N), generator=g, device=DEV) ** 4
    for b in range(sh.B):
        sd[b, int(lens[b]):] = 0
        st[b, int(lens[b]):] = 0
    return sd.contiguous(), st.contiguous()


def _check(sh, x, deltas, ks, sample, n_sink=4, n_window=32):
    qpast = synth.history_trajectory(x, deltas)
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    sd, st = _scores(sh, x, kv, 7)
    ms = [synth.tier_defaults(k)[2] for k in ks]
    arr = dk.dustin_policy_sweep(x.q, qpast, kv, sd, st, ks, ms, n_sink, n_window)
    arr2 = dk.dustin_policy_sweep(x.q, qpast, kv, sd, st, ks, ms, n_sink, n_window)
    torch.cuda.synchronize()
    assert torch.equal(arr, arr2), "not deterministic"
    g = arr.cpu().numpy().astype(np.float64)          # [P + 5][nk][B]
    P = len(deltas)
    exact = banded = 0
    for b in sample:
        n = int(x.seq_lens[b])
        K = oracle_kv(x, "K", b)
        sdb, stb = f64(sd[b, :n]), f64(st[b, :n])
        want = oracle.policy_sweep(f64(x.q[b]), f64(qpast[:, b]), K, sdb, stb, ks, ms, n_sink, n_window)
        A = oracle.window_attention(f64(x.q[b]), K)
        e, t = check_sweep_rows(g[:, :, b], want, A, f64(qpast[:, b]), K, ks)
        exact, banded = exact + e, banded + t
        say(f"  b={b} n={n} oracle {np.round(want[0], 4)} hist {np.round(want[1:P + 1, -1], 4)} "
            f"draft {want[P + 1, -1]:.4f} T/D/H {np.round(want[P + 2:, -1], 4)} (k={ks[-1]})")
    say(f"  entries with one correct set {exact}, with ties inside the 1e-5 band {banded}")
    return g


@pytest.mark.parametrize("name,over", [
    ("qwen72b", dict(base="c4", B=2, n=3000, L_d=1)),
    ("qwen7b-ragged", dict(base="c2", B=3, n=2500, n_lo=900, L_d=1)),
    ("paged", dict(base="c5", B=2, n=2600, n_lo=1000, L_d=1)),
    ("d64", dict(base="c4", B=2, n=2000, Hq=8, Hkv=2, d=64, L_d=1)),
])
def test_policy_sweep_matches_oracle(name, over):
    say("policy sweep", name)
    over = dict(over)
    sh = synth.preset(over.pop("base")).replace(**over)
    x = synth.make(sh, device=DEV)
    _check(sh, x, [1, 4, 16], [64, 256, 1024], sample=list(range(sh.B)))


def test_policy_sweep_tiny_f32():
    say("policy sweep tiny-f32")
    sh = synth.preset("c1")
    x = synth.make(sh, device=DEV)
    _check(sh, x, [1, 2, 8], [16, 64, 128, 1024], sample=[0], n_sink=2, n_window=6)


def test_window_mean_matches_definition():
    say("window mean")
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    A = torch.rand((3, 5, 777), generator=g, device=DEV)
    Abar = dk.dustin_window_mean(A)
    torch.cuda.synchronize()
    want = np.stack([oracle.sd_oracle(f64(A[b]), 1)[2] for b in range(A.shape[0])])   # Abar of Eq. (3)
    np.testing.assert_allclose(f64(Abar), want, rtol=1e-6, atol=1e-9)
