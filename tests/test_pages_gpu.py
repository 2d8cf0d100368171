"""GPU parity of the page-level estimator the pages compare Dustin's scoring
with (Quest in the translation's related work; Quest-16 in the blog's Fig. 8):
per-page min/max key bounds and the page scores computed from them, against
the oracle's page_key_bounds / page_scores on the same seeded inputs.

Bounds are min/max of stored values: bit-exact.  Scores are float32 sums of
products of stored values, grouped differently from the float64 oracle; each
page's error is held to 1e-5 of M_p = scale * sum_{s,h,d} |q| max(|kmin|, |kmax|),
which bounds the magnitude of every term in either grouping (float32 rounding
of a few dozen sequential additions per term stays well inside it).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_kv_verification_amd as dk
from _util import f64, oracle_kv, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    ("c4-shape", dict(base="c4", B=2, n=3000)),                          # Hq 64, Hkv 8, d 128, bf16
    ("ragged", dict(base="c2", B=4, n=2500, n_lo=700)),                  # ragged page tails
    ("paged", dict(base="c5", B=3, n=2600, n_lo=1000)),                  # the cache's own pages
    ("d64", dict(base="c4", B=2, n=2003, Hq=8, Hkv=2, d=64)),
    ("d32", dict(base="c4", B=2, n=1500, Hq=16, Hkv=4, d=32, w=2)),
    ("tiny-f32", dict(base="c1")),
]


def _run(name, over, zero_first=False):
    over = dict(over)
    sh = synth.preset(over.pop("base")).replace(**over)
    x = synth.make(sh, device=DEV)
    if zero_first:
        x.seq_lens[0] = 0
    kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
    kmin, kmax = dk.dustin_page_bounds(kv)
    sc = dk.dustin_page_scores(x.q, kv, kmin, kmax)
    sc2 = dk.dustin_page_scores(x.q, kv, kmin, kmax)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc2), "not deterministic"
    npg = (kv.desc.N_max + 15) // 16
    assert kmin.shape == (sh.B, npg, sh.Hkv, sh.d) and sc.shape == (sh.B, npg)
    lens = x.seq_lens.cpu().numpy()
    for b in range(sh.B):
        n = int(lens[b])
        used = -(-n // 16)
        gmin, gmax, gsc = f64(kmin[b]), f64(kmax[b]), f64(sc[b])
        # pages past the sequence hold zeros
        assert not gmin[used:].any() and not gmax[used:].any() and not gsc[used:].any()
        if n == 0:
            continue
        K = oracle_kv(x, "K", b)
        omin, omax = oracle.page_key_bounds(K, n)
        np.testing.assert_array_equal(gmin[:used], omin)
        np.testing.assert_array_equal(gmax[:used], omax)
        q = f64(x.q[b])
        want = oracle.page_scores(q, omin, omax)
        G = sh.Hq // sh.Hkv
        qabs = np.abs(q).reshape(q.shape[0], sh.Hkv, G, sh.d).sum(axis=(0, 2))        # [Hkv][d]
        mag = (qabs[None] * np.maximum(np.abs(omin), np.abs(omax))).sum(axis=(1, 2)) / np.sqrt(sh.d)
        err = np.abs(gsc[:used] - want)
        say(f"  b={b} n={n} pages={used} max|score|={np.abs(want).max():.4g} max err/M={np.max(err / mag):.3g}")
        assert np.all(err <= 1e-5 * mag + 1e-30), (b, np.argmax(err / mag))


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_page_estimator_matches_oracle(name, over):
    say("page estimator", name)
    _run(name, over)


def test_page_estimator_empty_sequence():
    say("page estimator empty sequence")
    _run("empty", dict(base="c2", B=3, n=1000, n_lo=300), zero_first=True)
