"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties an oracle function to a closed form, an invariant the pages
state, a library routine for a special case, or brute force on tiny inputs,
chosen so that a dropped term, a wrong sign or index, a transposed operand or
a wrong head mapping fails at least one of them.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _frac(s):
    return float(Fraction(s))


def _lnfrac(s):
    return math.log(float(Fraction(s.split("ln", 1)[1].strip().replace(" ", ""))))


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Hand-derived worked examples (translation section 3.1, Eq. 1-4)
# --------------------------------------------------------------------------

def _worked_inputs():
    g = _load("worked_example_arr.json")
    K = np.array([[[math.log(j + 1), 0.0]] for j in range(4)])  # [4][1][2]
    q = np.array(g["inputs"]["q"], dtype=np.float64)            # [w=2][Hq=2][2]
    V = np.array(g["inputs"]["V"], dtype=np.float64)            # [4][1][2]
    return g, q, K, V


def test_worked_example_window_attention():
    g, q, K, V = _worked_inputs()
    A = oracle.window_attention(q, K, scale=1.0)
    exp = np.array([[_frac(x) for x in row] for row in g["expected"]["A"]])
    np.testing.assert_allclose(A, exp, rtol=0, atol=1e-14)


def test_worked_example_arr_and_sd_oracle():
    g, q, K, V = _worked_inputs()
    A = oracle.window_attention(q, K, scale=1.0)
    ex = g["expected"]
    set_a = g["inputs"]["set_a"]
    np.testing.assert_allclose(oracle.arr_step(A, set_a), [_frac(x) for x in ex["arr_step_set_a"]], atol=1e-14)
    assert abs(oracle.arr_window(A, set_a) - _frac(ex["arr_window_set_a"])) < 1e-14
    sel, arr, Abar = oracle.sd_oracle(A, g["inputs"]["k"])
    np.testing.assert_allclose(Abar, [_frac(x) for x in ex["Abar"]], atol=1e-14)
    assert sel.tolist() == ex["orc_set"]
    assert abs(arr - _frac(ex["orc_arr"])) < 1e-14


def test_worked_example_dense_and_sparse_outputs():
    g, q, K, V = _worked_inputs()
    ex = g["expected"]
    O = oracle.dense_attention(q, K, V, scale=1.0)
    exp = np.array([[[_frac(x) for x in h] for h in s] for s in ex["dense_out"]])
    np.testing.assert_allclose(O, exp, atol=1e-14)
    Os, lse = oracle.sparse_attention(q, K, V, g["inputs"]["set_sparse"], scale=1.0)
    exp = np.array([[[_frac(x) for x in h] for h in s] for s in ex["sparse_out"]])
    np.testing.assert_allclose(Os, exp, atol=1e-14)
    exp_lse = np.array([[_lnfrac(x) for x in s] for s in ex["sparse_lse"]])
    np.testing.assert_allclose(lse, exp_lse, atol=1e-14)


def test_worked_example_tiers():
    g = _load("worked_example_tiers.json")
    for c in g["cases"]:
        idx, tier = oracle.select_verify_set(np.array(g["s_draft"], float), np.array(g["s_target"], float),
                                             g["n"], c["k"], c["m"], g["n_sink"], g["n_window"])
        assert idx.tolist() == c["idx"], c["why"]
        assert tier.tolist() == c["tier"], c["why"]


# --------------------------------------------------------------------------
# Library routines for special cases
# --------------------------------------------------------------------------

def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(3, 17)) * 5
    np.testing.assert_allclose(oracle.softmax(x), scipy.special.softmax(x, axis=-1), rtol=1e-13, atol=0)


@pytest.mark.parametrize("w,Hq,Hkv,d,n", [(4, 8, 2, 16, 37), (1, 1, 1, 8, 5), (3, 6, 3, 32, 64)])
def test_dense_attention_matches_torch_sdpa(w, Hq, Hkv, d, n):
    rng = np.random.default_rng(w * 100 + n)
    q = rng.normal(size=(w, Hq, d))
    K = rng.normal(size=(n, Hkv, d)) * 2
    V = rng.normal(size=(n, Hkv, d))
    O = oracle.dense_attention(q, K, V)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1][Hq][w][d]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_attention_matches_masked_sdpa_and_logsumexp():
    rng = np.random.default_rng(7)
    w, Hq, Hkv, d, n = 4, 8, 2, 16, 50
    q = rng.normal(size=(w, Hq, d))
    K = rng.normal(size=(n, Hkv, d)) * 2
    V = rng.normal(size=(n, Hkv, d))
    I = np.sort(rng.choice(n, 13, replace=False))
    O, lse = oracle.sparse_attention(q, K, V, np.concatenate([I, [-1, -1]]))
    mask = torch.zeros(n, dtype=torch.bool)
    mask[torch.from_numpy(I)] = True
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None, None, :], enable_gqa=True)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        logits = q[:, h, :] @ K[I, g, :].T / math.sqrt(d)
        np.testing.assert_allclose(lse[:, h], scipy.special.logsumexp(logits, axis=1), rtol=1e-13)


def test_sparse_equals_dense_when_set_is_everything():
    # k >= |V_i|: sparse attention over all rows equals full attention.
    rng = np.random.default_rng(3)
    q = rng.normal(size=(4, 8, 16))
    K = rng.normal(size=(40, 2, 16))
    V = rng.normal(size=(40, 2, 16))
    O, _ = oracle.sparse_attention(q, K, V, np.arange(40))
    np.testing.assert_allclose(O, oracle.dense_attention(q, K, V), rtol=1e-13, atol=1e-13)


def test_single_query_two_token_closed_form():
    # G = 1, w = 1: o = (e^a v0 + e^b v1) / (e^a + e^b) with a, b the scaled logits.
    q = np.array([[[1.0, 2.0, 0.0, 0.0]]])
    K = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]])
    V = np.array([[[1.0, 0.0, 3.0, 0.0]], [[0.0, 1.0, 0.0, -2.0]]])
    a, b = 1.0 / 2.0, 2.0 / 2.0       # scale 1/sqrt(4)
    pa = math.exp(a) / (math.exp(a) + math.exp(b))
    expect = pa * V[0, 0] + (1 - pa) * V[1, 0]
    np.testing.assert_allclose(oracle.dense_attention(q, K, V)[0, 0], expect, rtol=1e-14)


# --------------------------------------------------------------------------
# ARR invariants the pages state
# --------------------------------------------------------------------------

def _rand_A(rng, w=4, n=30, Hq=4, Hkv=2, d=8):
    q = rng.normal(size=(w, Hq, d)) * 1.5
    K = rng.normal(size=(n, Hkv, d)) * 1.5
    return oracle.window_attention(q, K)


def test_arr_of_full_history_is_one():
    # Translation section 3.1: sum_j A_{i,j} = 1 over V_i, so ARR(V_i) = 1.
    A = _rand_A(np.random.default_rng(1))
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.arr_step(A, np.arange(A.shape[1])), 1.0, rtol=1e-14)
    assert abs(oracle.arr_window(A, np.arange(A.shape[1])) - 1.0) < 1e-14


def test_orc_arr_is_sum_of_topk_via_partition():
    # Eq. (4) = Eq. (2) evaluated on Eq. (3)'s set; by linearity it is the sum
    # of the k largest entries of Abar.  np.partition is an independent route.
    rng = np.random.default_rng(2)
    A = _rand_A(rng, n=200)
    Abar = A.mean(axis=0)
    for k in (1, 5, 17, 100, 200):
        _, arr, _ = oracle.sd_oracle(A, k)
        top = np.partition(Abar, Abar.size - k)[Abar.size - k:]
        assert abs(arr - top.sum()) < 1e-13
        sel, _, _ = oracle.sd_oracle(A, k)
        assert abs(oracle.arr_window(A, sel) - arr) < 1e-13


def test_orc_is_upper_bound_brute_force():
    # Translation section 3.1: the SD oracle is an upper bound of windowed ARR
    # over every policy with budget k.  Brute force over all subsets, n = 12.
    rng = np.random.default_rng(4)
    A = _rand_A(rng, n=12)
    for k in (1, 3, 6):
        sel, arr, _ = oracle.sd_oracle(A, k)
        best = max(oracle.arr_window(A, list(c)) for c in itertools.combinations(range(12), k))
        assert abs(best - arr) < 1e-13
        for _ in range(50):
            other = rng.choice(12, k, replace=False)
            assert oracle.arr_window(A, other) <= arr + 1e-15


def test_arr_monotone_in_k():
    rng = np.random.default_rng(5)
    A = _rand_A(rng, n=300)
    prev = -1.0
    for k in range(1, 301, 7):
        _, arr, _ = oracle.sd_oracle(A, k)
        assert arr >= prev - 1e-15
        prev = arr


# --------------------------------------------------------------------------
# TopK and the tier rule
# --------------------------------------------------------------------------

def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(6)
    for trial in range(200):
        n = int(rng.integers(1, 14))
        s = rng.integers(0, 4, size=n).astype(float)      # many ties
        k = int(rng.integers(0, n + 2))
        got = oracle.topk_desc(s, k).tolist()
        # pure-Python reference: sort positions by (-score, position)
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        assert got == ref


def _best_subset(scores, cands, r):
    """Brute force: max-sum r-subset of cands, lowest positions among ties."""
    best, best_key = None, None
    for c in itertools.combinations(sorted(cands), r):
        key = (-sum(scores[j] for j in c), c)
        if best_key is None or key < best_key:
            best, best_key = set(c), key
    return best if best is not None else set()


def test_tiers_brute_force():
    rng = np.random.default_rng(8)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        sd = rng.integers(0, 5, size=n).astype(float)
        st = rng.integers(0, 5, size=n).astype(float)
        n_sink = int(rng.integers(0, 3))
        n_window = int(rng.integers(0, 3))
        k = int(rng.integers(n_sink + n_window, n_sink + n_window + 8))
        if k == 0:
            continue
        m = int(rng.integers(0, k + 2))
        idx, tier = oracle.select_verify_set(sd, st, n, k, m, n_sink, n_window)
        P = set(range(min(n_sink, n))) | set(range(max(0, n - n_window), n))
        rest = set(range(n)) - P
        m_eff = max(0, min(m, k - len(P), len(rest)))
        D = _best_subset(sd, rest, m_eff)
        T = _best_subset(st, rest - D, max(0, min(k - len(P) - m_eff, len(rest - D))))
        assert set(idx.tolist()) == P | D | T
        assert idx.tolist() == sorted(idx.tolist())
        assert len(idx) == min(k, n) == len(set(idx.tolist()))
        lab = dict(zip(idx.tolist(), tier.tolist()))
        assert all(lab[j] == 0 for j in P)
        assert all(lab[j] == 1 for j in D)
        assert all(lab[j] == 2 for j in T)


def test_tier_special_cases():
    rng = np.random.default_rng(9)
    n = 64
    sd = rng.random(n)
    st = rng.random(n)
    # m = 0, no protection: TopK_k of S_Target (Dustin-T in the blog's ablation)
    idx, _ = oracle.select_verify_set(sd, st, n, 10, 0, 0, 0)
    assert idx.tolist() == sorted(np.argsort(-st)[:10].tolist())
    # m = k, no protection: TopK_k of S_Draft (Dustin-D)
    idx, _ = oracle.select_verify_set(sd, st, n, 10, 10, 0, 0)
    assert idx.tolist() == sorted(np.argsort(-sd)[:10].tolist())
    # missing draft scores behave like m = 0; missing target scores like m = k
    assert oracle.select_verify_set(None, st, n, 10, 5, 0, 0)[0].tolist() == sorted(np.argsort(-st)[:10].tolist())
    assert oracle.select_verify_set(sd, None, n, 10, 5, 0, 0)[0].tolist() == sorted(np.argsort(-sd)[:10].tolist())
    # k >= n returns all positions; protected tokens always included
    assert oracle.select_verify_set(sd, st, n, 100, 7, 4, 8)[0].tolist() == list(range(n))
    idx, _ = oracle.select_verify_set(sd, st, n, 20, 7, 4, 8)
    assert set(range(4)) | set(range(56, 64)) <= set(idx.tolist())
    # protected window larger than the sequence
    assert oracle.protected_positions(5, 4, 8).tolist() == [0, 1, 2, 3, 4]
    with pytest.raises(ValueError):
        oracle.select_verify_set(sd, st, n, 5, 0, 4, 8)


# --------------------------------------------------------------------------
# Scoring: S_Target and S_Draft
# --------------------------------------------------------------------------

def test_scores_uniform_when_keys_identical():
    # Identical keys give a uniform softmax: S_T = S / n, S_D = L_d H_d Gamma / n.
    rng = np.random.default_rng(10)
    n, Hq, Hkv, d = 33, 8, 2, 16
    K = np.broadcast_to(rng.normal(size=(1, Hkv, d)), (n, Hkv, d))
    sub = [(0, 0), (0, 3), (0, 5)]
    qh = rng.normal(size=(3, d))
    np.testing.assert_allclose(oracle.score_target(qh, {0: K}, sub, Hq), 3.0 / n, rtol=1e-13)
    L_d, G_, H_d, Hkv_d, d_d = 2, 3, 4, 2, 8
    Kd = np.broadcast_to(rng.normal(size=(L_d, 1, Hkv_d, d_d)), (L_d, n, Hkv_d, d_d))
    qd = rng.normal(size=(L_d, G_, H_d, d_d))
    np.testing.assert_allclose(oracle.score_draft(qd, Kd), L_d * H_d * G_ / n, rtol=1e-13)


def test_score_sums_count_every_term():
    rng = np.random.default_rng(11)
    n, Hq, Hkv, d = 70, 8, 4, 16
    Ks = {0: rng.normal(size=(n, Hkv, d)), 2: rng.normal(size=(n, Hkv, d))}
    sub = [(0, 1), (2, 6), (2, 7), (0, 0)]
    st = oracle.score_target(rng.normal(size=(4, d)) * 3, Ks, sub, Hq)
    assert abs(st.sum() - 4.0) < 1e-12 and (st > 0).all()
    L_d, G_, H_d, Hkv_d, d_d = 3, 4, 6, 2, 8
    sd = oracle.score_draft(rng.normal(size=(L_d, G_, H_d, d_d)) * 3, rng.normal(size=(L_d, n, Hkv_d, d_d)))
    assert abs(sd.sum() - L_d * H_d * G_) < 1e-11 and (sd > 0).all()


def test_score_head_to_kv_mapping_and_scale():
    # KV head 0 holds identical keys (uniform softmax); KV head 1 holds one key
    # aligned with the query strongly enough that its softmax is one-hot at p.
    n, Hq, Hkv, d, p = 16, 8, 2, 4, 11
    K = np.zeros((n, Hkv, d))
    K[:, 0, :] = 0.5
    K[p, 1, 0] = 200.0
    qh = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0]])
    # head 4 -> kv 1 (4 // 4); head 1 -> kv 0.  A modulo mapping would swap them.
    st = oracle.score_target(qh, {0: K}, [(0, 4), (0, 1)], Hq)
    expect = np.full(n, 1.0 / n)
    expect[p] += 1.0
    np.testing.assert_allclose(st, expect, rtol=0, atol=1e-14)
    # S_Target's scale 1/sqrt(d): two keys with raw logits 3 and 1 at d = 4
    # give p0 = sigmoid((3 - 1) / 2) for a scored head.  Pair (2, 6) is head 6
    # of layer 2, in KV group 1 (6 // 4; a modulo map gives group 0, whose
    # keys differ); pair (0, 0) reads layer 0's group 0, whose two keys are
    # equal (uniform 1/2).  Layer 0's group 1 holds yet other keys, so reading
    # the wrong layer for either pair moves the result as well.
    K0 = np.zeros((2, Hkv, d))
    K0[0, 1, 0] = 5.0
    K2 = np.zeros((2, Hkv, d))
    K2[:, 1, 0] = [3.0, 1.0]
    K2[1, 0, 0] = 9.0
    qh = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0]])
    st = oracle.score_target(qh, {0: K0, 2: K2}, [(0, 0), (2, 6)], Hq)
    p0 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(st, [0.5 + p0, 0.5 + 1 - p0], rtol=1e-14)
    # scale 1/sqrt(d_d): two keys with raw logits 2 and 0 -> p0 = sigmoid(2/2)
    qd = np.zeros((1, 1, 4, 4))
    qd[0, 0, :, 0] = 2.0
    Kd = np.zeros((1, 2, 2, 4))
    Kd[0, 0, :, 0] = 1.0
    sd = oracle.score_draft(qd, Kd)
    p0 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(sd, [4 * p0, 4 * (1 - p0)], rtol=1e-14)
    # draft head 1 -> draft kv 0 with G_d = 2 (a modulo mapping gives kv 1)
    qd = np.zeros((1, 1, 4, 4))
    qd[0, 0, 1, 0] = 1.0
    Kd = np.zeros((1, 3, 2, 4))
    Kd[0, 2, 0, 0] = 400.0         # kv 0: one-hot at position 2 for head 1
    sd = oracle.score_draft(qd, Kd)
    # heads 0, 2, 3 have zero queries -> uniform 1/3 each; head 1 -> one-hot
    np.testing.assert_allclose(sd, np.array([1, 1, 1]) + np.array([0, 0, 1.0]), atol=1e-14)


def test_draft_row_lse_closed_forms():
    # All-zero keys: every logit is 0, so lse = ln n for every (layer, step, head).
    n = 37
    qd = np.random.default_rng(13).normal(size=(2, 3, 4, 8))
    np.testing.assert_allclose(oracle.draft_row_lse(qd, np.zeros((2, n, 2, 8))), math.log(n), rtol=1e-14)
    # One key per (layer, KV head) with raw logit x, n - 1 zero logits:
    # lse = ln(exp(x * scale) + n - 1), scale 1/sqrt(d_d) = 1/2 at d_d = 4.
    # Draft heads 0, 1 read KV head 0 and heads 2, 3 KV head 1 (G_d = 2); the
    # two layers hold their keys at different strengths.
    n = 5
    qd = np.zeros((2, 1, 4, 4))
    qd[:, 0, :, 0] = 1.0
    Kd = np.zeros((2, n, 2, 4))
    Kd[0, 3, 0, 0] = 6.0      # layer 0, KV head 0: x = 6  -> scaled 3
    Kd[0, 1, 1, 0] = 2.0      # layer 0, KV head 1: x = 2  -> scaled 1
    Kd[1, 0, 1, 0] = 8.0      # layer 1, KV head 1: x = 8  -> scaled 4; KV head 0 all zero
    lse = oracle.draft_row_lse(qd, Kd)
    e = lambda x: math.log(math.exp(x) + n - 1)
    np.testing.assert_allclose(lse[0, 0], [e(3), e(3), e(1), e(1)], rtol=1e-14)
    np.testing.assert_allclose(lse[1, 0], [math.log(n), math.log(n), e(4), e(4)], rtol=1e-14)
    # empty history: -inf
    assert np.isneginf(oracle.draft_row_lse(qd, np.zeros((2, 0, 2, 4)))).all()


def test_score_draft_given_lse():
    # With lse = ln n on all-zero keys every row contributes 1/n per position.
    n = 9
    qd = np.random.default_rng(14).normal(size=(2, 3, 4, 8))
    Kz = np.zeros((2, n, 2, 8))
    np.testing.assert_allclose(oracle.score_draft_given_lse(qd, Kz, np.full((2, 3, 4), math.log(n))),
                               2 * 3 * 4 / n, rtol=1e-14)
    # Each row's terms scale by exp(-delta) when its normaliser grows by delta:
    # raising one row's lse by ln 2 removes half of that row's mass (1/2 in total).
    rng = np.random.default_rng(15)
    qd = rng.normal(size=(2, 2, 4, 8))
    Kd = rng.normal(size=(2, 23, 2, 8))
    lse = oracle.draft_row_lse(qd, Kd)
    full = oracle.score_draft_given_lse(qd, Kd, lse)
    assert abs(full.sum() - 2 * 2 * 4) < 1e-12
    lse2 = lse.copy()
    lse2[1, 0, 3] += math.log(2.0)
    assert abs(oracle.score_draft_given_lse(qd, Kd, lse2).sum() - (2 * 2 * 4 - 0.5)) < 1e-12


# --------------------------------------------------------------------------
# Paged layout
# --------------------------------------------------------------------------

def test_pages_identity_and_permuted():
    rng = np.random.default_rng(12)
    n, ps = 45, 16
    logical = rng.normal(size=(48, 3, 4))
    pool = logical.reshape(3, ps, 3, 4)
    np.testing.assert_array_equal(oracle.pages_to_contiguous(pool, [0, 1, 2], n, ps), logical[:n])
    perm = np.array([2, 0, 1])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    np.testing.assert_array_equal(oracle.pages_to_contiguous(pool2, perm, n, ps), logical[:n])


# ---------------------------------------------------------------- verification window (blog Fig. 5, Stage 2)
def _window_case(seed, w=4, Hq=8, Hkv=2, d=16, n=30):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(w, Hq, d)), rng.normal(size=(n, Hkv, d)) * 1.5, rng.normal(size=(n, Hkv, d)),
            rng.normal(size=(w, Hkv, d)) * 1.5, rng.normal(size=(w, Hkv, d)))


def test_verify_attention_matches_causally_masked_sdpa():
    # history set I plus the window: query s sees I and window tokens 0..s
    q, K, V, Kw, Vw = _window_case(11)
    w, n = q.shape[0], K.shape[0]
    I = np.sort(np.random.default_rng(5).choice(n, 9, replace=False))
    O, lse = oracle.verify_attention(q, K, V, Kw, Vw, np.concatenate([I, [-1]]))
    Kc, Vc = np.concatenate([K, Kw]), np.concatenate([V, Vw])
    mask = torch.zeros(w, n + w, dtype=torch.bool)
    mask[:, torch.from_numpy(I)] = True
    for s in range(w):
        mask[s, n:n + s + 1] = True
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(Kc).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(Vc).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None], enable_gqa=True)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    Hq, Hkv, d = q.shape[1], K.shape[1], q.shape[2]
    for s in range(w):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = np.concatenate([K[I, g], Kw[:s + 1, g]])
            np.testing.assert_allclose(lse[s, h], scipy.special.logsumexp(keys @ q[s, h] / math.sqrt(d)), rtol=1e-13)


def test_verify_attention_without_history_is_causal_self_attention():
    q, K, V, Kw, Vw = _window_case(12)
    O, _ = oracle.verify_attention(q, K, V, Kw, Vw, [])
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(Kw).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(Vw).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_verify_attention_uniform_keys_average_the_visible_values():
    # identical keys -> uniform softmax: step s averages |I| + s + 1 value rows
    w, Hq, Hkv, d, n = 4, 4, 1, 8, 12
    rng = np.random.default_rng(13)
    key = rng.normal(size=d)
    K = np.tile(key, (n, Hkv, 1))
    Kw = np.tile(key, (w, Hkv, 1))
    V = rng.normal(size=(n, Hkv, d))
    Vw = rng.normal(size=(w, Hkv, d))
    q = rng.normal(size=(w, Hq, d))
    I = np.array([0, 3, 7])
    O, lse = oracle.verify_attention(q, K, V, Kw, Vw, I)
    for s in range(w):
        expect = np.concatenate([V[I, 0], Vw[:s + 1, 0]]).mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(O[s, h], expect, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[s, h], key @ q[s, h] / math.sqrt(d) + math.log(len(I) + s + 1), rtol=1e-12)


def test_single_step_window_is_sparse_attention_over_appended_row():
    # w = 1: the draft token sees I plus itself, i.e. the set I u {n} of the
    # cache after the window row is appended at position n
    q, K, V, Kw, Vw = _window_case(14, w=1)
    n = K.shape[0]
    I = np.array([2, 5, 9, 20])
    O, lse = oracle.verify_attention(q, K, V, Kw, Vw, I)
    Ka, Va = oracle.append_window_kv(np.concatenate([K, np.zeros((1,) + K.shape[1:])]),
                                     np.concatenate([V, np.zeros((1,) + V.shape[1:])]), n, Kw, Vw)
    O2, lse2 = oracle.sparse_attention(q, Ka, Va, np.concatenate([I, [n]]))
    np.testing.assert_allclose(O, O2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)


def test_append_and_commit_window():
    K = np.zeros((10, 1, 2))
    V = np.zeros((10, 1, 2))
    Kw = np.arange(8.0).reshape(4, 1, 2)
    Ka, Va = oracle.append_window_kv(K, V, 7, Kw, -Kw)
    assert (Ka[:7] == 0).all() and (Ka[7:10] == Kw[:3]).all() and (Va[7:10] == -Kw[:3]).all()   # row n+3 falls off
    assert oracle.commit_window(7, 2, 4) == 9
    assert oracle.commit_window(7, 9, 4) == 11 and oracle.commit_window(7, -1, 4) == 7


# --------------------------------------------------------------------------
# Policy sweep (translation sections 3.2-3.3, Figs. 2-3; blog Table 3)
# --------------------------------------------------------------------------
def _sweep_case(seed, w=4, P=3, Hq=8, Hkv=2, d=16, n=40):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, Hkv, d))
    K[rng.choice(n, 4, replace=False)] += 2.0          # a few salient keys
    q_window = rng.standard_normal((w, Hq, d))
    q_past = q_window[0] + 0.5 * rng.standard_normal((P, Hq, d)).cumsum(axis=0)
    s_draft = rng.random(n)
    s_target = rng.random(n)
    return q_window, q_past, K, s_draft, s_target


def test_sweep_oracle_row_bounds_every_policy_and_nested_rows_grow():
    """Eq. (4): the SD oracle maximises the windowed ARR over all k-subsets,
    so it bounds every policy row; TopK sets are nested in k, so the history,
    draft, Dustin-T and Dustin-D rows are non-decreasing in k."""
    qw, qp, K, sd, st = _sweep_case(1)
    ks = [4, 6, 8, 12, 20, 39]
    out = oracle.policy_sweep(qw, qp, K, sd, st, ks, [max(0, (k - 4) // 2) for k in ks], 2, 2)
    assert out.shape == (3 + 5, len(ks))
    assert (out[0][None, :] >= out - 1e-12).all()
    for row in range(0, out.shape[0] - 1):                # Dustin-H's m changes with k
        assert (np.diff(out[row]) >= -1e-12).all(), row
    # brute force: the oracle row is the best k-subset at a small k
    A = oracle.window_attention(qw, K)
    best = max(oracle.arr_window(A, list(c)) for c in itertools.combinations(range(K.shape[0]), 2))
    assert abs(oracle.policy_sweep(qw, qp, K, sd, st, [2], [0], 0, 0)[0, 0] - best) < 1e-12


def test_sweep_full_budget_recovers_everything():
    """ARR = 1 when the set covers V_i (translation section 3.1), for every policy."""
    qw, qp, K, sd, st = _sweep_case(2, n=25)
    out = oracle.policy_sweep(qw, qp, K, sd, st, [25, 40], [10, 10], 3, 5)
    np.testing.assert_allclose(out, 1.0, atol=1e-12)


def test_sweep_policies_reduce_to_the_oracle():
    """Special cases that turn each policy into the SD oracle: a past query
    equal to the (single) window query, draft scores equal to the window
    mean Abar, and Dustin-T without protected tokens on S_Target = Abar."""
    qw, qp, K, sd, st = _sweep_case(3, w=1, P=2)
    qp = np.stack([qw[0], qp[1]])
    Abar = oracle.window_attention(qw, K).mean(axis=0)
    anti = 1.0 - Abar                                            # ranks the least attended first
    ks = [3, 7, 15]
    # draft scores = Abar, target scores anti-correlated
    out = oracle.policy_sweep(qw, qp, K, Abar, anti, ks, [0, 0, 0], 0, 0)
    np.testing.assert_allclose(out[1], out[0], atol=1e-15)     # history with delta = 0
    np.testing.assert_allclose(out[3], out[0], atol=1e-15)     # draft lookahead = Abar
    np.testing.assert_allclose(out[5], out[0], atol=1e-15)     # Dustin-D: all budget to the draft
    assert (out[4] < out[0] - 1e-6).all()                       # Dustin-T ranks by the anti scores
    assert not np.allclose(out[2], out[0])                      # the drifted query is worse
    # the roles swapped
    out = oracle.policy_sweep(qw, qp, K, anti, Abar, ks, [0, 0, 0], 0, 0)
    np.testing.assert_allclose(out[4], out[0], atol=1e-15)     # Dustin-T on S_T = Abar
    assert (out[3] < out[0] - 1e-6).all() and (out[5] < out[0] - 1e-6).all()


def test_sweep_history_rows_use_the_past_query_attention():
    """The history row ranks by A_{i-delta,.} (Eq. 1 with the past query), not
    by the window: checked against a direct TopK of the past query's head
    mean attention computed with scipy."""
    qw, qp, K, sd, st = _sweep_case(4, P=1, Hq=4, Hkv=1)
    d = K.shape[2]
    logits = np.einsum("hd,nd->hn", qp[0], K[:, 0, :]) / np.sqrt(d)
    Ap = scipy.special.softmax(logits, axis=1).mean(axis=0)
    order = np.lexsort((np.arange(Ap.size), -Ap))
    A = oracle.window_attention(qw, K)
    for k in (3, 9):
        want = A[:, np.sort(order[:k])].sum(axis=1).mean()
        got = oracle.policy_sweep(qw, qp, K, sd, st, [k], [0], 0, 0)[1, 0]
        assert abs(got - want) < 1e-12


# --------------------------------------------------------------------------
# Page-level estimator (Quest-16 of the blog's Fig. 8)
# --------------------------------------------------------------------------
def test_page_bounds_enclose_and_touch_the_keys():
    """Every key of a page lies inside its box, each face is reached by some
    key of the page, single-token pages collapse to the key, and the ragged
    last page covers only the positions below n."""
    rng = np.random.default_rng(5)
    K = rng.standard_normal((50, 3, 8))
    kmin, kmax = oracle.page_key_bounds(K, 37, page=16)
    assert kmin.shape == (3, 3, 8)
    for p in range(3):
        blk = K[p * 16:min(37, p * 16 + 16)]
        assert (blk >= kmin[p] - 0).all() and (blk <= kmax[p]).all()
        assert (np.isclose(blk, kmin[p]).any(axis=0)).all() and (np.isclose(blk, kmax[p]).any(axis=0)).all()
    assert not np.allclose(kmax[2], K[32:48].max(axis=0))          # positions 37.. excluded
    k1, x1 = oracle.page_key_bounds(K, 7, page=1)
    assert np.array_equal(k1, K[:7]) and np.array_equal(x1, K[:7])


def test_page_scores_bound_the_logits_and_match_the_box_corners():
    """The score bounds the page's summed logits from above, is exact for
    single-token pages, and equals brute force over the 2^d corners of the
    box (per head and step); a one-hot key pins the head -> KV head map."""
    rng = np.random.default_rng(6)
    w, Hq, Hkv, d, n = 2, 4, 2, 3, 40
    q = rng.standard_normal((w, Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    kmin, kmax = oracle.page_key_bounds(K, n, 8)
    sc = oracle.page_scores(q, kmin, kmax)
    G = Hq // Hkv
    s = 1 / np.sqrt(d)
    for p in range(5):
        blk = K[p * 8:(p + 1) * 8]
        exact = max(sum(s * q[t, h] @ blk[j, h // G] for t in range(w) for h in range(Hq)) for j in range(8))
        assert sc[p] >= exact - 1e-12
        corners = 0.0
        for t in range(w):
            for h in range(Hq):
                g = h // G
                corners += s * max(q[t, h] @ np.where(c, kmax[p, g], kmin[p, g])
                                   for c in itertools.product([False, True], repeat=d))
        assert abs(sc[p] - corners) < 1e-12
    k1, x1 = oracle.page_key_bounds(K, n, 1)
    exact1 = np.array([sum(s * q[t, h] @ K[j, h // G] for t in range(w) for h in range(Hq)) for j in range(n)])
    np.testing.assert_allclose(oracle.page_scores(q, k1, x1), exact1, atol=1e-12)
    # one-hot: only KV head 1 holds a key, so only heads G.. 2G-1 see it
    K2 = np.zeros((1, Hkv, d))
    K2[0, 1, 0] = 1.0
    q2 = np.zeros((1, Hq, d))
    q2[0, G, 0] = 2.0                 # a head of group 1
    q2[0, 0, 0] = 5.0                 # a head of group 0 (sees a zero key)
    b0, b1 = oracle.page_key_bounds(K2, 1, 1)
    assert abs(oracle.page_scores(q2, b0, b1)[0] - 2.0 / np.sqrt(d)) < 1e-15


# ---------------------------------------------------------------------------
# Offline configuration search (blog section 2.4, Fig. 6)

def _search_case(seed, L=3, w=3, H=4, Hkv=2, d=8, n=24):
    """Several target layers: per-layer window attention A_l and per-head
    previous-query attention, plus a few draft-like score vectors."""
    rng = np.random.default_rng(seed)
    A_layers, head_prev = [], []
    for _ in range(L):
        K = rng.standard_normal((n, Hkv, d)) * 1.3
        q = rng.standard_normal((w, H, d)) * 1.3
        A_layers.append(oracle.window_attention(q, K))
        qp = q[0] + 0.4 * rng.standard_normal((H, d))
        head_prev.append(oracle.head_probs(qp[None], K)[:, 0, :])      # [H][n]
    draft = rng.random((5, n)) ** 3
    return A_layers, np.stack(head_prev), draft


def _top_mass(v, k):
    """Sum of the k largest entries, by a full sort (independent of topk_desc)."""
    return float(np.sort(np.asarray(v, dtype=np.float64))[::-1][:k].sum())


def test_search_objective_full_budget_and_oracle_unit():
    """Every layer's A sums to 1 per step, so the whole history scores 1; a
    target unit equal to the layer-mean Abar, without protected tokens,
    reproduces the SD oracle of that mean (Eq. 3-4) at every budget."""
    A_layers, head_prev, draft = _search_case(1)
    n = A_layers[0].shape[1]
    Abar = np.mean([A.mean(axis=0) for A in A_layers], axis=0)
    for k in (1, 5, 11, n):
        got = oracle.candidate_objectives(A_layers, k, 0, 0, 0, units_t=[Abar, head_prev[0, 0]])
        assert got[0] == pytest.approx(_top_mass(Abar, k), abs=1e-12)
        assert got[0] >= got[1] - 1e-12
    full = oracle.candidate_objectives(A_layers, n, 3, 2, 2, base_d=draft[0], base_t=draft[1])
    assert full[0] == pytest.approx(1.0, abs=1e-12)


def test_search_objective_is_the_layer_mean_and_sides_add():
    """One layer reproduces Eq. 2 of the set built by select_verify_set; the
    per-candidate sums base + unit and per-candidate m equal separate calls
    with the summed vectors."""
    A_layers, head_prev, draft = _search_case(2)
    n = A_layers[0].shape[1]
    k, m = 9, 3
    I, _ = oracle.select_verify_set(draft[0], draft[1], n, k, m, 1, 2)
    one = oracle.candidate_objectives(A_layers[:1], k, m, 1, 2, base_d=draft[0], base_t=draft[1])[0]
    assert one == pytest.approx(float(A_layers[0][:, I].sum(axis=1).mean()), abs=1e-12)
    got = oracle.candidate_objectives(A_layers, k, m, 1, 2, base_d=draft[0], units_d=draft[2:4], base_t=draft[1])
    for c in range(2):
        want = oracle.candidate_objectives(A_layers, k, m, 1, 2, base_d=draft[0] + draft[2 + c], base_t=draft[1])[0]
        assert got[c] == pytest.approx(want, abs=1e-12)
    ms = [0, 2, 6]
    gm = oracle.candidate_objectives(A_layers, k, m, 1, 2, base_d=draft[0], base_t=draft[1], ms=ms)
    for c, mm in enumerate(ms):
        assert gm[c] == pytest.approx(
            oracle.candidate_objectives(A_layers, k, mm, 1, 2, base_d=draft[0], base_t=draft[1])[0], abs=1e-12)


def test_srh_matrix_closed_forms_and_head_topk():
    """A head whose attention is the layer-mean Abar scores the SD oracle's
    ARR; a head with uniform attention takes the first k positions (ties to
    the lower position); the head TopK matches a plain sort of the matrix."""
    A_layers, head_prev, _ = _search_case(3, L=2, H=4)
    n = A_layers[0].shape[1]
    k = 6
    Abar = np.mean([A.mean(axis=0) for A in A_layers], axis=0)
    hp = head_prev.copy()
    hp[0, 1] = Abar
    hp[1, 2] = np.full(n, 1.0 / n)
    M = oracle.srh_head_scores(A_layers, hp, k, 0, 0)
    assert M.shape == (2, 4)
    assert M[0, 1] == pytest.approx(_top_mass(Abar, k), abs=1e-12)
    assert M[1, 2] == pytest.approx(float(Abar[:k].sum()), abs=1e-12)
    assert M.max() == pytest.approx(M[0, 1], abs=1e-12)
    want = sorted(((-M[l, h], l, h) for l in range(2) for h in range(4)))
    assert oracle.srh_select(M, 4) == sorted((l, h) for (_, l, h) in want[:4])
    # ties at the cut go to the lower (layer, head)
    Mt = np.array([[0.5, 0.7, 0.5, 0.1], [0.5, 0.2, 0.9, 0.5]])
    assert oracle.srh_select(Mt, 4) == [(0, 0), (0, 1), (0, 2), (1, 2)]


def test_greedy_matches_exhaustive_choices():
    """The first pick is the best single candidate and the second the best
    completion of it (exhaustive search over all pairs); the objective curve
    rises strictly; ties go to the lower index."""
    A_layers, head_prev, draft = _search_case(4)
    units = head_prev.reshape(-1, head_prev.shape[-1])[:6]
    k = 7

    def obj(ch):
        return oracle.candidate_objectives(A_layers, k, 0, 1, 1, base_t=units[list(ch)].sum(axis=0))[0]

    singles = [obj([c]) for c in range(6)]
    chosen, curve = oracle.greedy_target(A_layers, units, k, 1, 1, max_units=3)
    assert chosen[0] == int(np.argmax(singles))
    best2 = max(((obj([chosen[0], c]), -c) for c in range(6) if c != chosen[0]))
    if len(chosen) > 1:
        assert chosen[1] == -best2[1] and curve[1] == pytest.approx(best2[0], abs=1e-12)
    else:
        assert best2[0] <= curve[0]
    assert all(b > a for a, b in zip(curve, curve[1:]))
    # ties: the two best candidates are identical -> the lower index wins
    Abar = np.mean([A.mean(axis=0) for A in A_layers], axis=0)
    twin = np.stack([units[0], Abar, Abar])
    ch, _ = oracle.greedy_target(A_layers, twin, k, 1, 1, max_units=1)
    assert ch == [1]


def test_greedy_stops_at_a_perfect_unit_and_keeps_only_improving_draft_layers():
    """Once a unit reaches the SD-oracle bound (Eq. 4) nothing can improve on
    it strictly, so the greedy stops; a draft layer that does not raise the
    target-history objective is not kept."""
    A_layers, head_prev, draft = _search_case(5)
    n = A_layers[0].shape[1]
    k = 6
    Abar = np.mean([A.mean(axis=0) for A in A_layers], axis=0)
    units = np.stack([head_prev[0, 0], Abar, head_prev[1, 1]])
    chosen, curve = oracle.greedy_target(A_layers, units, k, 0, 0, max_units=3)
    assert chosen == [1] and curve[0] == pytest.approx(_top_mass(Abar, k), abs=1e-12)
    # draft side: a draft layer equal to Abar helps the uniform-target set; a
    # zero-information draft layer (constant) takes the lowest positions
    flat = np.full(n, 1.0)
    ch_d, curve_d = oracle.greedy_draft(A_layers, flat, np.stack([flat, Abar]), k, k, 0, 0, max_units=2)
    assert ch_d == [1]
    start = oracle.candidate_objectives(A_layers, k, 0, 0, 0, base_t=flat)[0]
    assert curve_d[0] > start
    ch_none, _ = oracle.greedy_draft(A_layers, Abar, np.stack([flat]), k, k, 0, 0, max_units=1)
    assert ch_none == []


def test_m_search_is_exhaustive_and_reduces_to_the_tiers():
    """The m search returns the grid's maximum (earliest on ties); m = 0 is
    the target-history set and m = k - |P| the draft-lookahead set."""
    A_layers, head_prev, draft = _search_case(6)
    k, ns, nw = 10, 1, 2
    ms = list(range(0, k - ns - nw + 1))
    vals, best = oracle.m_search(A_layers, draft[0], draft[1], k, ms, ns, nw)
    assert best == ms[[i for i, v in enumerate(vals) if v == vals.max()][0]]
    t_only = oracle.candidate_objectives(A_layers, k, 0, ns, nw, base_t=draft[1])[0]
    d_only = oracle.candidate_objectives(A_layers, k, 0, ns, nw, base_d=draft[0])[0]
    assert vals[0] == pytest.approx(t_only, abs=1e-12)
    assert vals[-1] == pytest.approx(d_only, abs=1e-12)


def test_config_search_is_consistent():
    """The composed search: target heads come from the head TopK, the curves
    rise, and the reported best m reproduces the objective of the final set."""
    A_layers, head_prev, draft = _search_case(7, L=3, H=4)
    k = 8
    r = oracle.config_search(A_layers, head_prev, draft, k, 3, [0, 1, 2, 3, 4, 5], 1, 1, T=6, S=3, max_draft=3)
    assert len(r["candidates"]) == 6 and set(r["target_heads"]) <= set(r["candidates"])
    assert all(b > a for a, b in zip(r["target_curve"], r["target_curve"][1:]))
    assert all(b > a for a, b in zip(r["draft_curve"], r["draft_curve"][1:]))
    if r["draft_layers"]:
        s_t = sum(head_prev[l, h] for (l, h) in r["target_heads"])
        s_d = draft[r["draft_layers"]].sum(axis=0)
        v = oracle.candidate_objectives(A_layers, k, r["m"], 1, 1, base_d=s_d, base_t=s_t)[0]
        assert v == pytest.approx(r["m_values"].max(), abs=1e-12)


def test_search_batch_is_the_mean_of_its_sequences():
    """A batch of equal-length sequences scores each configuration by the
    mean of the sequences' objectives: a batch of one equals the sequence,
    and a two-sequence batch of the same sequence equals it too, while a
    batch of two different sequences lies between their values."""
    A1, hp1, d1 = _search_case(8)
    A2, hp2, d2 = _search_case(9)
    k, m = 7, 2
    one = oracle.candidate_objectives(A1, k, m, 1, 1, base_d=d1[0], units_t=hp1[0])
    b1 = oracle.candidate_objectives([A1], k, m, 1, 1, base_d=d1[0][None], units_t=hp1[0][:, None])
    np.testing.assert_allclose(b1, one, rtol=0, atol=1e-12)
    same = oracle.candidate_objectives([A1, A1], k, m, 1, 1, base_d=np.stack([d1[0], d1[0]]),
                                       units_t=np.stack([hp1[0], hp1[0]], axis=1))
    np.testing.assert_allclose(same, one, rtol=0, atol=1e-12)
    two = oracle.candidate_objectives(A2, k, m, 1, 1, base_d=d2[0], units_t=hp2[0])
    mix = oracle.candidate_objectives([A1, A2], k, m, 1, 1, base_d=np.stack([d1[0], d2[0]]),
                                      units_t=np.stack([hp1[0], hp2[0]], axis=1))
    np.testing.assert_allclose(mix, (one + two) / 2, rtol=0, atol=1e-12)
    # the batched SRH matrix keeps the (layer, head) layout of the single-sequence one
    M1 = oracle.srh_head_scores(A1, hp1, k, 1, 1)
    np.testing.assert_allclose(oracle.srh_head_scores([A1, A1], np.stack([hp1, hp1]), k, 1, 1), M1, rtol=0, atol=1e-12)
    # the composed search runs on the batch layout
    r = oracle.config_search([A1, A2], np.stack([hp1, hp2]), np.stack([d1, d2], axis=1), k, 2, [0, 1, 2, 3], 1, 1,
                             T=4, S=2, max_draft=2)
    assert r["M"].shape == hp1.shape[:2]
