"""Plain CPU oracle for the Dustin sparse-verification step (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Sources (the three web pages about "Dustin: Draft-Augmented Sparse
Verification for Efficient Long-Context Generation with Speculative
Decoding", arXiv 2606.24957):

* the Chinese translation of the arXiv HTML (bittide.aicompass.dev),
  section 3.1, equations (1)-(4): ARR, windowed ARR and the SD oracle;
  section 3.2: history attention A_{i-delta,.} (delta = 1 for S_Target; the
  history-policy comparison of Fig. 2 over several delta);
  section 3.3 (Fig. 3): the draft lookahead compared with the oracle;
  related work: Quest's page scoring from min/max key statistics (the
  page-level estimator of section 5.4.1);
* the blog summary, section 2.4 and Fig. 6: the semantic-retrieval-head
  score matrix (layer x head) with its head TopK, and the offline
  configuration search (greedy target layers, then greedy draft layers with
  the target fixed, then the draft/target budget split m), whose objective
  is the windowed ARR;
* the blog summary (liuzhao09.github.io), section 2.2 (hybrid aggregation:
  S_Draft over H_d, L_d, Gamma; S_Target over H_t, L_t; one global index
  set), section 2.3 (verification set: protected sink + recent window, draft
  top-m, target fill), section 2.4 (scoring restricted to a few semantic
  retrieval heads), Fig. 5 (Stage 2: the target verifies the draft tokens
  with the compressed KV; accepted tokens are written back to the target KV,
  rejected ones are dropped).

The pages print the S_Draft / S_Target and verification-set formulas only as
prose (the formula slots of the blog are empty).  The readings taken here are
the plainest ones the prose supports; each function states its reading.

Everything is computed per sequence in float64 with no blocking, fusion or
reordering beyond the definitions.  Inputs may be float32/bfloat16-rounded
values; they are upcast to float64 first.

Layouts (per sequence):
  q        [w][Hq][d]            window queries q_{i+s}, s = 0..w-1
  K, V     [n][Hkv][d]           history keys/values of one target layer
  q_hist   [S][d]                most recent target query, one row per
                                 scored (layer, head) pair
  q_draft  [L_d][Gamma][H_d][d_d]
  K_draft  [L_d][n][Hkv_d][d_d]
Query head h reads KV head floor(h / G) with G = Hq / Hkv.

Parity pins for every function live in tests/test_oracle_pins.py; no
function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "softmax",
    "head_probs",
    "window_attention",
    "dense_attention",
    "sparse_attention",
    "verify_attention",
    "append_window_kv",
    "commit_window",
    "arr_step",
    "arr_window",
    "sd_oracle",
    "score_target",
    "draft_row_lse",
    "score_draft_given_lse",
    "score_draft",
    "select_verify_set",
    "history_policy",
    "policy_sweep",
    "page_key_bounds",
    "page_scores",
    "search_objective",
    "candidate_objectives",
    "srh_head_scores",
    "srh_select",
    "greedy_select",
    "greedy_target",
    "greedy_draft",
    "m_search",
    "config_search",
    "topk_desc",
    "protected_positions",
    "pages_to_contiguous",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def softmax(x, axis=-1):
    """Numerically plain softmax along ``axis`` (max-subtracted exp / sum)."""
    x = _f64(x)
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def _kv_head_of(h, Hq, Hkv):
    """Grouped-query mapping: query head h reads KV head floor(h / G)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def head_probs(q, K, scale=None):
    """Per-head attention probabilities of the window queries over history.

    P[h][s][j] = softmax_j(scale * q[s][h] . K[j][g(h)]), j in [0, n).

    Reading (translation section 3.1, definition of A_{i,j}): A is normalised
    over the valid history V_i only, so the w window tokens are not part of
    the denominator and sum_j A_{i,j} = 1 holds at every window step.
    """
    q = _f64(q)
    K = _f64(K)
    w, Hq, d = q.shape
    n, Hkv, dk = K.shape
    assert dk == d
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    P = np.empty((Hq, w, n))
    for h in range(Hq):
        g = _kv_head_of(h, Hq, Hkv)
        logits = scale * (q[:, h, :] @ K[:, g, :].T)  # [w][n]
        P[h] = softmax(logits, axis=-1)
    return P


def window_attention(q, K, scale=None):
    """A[s][j]: full-cache attention weight of window step s on position j.

    Translation section 3.1 defines a single normalised weight A_{i,j} per
    step without saying how heads are combined; reading taken: the mean over
    the query heads of one layer.  ARR is linear in A, so this equals the
    mean of the per-head ARRs, and one global set serves all heads (blog
    section 2.2).
    """
    return head_probs(q, K, scale).mean(axis=0)


def dense_attention(q, K, V, scale=None):
    """Full-cache verification attention (blog Fig. 7 "Full Cache" baseline).

    O[s][h] = sum_j P[h][s][j] * V[j][g(h)].
    """
    P = head_probs(q, K, scale)
    V = _f64(V)
    w, Hq, d = np.asarray(q).shape
    Hkv = V.shape[1]
    O = np.empty((w, Hq, V.shape[2]))
    for h in range(Hq):
        O[:, h, :] = P[h] @ V[:, _kv_head_of(h, Hq, Hkv), :]
    return O


def sparse_attention(q, K, V, I, scale=None):
    """Sparse verification attention over the compressed KV (blog Fig. 5,
    Stage 2): the target attends only to the rows in the index set I.

    O[s][h] = sum_{j in I} softmax_{j in I}(scale * q[s][h] . K[j][g(h)]) V[j][g(h)].
    Also returns lse[s][h] = log sum_{j in I} exp(scale * q . k_j) (natural log).
    Entries of I that are negative (padding) are ignored.
    """
    I = np.asarray(I, dtype=np.int64)
    I = I[I >= 0]
    q = _f64(q)
    w, Hq, d = q.shape
    Ks = _f64(K)[I]
    Vs = _f64(V)[I]
    Hkv = np.asarray(K).shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((w, Hq, np.asarray(V).shape[2]))
    lse = np.full((w, Hq), -np.inf)
    if I.size == 0:
        return O, lse
    for h in range(Hq):
        g = _kv_head_of(h, Hq, Hkv)
        logits = scale * (q[:, h, :] @ Ks[:, g, :].T)  # [w][|I|]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=1, keepdims=True)
        O[:, h, :] = (e / z) @ Vs[:, g, :]
        lse[:, h] = (m + np.log(z))[:, 0]
    return O, lse


def verify_attention(q, K, V, K_win, V_win, I, scale=None):
    """Stage 2 of blog Fig. 5 with the draft window itself in view: the w
    draft tokens are verified in one pass, and draft token s sees the
    compressed history I plus the draft tokens 0..s (the usual causal order
    inside a speculative window; the pages leave this block implicit, and
    this is its plainest reading).

    K_win, V_win [w][Hkv][d]: the window tokens' keys and values.
    O[s][h] = softmax over (I u window[0..s]) of scale * q[s][h] . k, times v.
    Returns O [w][Hq][d] and lse [w][Hq] (natural log).
    """
    I = np.asarray(I, dtype=np.int64)
    I = I[I >= 0]
    q = _f64(q)
    w, Hq, d = q.shape
    Kh, Vh = _f64(K)[I], _f64(V)[I]
    Kw, Vw = _f64(K_win), _f64(V_win)
    Hkv = Kw.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros((w, Hq, Vw.shape[2]))
    lse = np.zeros((w, Hq))
    for s in range(w):
        for h in range(Hq):
            g = _kv_head_of(h, Hq, Hkv)
            keys = np.concatenate([Kh[:, g, :], Kw[: s + 1, g, :]], axis=0)
            vals = np.concatenate([Vh[:, g, :], Vw[: s + 1, g, :]], axis=0)
            logits = scale * (keys @ q[s, h, :])
            m = logits.max()
            e = np.exp(logits - m)
            z = e.sum()
            O[s, h, :] = (e / z) @ vals
            lse[s, h] = m + np.log(z)
    return O, lse


def append_window_kv(K, V, n, K_win, V_win):
    """The draft tokens' keys and values go into the cache right after the
    history (positions n .. n + w - 1) before they are verified; positions
    past the cache end are dropped.  Returns new arrays (K, V of [N][Hkv][d])."""
    K, V = np.array(K, copy=True), np.array(V, copy=True)
    for t in range(np.asarray(K_win).shape[0]):
        if n + t < K.shape[0]:
            K[n + t] = K_win[t]
            V[n + t] = V_win[t]
    return K, V


def commit_window(n, accepted, w):
    """After verification the accepted draft tokens stay in the cache (blog
    Fig. 5): the history grows by the accepted count, clamped to [0, w]; the
    rows of rejected tokens lie past the new length and are never read."""
    return n + min(max(int(accepted), 0), w)


def arr_step(A, I):
    """Eq. (1) of translation section 3.1, one value per window step:
    ARR_{i+s} = sum_{j in K} A_{i+s, j}.  Negative entries of I are padding."""
    A = _f64(A)
    I = np.asarray(I, dtype=np.int64)
    I = I[I >= 0]
    return A[:, I].sum(axis=1)


def arr_window(A, I):
    """Eq. (2): windowed ARR = (1/w) * sum_{s=0}^{w-1} ARR_{i+s}."""
    return float(np.mean(arr_step(A, I)))


def topk_desc(scores, k, candidates=None):
    """TopK_k by (score descending, position ascending).

    The pages do not state a tie rule; reading taken: lower position first.
    Returns the chosen positions in selection order.
    """
    scores = _f64(scores)
    if candidates is None:
        candidates = np.arange(scores.shape[0])
    candidates = np.asarray(candidates, dtype=np.int64)
    if k <= 0 or candidates.size == 0:
        return np.zeros(0, dtype=np.int64)
    # np.lexsort sorts by the last key first: primary -score, secondary index.
    order = np.lexsort((candidates, -scores[candidates]))
    return candidates[order[: min(k, candidates.size)]]


def sd_oracle(A, k):
    """Eq. (3)-(4): SD oracle.

    Abar_j = (1/w) sum_s A_{i+s, j};  K_orc = TopK_k(Abar);
    ARR^(w)(orc) = sum_{j in K_orc} Abar_j.
    Returns (sorted K_orc, ARR^(w)(orc), Abar).
    """
    Abar = _f64(A).mean(axis=0)
    sel = np.sort(topk_desc(Abar, k))
    return sel, float(Abar[sel].sum()), Abar


def score_target(q_hist, K_layers, sub_heads, Hq, scale=None):
    """S_Target (blog section 2.2 and section 2.4).

    The target's most recent attention (translation section 3.2: history
    distance delta = 1) recomputed by QK^T on the searched subset of
    (layer, head) pairs only.  The blog gives the aggregation only in words
    ("aggregate into a global token-importance vector"); reading taken: the
    plain sum of the per-head softmax probabilities,
        S_T[j] = sum_{(l,h) in subset} softmax_j(scale * q_hist[l,h] . K_l[j][g(h)]).
    A mean would differ by a constant factor and rank identically.

    q_hist: [S][d]; K_layers: dict or list indexed by layer -> [n][Hkv][d];
    sub_heads: S pairs (layer, head).
    """
    q_hist = _f64(q_hist)
    S, d = q_hist.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n = np.asarray(K_layers[sub_heads[0][0]]).shape[0]
    out = np.zeros(n)
    for r, (layer, h) in enumerate(sub_heads):
        K = _f64(K_layers[layer])
        g = _kv_head_of(h, Hq, K.shape[1])
        out += softmax(scale * (K[:, g, :] @ q_hist[r]))
    return out


def score_draft(q_draft, K_draft, scale=None):
    """S_Draft (blog section 2.2 and Fig. 5: the draft's attention heat maps
    are summed along the draft steps).

    Reading taken: plain sum over draft layers l, draft query heads h and
    draft steps g of the draft's attention over the history positions,
        S_D[j] = sum_{l,h,g} softmax_j(scale_d * q_draft[l,g,h] . K_draft[l][j][c(h)]),
    with c(h) = floor(h / G_d) and the softmax taken over history positions
    only (the draft's own new tokens are not history).

    q_draft: [L_d][Gamma][H_d][d_d]; K_draft: [L_d][n][Hkv_d][d_d].
    """
    q_draft = _f64(q_draft)
    L_d, Gamma, H_d, d_d = q_draft.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d_d)
    n = np.asarray(K_draft[0]).shape[0]
    out = np.zeros(n)
    for l in range(L_d):
        K = _f64(K_draft[l])
        Hkv_d = K.shape[1]
        for h in range(H_d):
            c = _kv_head_of(h, H_d, Hkv_d)
            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)  # [Gamma][n]
            out += softmax(logits, axis=-1).sum(axis=0)
    return out


def draft_row_lse(q_draft, K_draft, scale=None):
    """Row normalisers of the softmaxes that S_Draft sums (blog section 2.2):
    for draft layer l, draft step g and draft head h,
        lse[l, g, h] = ln sum_j exp(scale_d * q_draft[l,g,h] . K_draft[l][j][c(h)]),
    j over the history positions, c(h) = floor(h / G_d).  These are what the
    draft model's own attention over the history computes for the same
    queries.  Returns [L_d][Gamma][H_d] (float64); -inf for an empty history.
    """
    q_draft = _f64(q_draft)
    L_d, Gamma, H_d, d_d = q_draft.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d_d)
    out = np.full((L_d, Gamma, H_d), -np.inf)
    for l in range(L_d):
        K = _f64(K_draft[l])
        if K.shape[0] == 0:
            continue
        for h in range(H_d):
            c = _kv_head_of(h, H_d, K.shape[1])
            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]
            m = logits.max(axis=-1, keepdims=True)
            out[l, :, h] = (m + np.log(np.exp(logits - m).sum(axis=-1, keepdims=True)))[:, 0]
    return out


def score_draft_given_lse(q_draft, K_draft, lse, scale=None):
    """S_Draft with the row normalisers supplied (blog section 2.2; the
    normalisers are the draft attention's, see draft_row_lse):
        S_D[j] = sum_{l,g,h} exp(scale_d * q_draft[l,g,h] . K_draft[l][j][c(h)] - lse[l,g,h]).
    With lse = draft_row_lse(q_draft, K_draft) this is score_draft.
    """
    q_draft = _f64(q_draft)
    lse = _f64(lse)
    L_d, Gamma, H_d, d_d = q_draft.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d_d)
    n = np.asarray(K_draft[0]).shape[0]
    out = np.zeros(n)
    for l in range(L_d):
        K = _f64(K_draft[l])
        for h in range(H_d):
            c = _kv_head_of(h, H_d, K.shape[1])
            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]
            out += np.exp(logits - lse[l, :, h][:, None]).sum(axis=0)
    return out


def protected_positions(n, n_sink, n_window):
    """Protected tier of the verification set (blog section 2.3): the first
    n_sink positions (attention sinks) and the last n_window positions
    (recent window), clipped to [0, n)."""
    sink = np.arange(0, min(n_sink, n))
    recent = np.arange(max(0, n - n_window), n)
    return np.union1d(sink, recent).astype(np.int64)


def select_verify_set(s_draft, s_target, n, k, m, n_sink, n_window):
    """Verification set I_verify (blog section 2.3), one per sequence, shared
    by every layer and head (blog section 2.2).

    Tiers, in the order the blog gives them:
      1. P = attention sinks [0, n_sink) and recent window [n - n_window, n);
      2. D = the m' highest-S_Draft positions outside P;
      3. T = the highest-S_Target positions outside P and D, filling the
         budget k.
    Reading of the budget: k counts the protected tokens; m' =
    min(m, k - |P|, |V \\ P|); |I| = min(k, n).  A missing S_Draft means
    m' = 0 (target only); a missing S_Target means the draft tier fills the
    budget (m' = k - |P|).  Ties: higher score first, then lower position.

    Returns (idx ascending int64 array, tier array aligned with idx:
    0 protected, 1 draft, 2 target).
    """
    if s_draft is None and s_target is None:
        raise ValueError("at least one score vector is required")
    if n_sink + n_window > k:
        raise ValueError("protected tokens exceed the budget")
    P = protected_positions(n, n_sink, n_window)
    rest = np.setdiff1d(np.arange(n), P)
    budget = k - P.size
    if s_draft is None:
        m_eff = 0
    elif s_target is None:
        m_eff = budget
    else:
        m_eff = m
    m_eff = max(0, min(m_eff, budget, rest.size))
    D = topk_desc(s_draft, m_eff, rest) if m_eff > 0 else np.zeros(0, np.int64)
    rest2 = np.setdiff1d(rest, D)
    t_cnt = max(0, min(budget - D.size, rest2.size))
    T = topk_desc(s_target, t_cnt, rest2) if t_cnt > 0 else np.zeros(0, np.int64)
    idx = np.concatenate([P, D, T]).astype(np.int64)
    tier = np.concatenate([
        np.zeros(P.size, np.int8),
        np.ones(D.size, np.int8),
        np.full(T.size, 2, np.int8),
    ])
    order = np.argsort(idx, kind="stable")
    return idx[order], tier[order]


def history_policy(A_past, k):
    """Translation section 3.2 (Fig. 2): rank the history positions by the
    head-mean full-cache attention A_{i-delta,.} of the query delta steps
    back and keep the top k (ties: lower position first).  Returns the
    positions ascending."""
    return np.sort(topk_desc(A_past, k))


def policy_sweep(q_window, q_past, K, s_draft, s_target, ks, m_hybrid, n_sink, n_window, scale=None):
    """Windowed ARR (Eq. 2) of the selection policies the pages compare, at
    every budget k in ks, for one sequence:

      row 0             the SD oracle (Eq. 3-4), the upper bound;
      rows 1 .. P       the history policy of each past query (translation
                        section 3.2, Fig. 2), P = len(q_past);
      row P + 1         the draft lookahead alone, TopK_k of S_Draft
                        (translation section 3.3, Fig. 3);
      rows P + 2 .. + 4 the verification set of blog section 2.3 with
                        m = 0 (target history only, Dustin-T), m = k - |P|
                        (draft lookahead only after the protected tokens,
                        Dustin-D) and m = m_hybrid[k] (Dustin-H), the three
                        variants of blog Table 3.

    A is the head-mean full-cache attention of the window queries (Eq. 1);
    the past queries' A_{i-delta,.} comes from the same definition with a
    one-step window.  q_window [w][Hq][d]; q_past [P][Hq][d]; K [n][Hkv][d];
    s_draft, s_target [n].  Returns [P + 5][len(ks)].
    """
    A = window_attention(q_window, K, scale)
    n = A.shape[1]
    q_past = _f64(q_past)
    A_past = [window_attention(q_past[p][None], K, scale)[0] for p in range(q_past.shape[0])]
    P = len(A_past)
    out = np.zeros((P + 5, len(ks)))
    for ki, k in enumerate(ks):
        out[0, ki] = arr_window(A, sd_oracle(A, k)[0])
        for p in range(P):
            out[1 + p, ki] = arr_window(A, history_policy(A_past[p], k))
        out[P + 1, ki] = arr_window(A, np.sort(topk_desc(s_draft, k)))
        ms = (0, k - n_sink - n_window, m_hybrid[ki])
        for r, m in enumerate(ms):
            I, _ = select_verify_set(s_draft, s_target, n, k, m, n_sink, n_window)
            out[P + 2 + r, ki] = arr_window(A, I)
    return out


def search_objective(A_layers, I):
    """Objective of the offline configuration search (blog section 2.4: the
    windowed ARR, Eq. 2, rather than task accuracy).  Reading taken for a
    model with several target layers: the global set (blog section 2.2)
    serves every layer, so the objective is Eq. 2 averaged over the target
    layers whose attention the set has to recover; with one layer it is
    Eq. 2 itself.  A_layers: [L][w][n] (each Eq. 1's A of one layer)."""
    return float(np.mean([arr_window(A, I) for A in A_layers]))


def candidate_objectives(A_layers, k, m, n_sink, n_window, base_d=None, units_d=None, base_t=None,
                         units_t=None, ms=None):
    """Search objective of the verification set (blog section 2.3) of each
    candidate configuration c:
        S_Draft  = base_d + units_d[c]   (a side is absent when neither is given)
        S_Target = base_t + units_t[c]
        m        = ms[c] if ms is given, else m.
    The number of candidates is the length of whichever per-candidate list
    is given (1 if none).

    One sequence: A_layers [L][w][n], base [n], units [C][n].  A batch of
    equal-length sequences (the profiling batch of the offline search):
    A_layers [B][L][w][n], base [B][n], units [C][B][n]; the objective of a
    configuration is then the mean over the batch of each sequence's.
    Returns [C]."""
    A_layers = [_f64(A) for A in A_layers] if np.ndim(A_layers[0]) == 2 else A_layers
    batch = np.ndim(A_layers[0]) == 3
    lens = [len(u) for u in (units_d, units_t, ms) if u is not None]
    C = lens[0] if lens else 1
    assert all(x == C for x in lens)
    B = len(A_layers) if batch else 1
    n = np.asarray(A_layers[0]).shape[-1]

    def side(base, units, c, b):
        if base is None and units is None:
            return None
        v = np.zeros(n)
        if base is not None:
            v = v + _f64(base[b] if batch else base)
        if units is not None:
            v = v + _f64(units[c][b] if batch else units[c])
        return v

    out = np.zeros(C)
    for c in range(C):
        mm = m if ms is None else ms[c]
        tot = 0.0
        for b in range(B):
            sd, st = side(base_d, units_d, c, b), side(base_t, units_t, c, b)
            I, _ = select_verify_set(sd, st, n, k, mm, n_sink, n_window)
            tot += search_objective(A_layers[b] if batch else A_layers, I)
        out[c] = tot / B
    return out


def srh_head_scores(A_layers, head_prev, k, n_sink, n_window):
    """Full SRH score matrix of the blog's Fig. 6 (layer x head).  Reading
    taken: the score of target head (l, h) is the search objective of the
    target-history set (blog section 2.3 with m = 0) built from that head
    alone, S_Target = its previous query's attention over the history
    (translation section 3.2, delta = 1).
    head_prev: [L_t][H_q][n] per-head probabilities ([B][L_t][H_q][n] for a
    batch, with A_layers [B][L][w][n]).  Returns [L_t][H_q]."""
    head_prev = _f64(head_prev)
    if head_prev.ndim == 4:
        Bn, L, H, n = head_prev.shape
        units = head_prev.transpose(1, 2, 0, 3).reshape(L * H, Bn, n)
    else:
        L, H, n = head_prev.shape
        units = head_prev.reshape(L * H, n)
    flat = candidate_objectives(A_layers, k, 0, n_sink, n_window, units_t=units)
    return flat.reshape(L, H)


def srh_select(M, T):
    """Head TopK of the blog's Fig. 6: the T (layer, head) pairs with the
    largest SRH score, ties to the lower (layer, head).  Returns the pairs in
    ascending (layer, head) order, the order in which the greedy step then
    breaks ties (the sparse SRH matrix is a set; the pages give no order)."""
    M = _f64(M)
    L, H = M.shape
    order = np.sort(topk_desc(M.ravel(), T))
    return [(int(i) // H, int(i) % H) for i in order]


def greedy_select(objective_of, n_cand, max_units, start=-np.inf):
    """Greedy forward selection (blog section 2.4, steps 1 and 2): starting
    from the objective `start` of the empty choice, add the candidate whose
    addition gives the largest objective; stop after max_units additions or
    when no remaining candidate improves the objective strictly.  Ties go to
    the lower candidate index.  objective_of(list of chosen indices) ->
    float.  Returns (chosen indices in order, objective after each)."""
    chosen, curve, best = [], [], start
    while len(chosen) < max_units:
        top_v, top_c = -np.inf, -1
        for c in range(n_cand):
            if c in chosen:
                continue
            v = objective_of(chosen + [c])
            if v > top_v:
                top_v, top_c = v, c
        if top_c < 0 or not top_v > best:
            break
        chosen.append(top_c)
        curve.append(top_v)
        best = top_v
    return chosen, curve


def greedy_target(A_layers, units_t, k, n_sink, n_window, max_units):
    """Step 1 of the configuration search (blog section 2.4): greedily choose
    target units (each a set of target heads, given by its S_Target vector)
    for the target-history set (m = 0); the first unit is always taken."""
    units_t = _f64(units_t)

    def obj(ch):
        return candidate_objectives(A_layers, k, 0, n_sink, n_window, base_t=units_t[ch].sum(axis=0))[0]

    return greedy_select(obj, units_t.shape[0], max_units)


def greedy_draft(A_layers, s_target, units_d, k, m, n_sink, n_window, max_units):
    """Step 2 (blog section 2.4): with the target heads fixed, greedily add
    draft units (each a draft layer, given by its S_Draft vector) to the
    hybrid set with draft budget m.  The empty choice is the target-history
    set, so a draft layer is kept only if it raises the objective."""
    units_d = _f64(units_d)
    start = candidate_objectives(A_layers, k, 0, n_sink, n_window, base_t=s_target)[0]

    def obj(ch):
        return candidate_objectives(A_layers, k, m, n_sink, n_window, base_d=units_d[ch].sum(axis=0),
                                    base_t=s_target)[0]

    return greedy_select(obj, units_d.shape[0], max_units, start=start)


def m_search(A_layers, s_draft, s_target, k, ms, n_sink, n_window):
    """Step 3 (blog section 2.4; the pages tune m with Optuna, here a plain
    search over the given grid): the objective at every m in ms and the best
    m (ties: the earlier grid entry).  Returns (values [len(ms)], best m)."""
    vals = candidate_objectives(A_layers, k, 0, n_sink, n_window, base_d=s_draft, base_t=s_target, ms=list(ms))
    return vals, int(ms[int(np.argmax(vals))])


def config_search(A_layers, head_prev, draft_units, k, m0, ms, n_sink, n_window, T, S, max_draft):
    """The offline configuration search of blog section 2.4: the SRH score
    matrix and its head TopK (Fig. 6, T candidates), greedy target heads
    among them (at most S), greedy draft layers with draft budget m0 (at
    most max_draft), then the plain m search.
    One sequence: head_prev [L_t][H_q][n], draft_units [L_d][n]; a batch:
    head_prev [B][L_t][H_q][n], draft_units [L_d][B][n] (A_layers batched
    likewise)."""
    head_prev = _f64(head_prev)
    draft_units = _f64(draft_units)
    M = srh_head_scores(A_layers, head_prev, k, n_sink, n_window)
    cand = srh_select(M, T)
    if head_prev.ndim == 4:
        units_t = np.stack([head_prev[:, l, h] for (l, h) in cand])
    else:
        units_t = np.stack([head_prev[l, h] for (l, h) in cand])
    ch_t, curve_t = greedy_target(A_layers, units_t, k, n_sink, n_window, S)
    s_target = units_t[ch_t].sum(axis=0)
    ch_d, curve_d = greedy_draft(A_layers, s_target, draft_units, k, m0, n_sink, n_window, max_draft)
    if ch_d:
        s_draft = draft_units[ch_d].sum(axis=0)
        vals, m_best = m_search(A_layers, s_draft, s_target, k, ms, n_sink, n_window)
    else:
        vals, m_best = None, 0
    return {"M": M, "candidates": cand, "target_choice": ch_t, "target_curve": curve_t,
            "target_heads": [cand[c] for c in ch_t], "draft_layers": ch_d, "draft_curve": curve_d,
            "m_values": vals, "m": m_best}


def page_key_bounds(K, n, page=16):
    """Page statistics of the page-level estimator the pages compare with
    (Quest, in the translation's related work: the full cache stays and
    pages are scored with cheap min/max key statistics instead of exact
    QK^T; Quest-16 in the blog's Fig. 8): for each page of `page`
    consecutive history positions and each KV head, the elementwise minimum
    and maximum of the keys over the page's positions below n.
    K [>= n][Hkv][d] -> (kmin, kmax), each [ceil(n / page)][Hkv][d]."""
    K = _f64(K)[:n]
    npg = -(-n // page)
    kmin = np.empty((npg,) + K.shape[1:])
    kmax = np.empty((npg,) + K.shape[1:])
    for p in range(npg):
        blk = K[p * page:min(n, (p + 1) * page)]
        kmin[p] = blk.min(axis=0)
        kmax[p] = blk.max(axis=0)
    return kmin, kmax


def page_scores(q, kmin, kmax, scale=None):
    """Page criticality from the bounds alone: for window step s and query
    head h (KV head g(h)), the largest value scale * q . k can take over any
    key inside the page's box, scale * sum_d max(q_d kmin_d, q_d kmax_d).
    Reading taken for one global page set: these bounds summed over the
    window steps and query heads (as S_Target sums its heads).
    q [w][Hq][d]; kmin, kmax [npages][Hkv][d] -> [npages]."""
    q = _f64(q)
    w, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kmin, kmax = _f64(kmin), _f64(kmax)
    out = np.zeros(kmin.shape[0])
    for h in range(Hq):
        g = _kv_head_of(h, Hq, kmin.shape[1])
        for s in range(w):
            qq = q[s, h]
            out += scale * np.maximum(kmin[:, g, :] * qq, kmax[:, g, :] * qq).sum(axis=1)
    return out


def pages_to_contiguous(pool, page_row, n, page_size):
    """Logical history rows [0, n) of a paged cache.

    pool: [num_pages][page_size][...]; page_row: physical page id of each
    logical page of this sequence.  Logical position j lives in physical page
    page_row[j // page_size], slot j % page_size.
    """
    pool = np.asarray(pool)
    n_pages = (n + page_size - 1) // page_size
    rows = [pool[int(page_row[p])] for p in range(n_pages)]
    flat = np.concatenate(rows, axis=0) if rows else pool[:0].reshape((0,) + pool.shape[2:])
    return flat[:n]
