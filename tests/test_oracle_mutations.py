"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of ``oracle/dustin.py`` (a
dropped scale, a modulo head map, a sum where the definition takes a mean, a
wrong tie direction, an off-by-one window, ...), then runs the pins of
``tests/test_oracle_pins.py`` against that copy in a fresh interpreter.  A
case passes when at least one pin fails on the mutated oracle.  The unmutated
copy must pass every pin, so a broken harness cannot pass for a caught
mistake.  CPU only.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, [(text, replacement), ...]); each text occurs exactly once in oracle/dustin.py.
MUTATIONS = [
    ("score_target: no 1/sqrt(d) scale",
     [("out += softmax(scale * (K[:, g, :] @ q_hist[r]))", "out += softmax(K[:, g, :] @ q_hist[r])")]),
    ("score_target: scale 1/d",
     [("        scale = 1.0 / np.sqrt(d)\n    n = np.asarray(K_layers", "        scale = 1.0 / d\n    n = np.asarray(K_layers")]),
    ("score_target: keys of the first scored layer for every pair",
     [("K = _f64(K_layers[layer])", "K = _f64(K_layers[sub_heads[0][0]])")]),
    ("score_target: modulo head map",
     [("g = _kv_head_of(h, Hq, K.shape[1])", "g = h % K.shape[1]")]),
    ("score_draft: no 1/sqrt(d_d) scale",
     [("logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)  # [Gamma][n]\n            out += softmax(",
       "logits = q_draft[l, :, h, :] @ K[:, c, :].T  # [Gamma][n]\n            out += softmax(")]),
    ("score_draft: first draft step only (dropped Gamma sum)",
     [("out += softmax(logits, axis=-1).sum(axis=0)", "out += softmax(logits, axis=-1)[0]")]),
    ("score_draft: softmax over the draft steps instead of the history",
     [("out += softmax(logits, axis=-1).sum(axis=0)", "out += softmax(logits, axis=0).sum(axis=0)")]),
    ("grouped-query map: modulo instead of floor division",
     [("return h // (Hq // Hkv)", "return h % Hkv")]),
    ("head_probs: scale 1/d",
     [("        scale = 1.0 / np.sqrt(d)\n    P = np.empty", "        scale = 1.0 / d\n    P = np.empty")]),
    ("window_attention: head sum instead of mean",
     [("return head_probs(q, K, scale).mean(axis=0)", "return head_probs(q, K, scale).sum(axis=0)")]),
    ("dense_attention: modulo head map for V",
     [("O[:, h, :] = P[h] @ V[:, _kv_head_of(h, Hq, Hkv), :]", "O[:, h, :] = P[h] @ V[:, h % Hkv, :]")]),
    ("sparse_attention: LSE sign",
     [("lse[:, h] = (m + np.log(z))[:, 0]", "lse[:, h] = (m - np.log(z))[:, 0]")]),
    ("sparse_attention: padding entries kept",
     [("    I = I[I >= 0]\n    q = _f64(q)\n    w, Hq, d = q.shape\n    Ks", "    q = _f64(q)\n    w, Hq, d = q.shape\n    Ks")]),
    ("verify_attention: window not causal",
     [("keys = np.concatenate([Kh[:, g, :], Kw[: s + 1, g, :]], axis=0)",
       "keys = np.concatenate([Kh[:, g, :], Kw[:, g, :]], axis=0)"),
      ("vals = np.concatenate([Vh[:, g, :], Vw[: s + 1, g, :]], axis=0)",
       "vals = np.concatenate([Vh[:, g, :], Vw[:, g, :]], axis=0)")]),
    ("append_window_kv: rows shifted by one",
     [("            K[n + t] = K_win[t]\n            V[n + t] = V_win[t]",
       "            K[n + t - 1] = K_win[t]\n            V[n + t - 1] = V_win[t]")]),
    ("commit_window: accepted count not clamped to w",
     [("return n + min(max(int(accepted), 0), w)", "return n + max(int(accepted), 0)")]),
    ("arr_window: sum over steps instead of mean",
     [("return float(np.mean(arr_step(A, I)))", "return float(np.sum(arr_step(A, I)))")]),
    ("topk_desc: ties to the higher position",
     [("order = np.lexsort((candidates, -scores[candidates]))", "order = np.lexsort((-candidates, -scores[candidates]))")]),
    ("sd_oracle: first window step instead of the window mean",
     [("    Abar = _f64(A).mean(axis=0)\n    sel = np.sort(topk_desc(Abar, k))", "    Abar = _f64(A)[0]\n    sel = np.sort(topk_desc(Abar, k))")]),
    ("protected_positions: recent window one short",
     [("recent = np.arange(max(0, n - n_window), n)", "recent = np.arange(max(0, n - n_window + 1), n)")]),
    ("select_verify_set: draft tier ranked by S_Target",
     [("D = topk_desc(s_draft, m_eff, rest)", "D = topk_desc(s_target, m_eff, rest)")]),
    ("select_verify_set: draft share not capped by the budget",
     [("m_eff = max(0, min(m_eff, budget, rest.size))", "m_eff = max(0, min(m_eff, rest.size))")]),
    ("select_verify_set: missing S_Target leaves the draft tier at m",
     [("    elif s_target is None:\n        m_eff = budget", "    elif s_target is None:\n        m_eff = m")]),
    ("history_policy: lowest attention kept",
     [("return np.sort(topk_desc(A_past, k))", "return np.sort(topk_desc(-_f64(A_past), k))")]),
    ("policy_sweep: Dustin-D with no draft share",
     [("ms = (0, k - n_sink - n_window, m_hybrid[ki])", "ms = (0, 0, m_hybrid[ki])")]),
    ("search_objective: first layer only",
     [("return float(np.mean([arr_window(A, I) for A in A_layers]))", "return float(arr_window(A_layers[0], I))")]),
    ("search_objective: layer sum instead of mean",
     [("return float(np.mean([arr_window(A, I) for A in A_layers]))", "return float(np.sum([arr_window(A, I) for A in A_layers]))")]),
    ("candidate_objectives: base vector dropped",
     [("            v = v + _f64(base[b] if batch else base)", "            v = v + 0.0")]),
    ("candidate_objectives: per-candidate m ignored",
     [("mm = m if ms is None else ms[c]", "mm = m")]),
    ("candidate_objectives: first batch element only",
     [("tot += search_objective(A_layers[b] if batch else A_layers, I)",
       "tot += search_objective(A_layers[0] if batch else A_layers, I)")]),
    ("srh_head_scores: batch units in (head, layer) order",
     [("units = head_prev.transpose(1, 2, 0, 3).reshape(L * H, Bn, n)",
       "units = head_prev.transpose(2, 1, 0, 3).reshape(L * H, Bn, n)")]),
    ("srh_select: pairs in descending order",
     [("order = np.sort(topk_desc(M.ravel(), T))", "order = np.sort(topk_desc(M.ravel(), T))[::-1]")]),
    ("greedy_select: stops only when the objective falls",
     [("if top_c < 0 or not top_v > best:", "if top_c < 0 or not top_v >= best:")]),
    ("greedy_draft: no start value (a useless draft layer is kept)",
     [("return greedy_select(obj, units_d.shape[0], max_units, start=start)",
       "return greedy_select(obj, units_d.shape[0], max_units)")]),
    ("candidate_objectives: batch sum instead of mean",
     [("out[c] = tot / B", "out[c] = tot")]),
    ("srh_select: transposed (layer, head) index",
     [("return [(int(i) // H, int(i) % H) for i in order]", "return [(int(i) % L, int(i) // L) for i in order]")]),
    ("greedy_select: ties to the higher candidate",
     [("            if v > top_v:", "            if v >= top_v:")]),
    ("greedy_select: no stop rule",
     [("if top_c < 0 or not top_v > best:", "if top_c < 0:")]),
    ("m_search: ties to the last grid entry",
     [("return vals, int(ms[int(np.argmax(vals))])", "return vals, int(ms[len(vals) - 1 - int(np.argmax(vals[::-1]))])")]),
    ("page_key_bounds: positions past n included",
     [("K = _f64(K)[:n]\n    npg", "K = _f64(K)\n    npg"),
      ("blk = K[p * page:min(n, (p + 1) * page)]", "blk = K[p * page:(p + 1) * page]")]),
    ("page_scores: upper face only",
     [("np.maximum(kmin[:, g, :] * qq, kmax[:, g, :] * qq)", "(kmax[:, g, :] * qq)")]),
    ("draft_row_lse: no 1/sqrt(d_d) scale",
     [("            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            m = logits.max",
       "            logits = (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            m = logits.max")]),
    ("draft_row_lse: modulo head map",
     [("            c = _kv_head_of(h, H_d, K.shape[1])\n            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            m = logits.max",
       "            c = h % K.shape[1]\n            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            m = logits.max")]),
    ("score_draft_given_lse: no 1/sqrt(d_d) scale",
     [("            logits = scale * (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            out += np.exp(",
       "            logits = (q_draft[l, :, h, :] @ K[:, c, :].T)   # [Gamma][n]\n            out += np.exp(")]),
    ("draft_row_lse: max left out of the log-sum-exp",
     [("out[l, :, h] = (m + np.log(np.exp(logits - m)", "out[l, :, h] = (np.log(np.exp(logits - m)")]),
    ("score_draft_given_lse: normaliser of step 0 for every step",
     [("out += np.exp(logits - lse[l, :, h][:, None]).sum(axis=0)",
       "out += np.exp(logits - lse[l, 0, h]).sum(axis=0)")]),
    ("score_draft_given_lse: normaliser added instead of subtracted",
     [("out += np.exp(logits - lse[l, :, h][:, None]).sum(axis=0)",
       "out += np.exp(logits + lse[l, :, h][:, None]).sum(axis=0)")]),
    ("pages_to_contiguous: page table ignored",
     [("rows = [pool[int(page_row[p])] for p in range(n_pages)]", "rows = [pool[p] for p in range(n_pages)]")]),
]


def _tree(tmp, subs):
    """A copy of the oracle (mutated), the generator and the pins under tmp."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(tmp, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(tmp, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(tmp, "pytest.ini"))
    path = os.path.join(tmp, "oracle", "dustin.py")
    src = open(path).read()
    for old, new in subs:
        assert src.count(old) == 1, f"mutation text not found exactly once: {old!r}"
        src = src.replace(old, new)
    with open(path, "w") as f:
        f.write(src)


def _run_pins(subs):
    with tempfile.TemporaryDirectory() as tmp:
        _tree(tmp, subs)
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
        env.pop("PYTHONPATH", None)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "tests/test_oracle_pins.py"], cwd=tmp, env=env, capture_output=True, text=True,
                           timeout=600)
        return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def outcomes():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        futs = {name: ex.submit(_run_pins, subs) for name, subs in [("unmutated", [])] + MUTATIONS}
        return {name: f.result() for name, f in futs.items()}


def test_unmutated_copy_passes_every_pin(outcomes):
    rc, out = outcomes["unmutated"]
    assert rc == 0, out[-3000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(outcomes, name):
    rc, out = outcomes[name]
    # exit status 1 = tests ran and at least one failed (not a collection or usage error)
    assert rc == 1 and " failed" in out, f"no pin caught '{name}':\n{out[-3000:]}"
