"""Planted mistakes in the oracle (on the CPU) must each be caught by some pin.

Each mutant replaces one oracle function with a plausibly wrong variant (a dropped term, a
wrong sign, a wrong index, a transposed or reversed operand, a wrong tie rule...).  The
test asserts that at least one pin of tests/test_oracle_pins.py fails under it, which is
the evidence that the pins constrain every step of the oracle.
"""
import math

import numpy as np
import pytest

import oracle.jet_oracle as jom
from tests import test_oracle_pins as pins


def _lse_no_shift(z):
    return np.log(np.exp(z).sum(axis=1))


def _lse_sign(z):
    m = z.max(axis=1, keepdims=True)
    return m[:, 0] - np.log(np.exp(z - m).sum(axis=1))


def _lse_drop_max(z):
    m = z.max(axis=1, keepdims=True)
    return np.log(np.exp(z - m).sum(axis=1))


def _lse_partial_vocab(z):
    z = z[:, :-1]
    m = z.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(z - m).sum(axis=1))


def _logp_sign(zt, lse):
    return lse - zt


def _logits_reversed_vocab(H, W):
    return (H @ W.T)[:, ::-1]


def _logits_transposed(H, W):
    n = min(H.shape[1], W.shape[0])
    return H[:, :n] @ W[:n, :n].T if H.shape[0] else H @ W.T


def _scores_mean(tok_logp, off):
    n = len(off) - 1
    return np.array([float(np.mean(tok_logp[off[c]:off[c + 1]])) for c in range(n)])


def _scores_drop_last(tok_logp, off):
    n = len(off) - 1
    return np.array([float(np.sum(tok_logp[off[c]:max(off[c], off[c + 1] - 1)])) for c in range(n)])


_orig_decide_question = jom.decide_question


def _decide_T_times(s, T, *a, **k):
    return _orig_decide_question(np.asarray(s) * float(T) * float(T), T, *a, **k)


def _decide_last_tie(s, T, *a, **k):
    r = _orig_decide_question(s, T, *a, **k)
    a = np.asarray(s, np.float64) / T
    r["argmax"] = int(np.flatnonzero(a == a.max())[-1])
    return r


def _decide_on_float32(s, T, *a, **k):
    r = _orig_decide_question(s, T, *a, **k)
    a32 = (np.asarray(s, np.float64) / T).astype(np.float32)
    r["argmax"] = int(np.flatnonzero(a32 == a32.max())[0])
    return r


def _decide_levels_from_one(s, T, *a, **k):
    r = _orig_decide_question(s, T, *a, **k)
    r["expect"] = float(np.sum(np.arange(1, len(s) + 1) * r["q"]))
    return r


def _decide_gold_first_only(s, T, text_id=None, gold_text=None, true_idx=None):
    r = _orig_decide_question(s, T, text_id, gold_text, true_idx)
    if text_id is not None and gold_text is not None:
        g = np.flatnonzero(np.asarray(text_id) == gold_text)
        r["nll"] = math.inf if len(g) == 0 else -math.log(r["q"][g[0]])
    return r


def _decide_true_first(s, T, text_id=None, gold_text=None, true_idx=None):
    r = _orig_decide_question(s, T, text_id, gold_text, true_idx)
    if true_idx is None and len(s) == 2:
        r["q_true"] = float(r["q"][0])
    return r


def _decide_no_temperature(s, T, *a, **k):
    return _orig_decide_question(s, 1.0, *a, **k)


def _widen_bad_shift(a, dtype):
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _union_unsorted(ids, off, V):
    u, su = np.unique(np.asarray(ids)), None
    u = u[::-1].copy()
    su = np.array([int(np.flatnonzero(u == x)[0]) for x in ids], dtype=np.int32)
    return u.astype(np.int32), su


def _conf_unnormalised(q):
    q = np.asarray(q, np.float64)
    nz = q[q > 0]
    return 1.0 + float(np.sum(nz * np.log(nz)))


def _conf_bits_not_normalised(q):
    q = np.asarray(q, np.float64)
    nz = q[q > 0]
    return 1.0 + float(np.sum(nz * np.log2(nz)))


def _conf_entropy_itself(q):
    q = np.asarray(q, np.float64)
    if len(q) == 1:
        return 0.0
    nz = q[q > 0]
    return -float(np.sum(nz * np.log(nz))) / math.log(len(q))


def _mass_tempered(s):
    return float(np.sum(np.exp(np.asarray(s, np.float64) / 2.0)))


def _mass_best_only(s):
    return float(np.exp(np.max(np.asarray(s, np.float64))))


def _trie_token_only_key(tok_target, cand_tok_off, q_cand_off):
    """Child keyed by (question, token): forgets the parent history."""
    co, qo = list(cand_tok_off), list(q_cand_off)
    tok_node, node_tok, number = [-1] * len(tok_target), [], {}
    for g in range(len(qo) - 1):
        for c in range(qo[g], qo[g + 1]):
            v = ("root", g)
            for k in range(co[c], co[c + 1]):
                if v not in number:
                    number[v] = len(node_tok)
                    node_tok.append(k)
                tok_node[k] = number[v]
                v = (g, int(tok_target[k]))
    return np.array(tok_node), np.array(node_tok)


def _trie_shared_root(tok_target, cand_tok_off, q_cand_off):
    """One root for every question."""
    n_cand = len(cand_tok_off) - 1
    return _orig_trie(tok_target, cand_tok_off, np.array([0, n_cand]))


_orig_trie = jom.predictor_trie


def _trie_node_of_own_token(tok_target, cand_tok_off, q_cand_off):
    """Token mapped to the node its own token creates, not to its preceding history."""
    tn, nt = _orig_trie(tok_target, cand_tok_off, q_cand_off)
    co = np.asarray(cand_tok_off)
    out = tn.copy()
    for c in range(len(co) - 1):
        out[co[c]:co[c + 1] - 1] = tn[co[c] + 1:co[c + 1]]
    return out, nt


def _sens_variant(center=True, ddof=0, floor=True, reduce="mean"):
    def f(z, z_skip, seg_off, eps=1e-8):
        z = np.asarray(z, np.float64)
        zs = np.asarray(z_skip, np.float64).reshape(-1, len(z))
        off = [int(o) for o in seg_off]
        d = np.empty((zs.shape[0], len(off) - 1))
        for x in range(len(off) - 1):
            a, b = off[x], off[x + 1]
            zx = z[a:b]
            c = (lambda v: v - v.mean()) if center else (lambda v: v)
            rms = lambda v: math.sqrt(float(np.sum(v * v)) / max(len(v) - ddof, 1))  # noqa: E731
            den = max(eps, rms(c(zx))) if floor else rms(c(zx))
            for l in range(zs.shape[0]):
                with np.errstate(all="ignore"):
                    d[l, x] = rms(c(zs[l, a:b] - zx)) / den if den else math.inf
        return d, (d.mean(axis=1) if reduce == "mean" else d.sum(axis=1))
    return f


def _select_ties_high(J, k):
    order = sorted(range(len(J)), key=lambda l: (J[l], -l))
    return np.array(order[:k], dtype=np.int64)


def _select_largest(J, k):
    order = sorted(range(len(J)), key=lambda l: (-J[l], l))
    return np.array(order[:k], dtype=np.int64)


_orig_nll = jom.mean_gold_nll


def _nll_first_gold_only(s, q_cand_off, cand_text_id, q_gold_text_id, T, _mat=None):
    S, G = _mat if _mat is not None else jom._labelled_matrix(s, q_cand_off, cand_text_id, q_gold_text_id)
    first = G & (np.cumsum(G, axis=1) == 1)
    return _orig_nll(None, None, None, None, T, _mat=(S, first))


def _nll_T_multiplies(s, q_cand_off, cand_text_id, q_gold_text_id, T, _mat=None):
    return _orig_nll(s, q_cand_off, cand_text_id, q_gold_text_id, 1.0 / T, _mat=_mat)


def _nll_counts_unlabelled(s, q_cand_off, cand_text_id, q_gold_text_id, T, _mat=None):
    v, n = _orig_nll(s, q_cand_off, cand_text_id, q_gold_text_id, T, _mat=_mat)
    if _mat is not None or q_gold_text_id is None:
        return v, n
    tot = len(q_gold_text_id)
    return v * n / tot, tot


def _fit_grid_only(s, q_cand_off, cand_text_id, q_gold_text_id, T_min=1e-2, T_max=1e2):
    mat = jom._labelled_matrix(s, q_cand_off, cand_text_id, q_gold_text_id)
    grid = np.linspace(math.log(T_min), math.log(T_max), 801)
    vals = [_orig_nll(None, None, None, None, math.exp(u), _mat=mat)[0] for u in grid]
    i = int(np.argmin(vals))
    return math.exp(grid[i]), float(vals[i])


def _restricted_variant(kind):
    """score_restricted with one planted mistake: 'field_as_row' scores field f from row f
    (ignoring field_row), 'no_temperature' drops T, 'union_softmax' normalises each field
    over the whole union of allowed ids instead of its own slots."""
    def fn(rp):
        fo = np.asarray(rp["field_off"])
        ids = np.asarray(rp["field_ids"], dtype=np.int64)
        rows = np.asarray(rp["field_row"], dtype=np.int64)
        H64 = jom.widen(rp["H"], rp["h_dtype"])
        W64 = jom.widen(np.asarray(rp["W"])[ids], rp["w_dtype"])
        n_f = len(fo) - 1
        logit, qv = np.empty(len(ids)), np.empty(len(ids))
        am, gap = np.empty(n_f, dtype=np.int64), np.empty(n_f)
        uni = np.unique(ids)
        for f in range(n_f):
            a0, a1 = int(fo[f]), int(fo[f + 1])
            r_f = f % H64.shape[0] if kind == "field_as_row" else rows[f]
            b = W64[a0:a1] @ H64[r_f]
            logit[a0:a1] = b
            T = 1.0 if kind == "no_temperature" else rp["T"]
            r = jom.decide_question(b, T)
            q = r["q"]
            if kind == "union_softmax":
                allz = jom.widen(np.asarray(rp["W"])[uni], rp["w_dtype"]) @ H64[r_f] / T
                q = np.exp(b / T - allz.max()) / np.exp(allz - allz.max()).sum()
            qv[a0:a1] = q
            am[f] = r["argmax"]
            gap[f] = r["gap"]
        return dict(slot_logit=logit, slot_q=qv, field_argmax=am, field_gap=gap)
    return fn


MUTANTS = {
    "restricted_field_index_as_row": ("score_restricted", _restricted_variant("field_as_row")),
    "restricted_temperature_dropped": ("score_restricted", _restricted_variant("no_temperature")),
    "restricted_softmax_over_union": ("score_restricted", _restricted_variant("union_softmax")),
    "lse_without_max_shift": ("logsumexp_rows", _lse_no_shift),
    "lse_sign_error": ("logsumexp_rows", _lse_sign),
    "lse_dropped_max_term": ("logsumexp_rows", _lse_drop_max),
    "lse_missing_vocab_entry": ("logsumexp_rows", _lse_partial_vocab),
    "logprob_sign_flip": ("token_logprobs", _logp_sign),
    "logits_reversed_vocab_index": ("logits", _logits_reversed_vocab),
    "logits_transposed_operand": ("logits", _logits_transposed),
    "length_normalised_scores": ("candidate_scores", _scores_mean),
    "scores_drop_last_token": ("candidate_scores", _scores_drop_last),
    "temperature_multiplies": ("decide_question", _decide_T_times),
    "temperature_ignored": ("decide_question", _decide_no_temperature),
    "tie_goes_to_last": ("decide_question", _decide_last_tie),
    "decision_on_float32_scores": ("decide_question", _decide_on_float32),
    "ordinal_levels_from_one": ("decide_question", _decide_levels_from_one),
    "gold_nll_not_summed": ("decide_question", _decide_gold_first_only),
    "binary_true_is_first": ("decide_question", _decide_true_first),
    "bf16_widen_wrong_shift": ("widen", _widen_bad_shift),
    "union_not_sorted": ("build_union", _union_unsorted),
    "confidence_entropy_not_normalised": ("confidence", _conf_unnormalised),
    "confidence_entropy_in_bits": ("confidence", _conf_bits_not_normalised),
    "confidence_is_the_entropy": ("confidence", _conf_entropy_itself),
    "mass_with_temperature": ("allowed_mass", _mass_tempered),
    "mass_of_best_candidate_only": ("allowed_mass", _mass_best_only),
    "trie_forgets_parent": ("predictor_trie", _trie_token_only_key),
    "trie_one_root_for_all_questions": ("predictor_trie", _trie_shared_root),
    "trie_token_uses_its_own_node": ("predictor_trie", _trie_node_of_own_token),
    "sensitivity_not_centred": ("decision_sensitivity", _sens_variant(center=False)),
    "sensitivity_sample_std": ("decision_sensitivity", _sens_variant(ddof=1)),
    "sensitivity_no_eps_floor": ("decision_sensitivity", _sens_variant(floor=False)),
    "sensitivity_J_summed": ("decision_sensitivity", _sens_variant(reduce="sum")),
    "selection_ties_to_higher_layer": ("select_layers", _select_ties_high),
    "selection_of_largest_scores": ("select_layers", _select_largest),
    "nll_first_gold_only": ("mean_gold_nll", _nll_first_gold_only),
    "nll_temperature_multiplies": ("mean_gold_nll", _nll_T_multiplies),
    "nll_counts_unlabelled_questions": ("mean_gold_nll", _nll_counts_unlabelled),
    "fit_without_refinement": ("fit_temperature", _fit_grid_only),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(jom, attr, fn)
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # any failure (assertion, shape error, overflow) counts
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake {name}"
