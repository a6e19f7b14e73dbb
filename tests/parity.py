"""Comparison of HIP outputs with the fp64 oracle at the stated tolerances.

Tolerances (per token l and per row LSE: 1e-4 with an fp32 head, 2e-3 with a bf16 head
evaluated by the oracle on the same bf16 bits; q: 1e-4) and the ones derived from them:
  s(c)      m_c * tol_l            (a sum of m_c token log-probabilities)
  q(true)   1e-4                   (an entry of q)
  E         1e-4 * K (K - 1) / 2   (sum_i i q_i with each q_i within 1e-4)
  gold NLL  2 * m_max * tol_l / T  (difference of two log-sum-exps of s / T)
  mass      relative m_max * tol_l (sum_c exp s(c))
  confidence  2 m_max tol_l / T + 1e-5 (first-order bound through the entropy)
Decisions (check_decisions), for every question:
  * the kernel's own tie rule: its decision is the lowest index among the exact maxima of
    its own a = float32(s) / T (the kernel divides with correct rounding, as numpy does),
    so candidates with bitwise-equal scores always go to the first;
  * outside the near-tie band (the oracle's top-two gap in q above 1e-4) the decision
    equals the oracle's, which is taken on the exact fp64 scores;
  * inside the band the decision is one of the oracle's near-maximal candidates: its
    oracle q is within 1e-4 of the largest.
"""
from __future__ import annotations

import sys

import numpy as np

Q_TOL = 1e-4


def tol_logp(p) -> float:
    return 1e-4 if p["w_dtype"] == "f32" else 2e-3


def _maxerr(a, b, mask=None):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_nan | same_inf, 0.0, np.abs(a - b))
    err = np.where(np.isnan(err), np.inf, err)
    if mask is not None:
        err = err[mask]
    return float(err.max()) if err.size else 0.0


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def check_decisions(argmax, s_out, off, T, ref_argmax, ref_gap, ref_q, name="", qmask=None) -> dict:
    """Assert the decision rules above for the groups [off[g], off[g+1]) (questions, or
    fields of the restricted path).  s_out: the kernel's fp32 scores (cand_s, or the
    restricted slot logits); qmask: groups the oracle computed (None: all).  Returns the
    number of groups decided outside the band and inside it."""
    a = np.asarray(s_out, np.float32) / np.float32(T)
    off = np.asarray(off)
    n_clear = n_band = 0
    for g in range(len(off) - 1):
        c0, c1 = int(off[g]), int(off[g + 1])
        ag = a[c0:c1]
        top = np.flatnonzero(ag == ag.max())
        assert top.size and int(argmax[g]) == int(top[0]), (name, "own tie rule", g, int(argmax[g]), top[:8])
        if qmask is not None and not qmask[g]:
            continue
        if ref_gap[g] > Q_TOL:
            n_clear += 1
            assert int(argmax[g]) == int(ref_argmax[g]), (name, "argmax", g, int(argmax[g]), int(ref_argmax[g]))
        else:
            n_band += 1
            qg = np.asarray(ref_q[c0:c1], np.float64)
            assert qg[int(argmax[g])] >= qg.max() - Q_TOL, (name, "near-tie decision", g, int(argmax[g]))
    return dict(argmax_checked=n_clear, argmax_in_band=n_band)


def compare(p: dict, out: dict, ref: dict, name: str = "", sampled: bool = False) -> dict:
    """Assert every output of `out` (numpy) against the oracle `ref`; return observed errors.

    sampled: the oracle computed only some rows; compare only where it is finite/defined."""
    tl = tol_logp(p)
    T = float(p["T"])
    co = np.asarray(p["cand_tok_off"])
    qo = np.asarray(p["q_cand_off"])
    m = np.diff(co)
    K = np.diff(qo)
    m_max_q = np.array([m[qo[g]:qo[g + 1]].max() for g in range(len(K))]) if len(K) else np.zeros(0)
    errs = {}
    assert int(out["dev_flags"][0]) == 0, f"{name}: device flags {out['dev_flags'][0]}"
    tok_mask = ~np.isnan(ref["tok_logp"]) if sampled else None
    errs["tok_logp"] = _maxerr(out["tok_logp"], ref["tok_logp"], tok_mask)
    assert errs["tok_logp"] <= tl, (name, "tok_logp", errs["tok_logp"], tl)
    if "row_lse" in out:
        rmask = ~np.isnan(ref["lse"]) if sampled else None
        errs["row_lse"] = _maxerr(out["row_lse"], ref["lse"], rmask)
        assert errs["row_lse"] <= tl, (name, "row_lse", errs["row_lse"])
    cmask = ~np.isnan(ref["cand_s"]) if sampled else np.ones(len(m), bool)
    ds = np.abs(out["cand_s"].astype(np.float64) - ref["cand_s"])
    assert np.all(ds[cmask] <= m[cmask] * tl), (name, "cand_s", float(ds[cmask].max()))
    errs["cand_s"] = float(ds[cmask].max()) if cmask.any() else 0.0
    errs["cand_q"] = _maxerr(out["cand_q"], ref["cand_q"], cmask)
    assert errs["cand_q"] <= Q_TOL, (name, "cand_q", errs["cand_q"])
    qmask = ~np.isnan(ref["q_expect"]) if sampled else np.ones(len(K), bool)
    errs.update(check_decisions(out["q_argmax"], out["cand_s"], qo, T, ref["q_argmax"],
                                ref["q_gap"], ref["cand_q"], name, qmask))
    if "q_true" in out:
        errs["q_true"] = _maxerr(out["q_true"], ref["q_true"], qmask)
        assert errs["q_true"] <= Q_TOL, (name, "q_true", errs["q_true"])
    if "q_expect" in out:
        de = np.abs(out["q_expect"] - ref["q_expect"])
        lim = Q_TOL * K * (K - 1) / 2 + 1e-6
        assert np.all(de[qmask] <= lim[qmask]), (name, "q_expect", float(de[qmask].max()))
        errs["q_expect"] = float(de[qmask].max()) if qmask.any() else 0.0
    if "q_gold_nll" in out and p.get("cand_text_id") is not None:
        a, b = out["q_gold_nll"].astype(np.float64), ref["q_nll"]
        inf_ok = np.isinf(a) == np.isinf(b)
        assert np.all(inf_ok[qmask]), (name, "nll inf pattern")
        fin = qmask & np.isfinite(b)
        dn = np.abs(a - b)
        assert np.all(dn[fin] <= 2 * m_max_q[fin] * tl / T), (name, "nll", float(dn[fin].max()))
        errs["q_gold_nll"] = float(dn[fin].max()) if fin.any() else 0.0
    if "q_mass" in out:
        # exp of scores each within m_c * tol_l: relative error m_max * tol_l (fp32 range only)
        mass_ref = ref["q_mass"]
        rel = np.abs(out["q_mass"] - mass_ref) / np.maximum(mass_ref, 1e-300)
        ok = qmask & (mass_ref > 1e-30)
        assert np.all(rel[ok] <= m_max_q[ok] * tl + 1e-5), (name, "q_mass", float(rel[ok].max()))
        errs["q_mass_rel"] = float(rel[ok].max()) if ok.any() else 0.0
    if "q_confidence" in out:
        # scores a_c within eps = m_max tol_l / T move each q_c by at most 2 eps q_c, so the
        # entropy by at most 2 eps H <= 2 eps ln K: |d confidence| <= 2 eps (+ fp32 rounding)
        dc = np.abs(out["q_confidence"].astype(np.float64) - ref["q_confidence"])
        tol_c = 2.0 * m_max_q * tl / T + 1e-5
        assert np.all(dc[qmask] <= tol_c[qmask]), (name, "q_confidence", float(dc[qmask].max()))
        one = qmask & (K == 1)
        assert np.all(out["q_confidence"][one] == 1.0), (name, "confidence of a single choice")
        errs["q_confidence"] = float(dc[qmask].max()) if qmask.any() else 0.0
    return errs
