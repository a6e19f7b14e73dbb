"""Pins for the fp64 oracle: values and identities fixed by the pages and by mathematics.

Each pin is a plain function (so tests/test_oracle_mutants.py can re-run them against
oracles with planted mistakes).  None of them re-types the oracle's formulas: they use the
pages' worked example, closed forms, invariances, and an exact-summation brute force
written in pure Python (math.fsum, struct) for tiny vocabularies.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle as jo
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------
# helpers independent of the oracle
# ----------------------------------------------------------------------------------------

def _bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _operand(a, dtype):
    a = np.asarray(a)
    if dtype == "f32":
        return [[float(x) for x in row] for row in a]
    return [[_bf16_to_float(x) for x in row] for row in a]


def brute_force(p: dict) -> dict:
    """Direct evaluation of the definitions with exact summation, no max shift.

    Valid only for tiny vocabularies with moderate logits (no overflow of exp)."""
    H = _operand(p["H"], p["h_dtype"])
    W = _operand(p["W"], p["w_dtype"])
    V = len(W)
    n_tok = len(p["tok_target"])
    tok_row = list(range(n_tok)) if p.get("tok_row") is None else [int(r) for r in p["tok_row"]]
    z = [[math.fsum(h * w for h, w in zip(H[r], W[v])) for v in range(V)] for r in range(len(H))]
    lse = [math.log(math.fsum(math.exp(x) for x in row)) for row in z]
    ell = [z[tok_row[k]][int(p["tok_target"][k])] - lse[tok_row[k]] for k in range(n_tok)]
    co = [int(x) for x in p["cand_tok_off"]]
    s = [math.fsum(ell[co[c]:co[c + 1]]) for c in range(len(co) - 1)]
    qo = [int(x) for x in p["q_cand_off"]]
    T = float(p["T"])
    out = dict(lse=lse, tok_logp=ell, cand_s=s, cand_q=[], q_argmax=[], q_true=[], q_expect=[], q_nll=[])
    for g in range(len(qo) - 1):
        a = [s[c] / T for c in range(qo[g], qo[g + 1])]
        e = [math.exp(x) for x in a]
        Z = math.fsum(e)
        q = [x / Z for x in e]
        out["cand_q"] += q
        best = max(a)
        out["q_argmax"].append(a.index(best))  # list.index: the first (lowest) maximum
        K = len(a)
        t = (1 if K == 2 else -1) if p.get("q_true_idx") is None else int(p["q_true_idx"][g])
        out["q_true"].append(q[t] if 0 <= t < K else math.nan)
        out["q_expect"].append(math.fsum(i * q[i] for i in range(K)))
        if p.get("cand_text_id") is None or p.get("q_gold_text_id") is None:
            out["q_nll"].append(math.nan)
        else:
            gold = int(p["q_gold_text_id"][g])
            mass = math.fsum(q[i] for i in range(K) if int(p["cand_text_id"][qo[g] + i]) == gold)
            out["q_nll"].append(-math.log(mass) if mass > 0 else math.inf)
    return out


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))) | (np.isnan(a) & np.isnan(b))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(err <= tol), f"{what}: max err {np.nanmax(err)} > {tol}"


def _tiny_problem(seed, layout="prefix", V=37, d=8, n_q=3, K=(1, 5), lengths=(1, 4), T=1.0,
                  dups=1, h="f32", w="f32"):
    return wl.make_problem(V=V, d=d, n_q=n_q, K=K, lengths=lengths, layout=layout, h_dtype=h,
                           w_dtype=w, T=T, seed=seed, dups=dups, n_extra_rows=2 if layout != "own" else 0)


def _onehot_problem(log_rows, cands, T=1.0, text=None, gold=None, true_idx=None):
    """H row r = e_r and W[v, r] = log_rows[r][v], so that z[r, v] = log_rows[r][v] (f32)."""
    R = len(log_rows)
    V = len(log_rows[0])
    H = np.eye(R, dtype=np.float32)
    W = np.array(log_rows, dtype=np.float32).T.copy()
    tok_row, tok_target, off = [], [], [0]
    for rows, tg in cands:
        tok_row += rows
        tok_target += tg
        off.append(len(tok_row))
    n = len(cands)
    return dict(name="onehot", V=V, d=R, n_rows=R, H=H, h_dtype="f32", W=W, w_dtype="f32",
                tok_row=np.array(tok_row, np.int32), tok_target=np.array(tok_target, np.int32),
                cand_tok_off=np.array(off, np.int32), q_cand_off=np.array([0, n], np.int32),
                cand_text_id=None if text is None else np.array(text, np.int32),
                q_gold_text_id=None if gold is None else np.array([gold], np.int32),
                q_true_idx=None if true_idx is None else np.array([true_idx], np.int32), T=T)


# ----------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------

def pin_worked_example():
    """JET, Eq. 4 and its example: likelihoods 0.06 and 0.02 normalise to 0.75 and 0.25.

    Candidate 0 has two tokens with probabilities 0.3 (prefix row) and 0.2 (its own row),
    so its likelihood is the chain-rule product 0.06; candidate 1 has one token of
    probability 0.02 from the prefix row.  Logits are log-probabilities, rounded to f32."""
    g = json.load(open(os.path.join(GOLDEN, "jet_worked_example.json")))
    p_prefix = [0.3, 0.02, 0.5, 0.18]
    p_row1 = [0.2, 0.3, 0.25, 0.25]
    prob = _onehot_problem([np.log(p_prefix), np.log(p_row1)],
                           [([0, 1], [0, 0]), ([0], [1])])
    r = jo.score(prob)
    _close(np.exp(r["cand_s"]), g["candidate_likelihoods"], 2e-8, "likelihoods")
    _close(r["cand_q"], g["normalized"], 1e-7, "normalised")
    assert r["q_argmax"][0] == 0


def pin_shift_invariance():
    """Adding a constant c to every logit of a row (H' = [H, 1], W' = [W, c]) leaves l, s and
    q unchanged (FastJEV Sec. 3.4: a common shift leaves softmax unchanged).  With c = 1000
    an evaluation without the max shift overflows, so this also pins the stable form."""
    p = _tiny_problem(11)
    base = jo.score(p)
    for c in (1000.0, -1000.0, 3.5):
        q = dict(p)
        q["H"] = np.concatenate([p["H"], np.ones((p["n_rows"], 1), np.float32)], axis=1)
        q["W"] = np.concatenate([p["W"], np.full((p["V"], 1), c, np.float32)], axis=1)
        q["d"] = p["d"] + 1
        r = jo.score(q)
        _close(r["tok_logp"], base["tok_logp"], 1e-9, f"l shift {c}")
        _close(r["cand_q"], base["cand_q"], 1e-12, f"q shift {c}")
        _close(r["lse"], base["lse"] + c, 1e-9, f"lse shift {c}")


def pin_brute_force():
    """Oracle vs direct exact-summation evaluation on tiny vocabularies, several layouts,
    temperatures, dtypes and duplicate candidates."""
    cases = [
        dict(seed=1, layout="prefix"), dict(seed=2, layout="own"), dict(seed=3, layout="field"),
        dict(seed=4, layout="prefix", T=0.5), dict(seed=5, layout="own", T=2.0, dups=2),
        dict(seed=6, layout="field", h="bf16", w="bf16"), dict(seed=7, layout="prefix", h="f32", w="bf16"),
        dict(seed=8, layout="own", V=64, d=16, K=(2, 2)),
    ]
    for cs in cases:
        p = _tiny_problem(**cs)
        r = jo.score(p)
        b = brute_force(p)
        _close(r["lse"], b["lse"], 1e-12, f"lse {cs}")
        _close(r["tok_logp"], b["tok_logp"], 1e-12, f"l {cs}")
        _close(r["cand_s"], b["cand_s"], 1e-11, f"s {cs}")
        _close(r["cand_q"], b["cand_q"], 1e-12, f"q {cs}")
        _close(r["q_true"], b["q_true"], 1e-12, f"q_true {cs}")
        _close(r["q_expect"], b["q_expect"], 1e-11, f"E {cs}")
        _close(r["q_nll"], b["q_nll"], 1e-10, f"nll {cs}")
        assert list(r["q_argmax"]) == b["q_argmax"], cs


def pin_zero_head_closed_form():
    """W = 0: every logit is 0, so LSE = ln V, l = -ln V, s(c) = -m_c ln V and
    q(c) is proportional to V^(-m_c / T)."""
    for T in (1.0, 0.7):
        p = _tiny_problem(21, V=1000, d=16, T=T)
        p["W"] = np.zeros_like(p["W"])
        r = jo.score(p)
        lnV = math.log(1000)
        _close(r["lse"], np.full(p["n_rows"], lnV), 1e-12, "lse")
        _close(r["tok_logp"], np.full(len(p["tok_target"]), -lnV), 1e-12, "l")
        m = np.diff(p["cand_tok_off"])
        _close(r["cand_s"], -m * lnV, 1e-11, "s")
        qo = p["q_cand_off"]
        for g in range(len(qo) - 1):
            mm = m[qo[g]:qo[g + 1]].astype(np.float64)
            w = 1000.0 ** (-(mm - mm.min()) / T)
            _close(r["cand_q"][qo[g]:qo[g + 1]], w / w.sum(), 1e-12, "q")


def pin_peaked_closed_form():
    """One logit a_r per row, zeros elsewhere: LSE_r = ln(V - 1 + e^{a_r}); the peaked
    target gets a_r - LSE_r, any other target -LSE_r.  H is one-hot, so z = a W[:, r]."""
    V = 500
    a = [3.0, -2.0, 10.0, 0.5, 30.0]
    peak = [7, 0, 499, 250, 123]
    rows = []
    for r in range(len(a)):
        row = np.zeros(V)
        row[peak[r]] = a[r]
        rows.append(row)
    cands = [([0], [7]), ([1], [1]), ([2, 3], [499, 250]), ([4, 0], [123, 8])]
    p = _onehot_problem(rows, cands, T=1.0)
    r = jo.score(p)
    lse = [math.log(V - 1 + math.exp(x)) for x in a]
    _close(r["lse"], lse, 1e-12, "lse")
    expect_l = [a[0] - lse[0], -lse[1], a[2] - lse[2], a[3] - lse[3], a[4] - lse[4], -lse[0]]
    _close(r["tok_logp"], expect_l, 1e-12, "l")
    _close(r["cand_s"], [expect_l[0], expect_l[1], expect_l[2] + expect_l[3], expect_l[4] + expect_l[5]], 1e-12, "s")
    z = jo.logits(np.eye(5)[2:3], np.array(rows).T.copy())
    _close(z[0], rows[2], 0.0, "one-hot logits")


def pin_single_token_rule():
    """Single-token candidates are scored from the prefix row alone (JET, hybrid execution:
    the prefix output supplies first-token probabilities; gemma-e2b doc: one vocabulary
    vector per single-token field): perturbing every other row leaves their s bitwise
    unchanged."""
    p = _tiny_problem(31, layout="prefix", lengths=(1, 3), n_q=4, K=(3, 6))
    base = jo.score(p)
    m = np.diff(p["cand_tok_off"])
    used_first = set(int(p["tok_row"][o]) for o in p["cand_tok_off"][:-1])
    q = dict(p)
    H = p["H"].copy()
    rng = np.random.default_rng(5)
    for r in range(p["n_rows"]):
        if r not in used_first:
            H[r] = rng.standard_normal(p["d"]).astype(np.float32)
    q["H"] = H
    r = jo.score(q)
    single = m == 1
    assert single.any()
    assert np.array_equal(r["cand_s"][single], base["cand_s"][single])


def pin_prefix_factoring():
    """A token prefix shared by all candidates (same row, same target) can move into the
    field prefix without changing q (gemma-e2b doc, "Candidate likelihoods")."""
    V, d = 41, 8
    rng = np.random.default_rng(3)
    H = rng.standard_normal((12, d)).astype(np.float32)
    W = (rng.standard_normal((V, d)) / math.sqrt(d)).astype(np.float32)
    shared = 17
    cands = [[(0, shared), (1, 3), (2, 9)], [(0, shared), (3, 4)], [(0, shared), (4, 30), (5, 2), (6, 6)]]

    def prob(cs):
        tr, tt, off = [], [], [0]
        for c in cs:
            tr += [x[0] for x in c]
            tt += [x[1] for x in c]
            off.append(len(tr))
        return dict(name="pf", V=V, d=d, n_rows=12, H=H, h_dtype="f32", W=W, w_dtype="f32",
                    tok_row=np.array(tr, np.int32), tok_target=np.array(tt, np.int32),
                    cand_tok_off=np.array(off, np.int32), q_cand_off=np.array([0, len(cs)], np.int32),
                    cand_text_id=None, q_gold_text_id=None, q_true_idx=None, T=1.3)

    full = jo.score(prob(cands))
    factored = jo.score(prob([c[1:] for c in cands]))
    _close(full["cand_q"], factored["cand_q"], 1e-12, "q")
    assert not np.allclose(full["cand_s"], factored["cand_s"])


def pin_duplication():
    """Duplicating candidate c* changes the distribution (JET, after Eq. 4): originals
    become q_c / (1 + q_c*), both copies get q_c* / (1 + q_c*), and the tie goes to the
    lower index (JET Eq. 5, fixed order; equal text gives equal likelihood)."""
    s = np.array([-3.0, -1.5, -2.2, -1.5001])
    base = jo.decide_question(s, 1.0)
    for cstar in range(4):
        s2 = np.concatenate([s[:cstar + 1], [s[cstar]], s[cstar + 1:]])
        r = jo.decide_question(s2, 1.0)
        expect = np.concatenate([base["q"][:cstar + 1], [base["q"][cstar]], base["q"][cstar + 1:]])
        _close(r["q"], expect / (1.0 + base["q"][cstar]), 1e-15, "dup q")
        if cstar == 1:
            assert r["argmax"] == 1
    r = jo.decide_question(np.array([-1.0, -0.5, -0.5, -2.0]), 1.0)
    assert r["argmax"] == 1


def pin_ordinal():
    """Ordinal rule (JET, decision rules): E = sum_{i=0}^{K-1} i q(i), possibly fractional."""
    with np.errstate(divide="ignore"):
        r = jo.decide_question(np.log(np.array([0.0, 0.0, 1.0, 0.0, 0.0])), 1.0)
        assert r["expect"] == 2.0
        r = jo.decide_question(np.log(np.array([0.5, 0.5, 0.0, 0.0, 0.0])), 1.0)
        assert r["expect"] == 0.5
        r = jo.decide_question(np.log(np.array([0.1, 0.2, 0.3, 0.4])), 1.0)
        assert abs(r["expect"] - 2.0) < 1e-15


def pin_binary():
    """Binary rule: C = {false, true} with default order [false, true]; q(true) is the
    second entry, the pair sums to one; an explicit order may put true first (nimble page:
    explicit boolean choices may reverse the order)."""
    s = np.array([-0.7, -2.1])
    r = jo.decide_question(s, 1.0)
    assert abs(r["q"][0] + r["q"][1] - 1.0) < 1e-15
    assert r["q_true"] == r["q"][1]
    assert abs(r["q_true"] - 1.0 / (1.0 + math.exp(-0.7 - (-2.1)))) < 1e-15
    r2 = jo.decide_question(s, 1.0, true_idx=0)
    assert r2["q_true"] == r["q"][0]
    assert math.isnan(jo.decide_question(np.array([0.0, 1.0, 2.0]), 1.0)["q_true"])


def pin_temperature():
    """Temperature scales candidate scores once before the softmax and does not change the
    argmax (nimble page, "V2 probability default"); T -> infinity gives the uniform
    distribution and T = 1 is the plain likelihood ratio of JET Eq. 4."""
    s = np.array([-5.0, -2.0, -2.5, -9.0, -2.01])
    am = jo.decide_question(s, 1.0)["argmax"]
    for T in (0.05, 0.5, 2.0, 2.179, 50.0):
        assert jo.decide_question(s, T)["argmax"] == am
    _close(jo.decide_question(s, 1e9)["q"], np.full(5, 0.2), 1e-8, "uniform")
    L = np.exp(s)
    _close(jo.decide_question(s, 1.0)["q"], L / L.sum(), 1e-15, "ratio")
    q2 = jo.decide_question(s, 2.0)["q"]
    _close(q2, np.sqrt(L) / np.sqrt(L).sum(), 1e-15, "T=2 is the square root")


def pin_exact_decision():
    """The decision is the lowest index among the exact maxima of a = s / T (JET Eq. 5 with
    ties resolved by a fixed ordering).  Scores 1e-12 apart are distinct: the larger wins
    even though both round to the same fp32 value; bitwise-equal scores tie and go to the
    first; a near tie after scaling is still decided by the exact values."""
    s = np.array([-1.0 - 1e-12, -1.0, -3.0])
    assert np.float32(s[0]) == np.float32(s[1])
    assert jo.decide_question(s, 1.0)["argmax"] == 1
    assert jo.decide_question(s, 0.3)["argmax"] == 1
    s = np.array([-2.0, -0.5, -0.5, -0.5 - 2.0 ** -40])
    assert jo.decide_question(s, 1.0)["argmax"] == 1
    assert jo.decide_question(s[::-1].copy(), 1.0)["argmax"] == 1  # now -0.5 at 1 and 2


def pin_gold_nll():
    """Gold NLL sums the probability of every label carrying the gold text (JET, labels
    vs answer text): NLL = -ln(q_a + q_b); +inf when the gold text is absent; 0 for K = 1."""
    s = np.array([-1.0, -2.0, -1.0, -3.0])
    text = np.array([5, 7, 5, 9])
    r = jo.decide_question(s, 1.0, text, 5)
    assert abs(r["nll"] + math.log(r["q"][0] + r["q"][2])) < 1e-14
    r = jo.decide_question(s, 1.0, text, 6)
    assert r["nll"] == math.inf
    r = jo.decide_question(np.array([-4.0]), 1.0, np.array([3]), 3)
    assert r["nll"] == 0.0 and r["q"][0] == 1.0 and r["argmax"] == 0 and r["expect"] == 0.0


def pin_restricted_equals_full():
    """For single-token fields the allowed-token softmax equals the full-vocabulary
    candidate softmax at the same T, because the row's full-vocabulary normaliser cancels
    (nimble page, Execution steps 5-6, against JET Eq. 1-4)."""
    for seed, mx in ((1, False), (2, True)):
        rp = wl.make_restricted(n_fields=6, V=300, d=32, K=(1, 9) if not mx else 9, T=2.0, seed=seed,
                                shared_rows=mx, n_rows=4 if mx else None)
        rr = jo.score_restricted(rp)
        full = jo.score(wl.restricted_as_full(rp))
        _close(rr["slot_q"], full["cand_q"], 1e-12, "q")
        assert np.array_equal(rr["field_argmax"], full["q_argmax"])
        tok_row = np.repeat(rp["field_row"], np.diff(rp["field_off"]))
        _close(rr["slot_logit"], full["tok_logp"] + full["lse"][tok_row], 1e-12, "logit")


def pin_lse_statistics():
    """For W ~ N(0, 1/d) and large V, z[r, .] ~ N(0, |h_r|^2 / d), so LSE_r is close to
    ln V + |h_r|^2 / (2 d) (moment generating function of the normal).  Loose check."""
    V, d = 20000, 64
    p = wl.make_problem(V=V, d=d, n_q=4, K=2, lengths=1, layout="field", w_dtype="f32", seed=9)
    r = jo.score(p)
    h = p["H"].astype(np.float64)
    pred = math.log(V) + (h * h).sum(1) / (2 * d)
    assert np.all(np.abs(r["lse"] - pred) < 0.05)


def pin_build_union():
    """The union is the sorted set of allowed ids; each slot's index points at its id."""
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 50, size=60).astype(np.int32)
    off = np.array([0, 10, 10 + 15, 60], np.int32)
    u, su = jo.build_union(ids, off, 50)
    assert list(u) == sorted(set(int(x) for x in ids))
    assert all(int(u[su[j]]) == int(ids[j]) for j in range(len(ids)))
    with pytest.raises(ValueError):
        jo.build_union(np.array([3, 50], np.int32), np.array([0, 2], np.int32), 50)


def pin_bf16_widening():
    """bf16 bits widen to the values the format defines (golden table)."""
    g = json.load(open(os.path.join(GOLDEN, "bf16_format.json")))
    bits = np.array([int(b, 16) for b, _ in g["bits_to_value"]], dtype=np.uint16)
    vals = jo.widen(bits, "bf16")
    assert list(vals) == [v for _, v in g["bits_to_value"]]


def pin_sampled_rows():
    """Sampled-row scoring agrees with the full evaluation on the sampled rows' tokens
    and marks everything else NaN."""
    p = _tiny_problem(41, layout="own", n_q=5)
    full = jo.score(p)
    rows = np.array([0, 1, 2, 3, 4, 5])
    r = jo.score(p, rows=rows)
    n_tok = len(p["tok_target"])
    tok_row = np.arange(n_tok) if p["tok_row"] is None else p["tok_row"]
    on = np.isin(tok_row, rows)
    assert on.any() and (~on).any()
    _close(r["tok_logp"][on], full["tok_logp"][on], 1e-13, "sampled l")
    assert np.all(np.isnan(r["tok_logp"][~on]))


def pin_confidence_and_mass():
    """Confidence = 1 - normalised entropy of q and allowed mass = full-vocabulary
    probability of the allowed choices (gemma-e2b doc, "Output contracts").

    JET's worked example: the two candidates' sequence likelihoods 0.06 and 0.02 give
    mass 0.08, and q = (3/4, 1/4) has binary entropy 2 - (3/4) log2 3 bits, so the
    confidence is (3/4) log2 3 - 1.  A zero head makes every single-token candidate
    probability 1/V (mass K / V, uniform q, confidence 0); one overwhelming candidate makes
    q one-hot (confidence 1); one choice is confidence 1; mass ignores the temperature."""
    g = json.load(open(os.path.join(GOLDEN, "jet_worked_example.json")))
    p_prefix = [0.3, 0.02, 0.5, 0.18]
    p_row1 = [0.2, 0.3, 0.25, 0.25]
    prob = _onehot_problem([np.log(p_prefix), np.log(p_row1)],
                           [([0, 1], [0, 0]), ([0], [1])])
    r = jo.score(prob)
    _close(r["q_mass"], [sum(g["candidate_likelihoods"])], 5e-8, "worked-example mass")
    _close(r["q_confidence"], [0.75 * math.log2(3.0) - 1.0], 1e-7, "worked-example confidence")
    # zero head, single-token candidates: uniform over the question
    p = _tiny_problem(23, V=1000, d=16, lengths=(1, 1), K=(2, 7))
    p["W"] = np.zeros_like(p["W"])
    r = jo.score(p)
    K = np.diff(p["q_cand_off"])
    _close(r["q_mass"], K / 1000.0, 1e-13, "zero-head mass K / V")
    _close(r["q_confidence"], np.zeros(len(K)), 1e-13, "uniform q: confidence 0")
    # one overwhelming candidate (score gap 5000 nats): q is exactly one-hot in fp64
    assert jo.decide_question(np.array([-3.0, -5003.0, -5010.0]), 1.0)["confidence"] == 1.0
    assert jo.decide_question(np.array([-3.0]), 1.0)["confidence"] == 1.0
    s = np.array([-1.5, -2.25, -0.75, -4.0])
    masses = {jo.decide_question(s, T)["mass"] for T in (0.5, 1.0, 2.0)}
    assert len(masses) == 1 and abs(masses.pop() - float(np.exp(s).sum())) < 1e-15
    # confidence does not depend on the order of the candidates
    c = jo.decide_question(s, 1.3)["confidence"]
    assert abs(jo.decide_question(s[::-1].copy(), 1.3)["confidence"] - c) < 1e-15


def _seq_arrays(questions):
    """CSR arrays for a list of questions, each a list of candidate token tuples."""
    tg, co, qo = [], [0], [0]
    for cands in questions:
        for seq in cands:
            tg.extend(seq)
            co.append(len(tg))
        qo.append(len(co) - 1)
    return np.array(tg), np.array(co), np.array(qo)


def pin_predictor_trie():
    """History-consistent merging (FastJEV Sec. 3.3, Eq. 4): a token's predictor is the node
    of its preceding history; nodes are keyed by (parent, token) from a per-question root,
    so equal tokens after different histories stay separate.

    Worked by hand: question 0 has candidates (a b c), (a b d), (a e), (f b d); question 1
    has (a b c).  Predictors: root0 for every first token; 'a' for b, b, e; 'ab' for c, d;
    'f' for b; 'fb' for d (not 'ab': its parent differs); question 1 repeats nothing of
    question 0.  Numbering follows first use."""
    a, b, c, d, e, f = 10, 20, 30, 40, 50, 60
    tg, co, qo = _seq_arrays([[(a, b, c), (a, b, d), (a, e), (f, b, d)], [(a, b, c)]])
    tok_node, node_tok = jo.predictor_trie(tg, co, qo)
    assert list(tok_node) == [0, 1, 2, 0, 1, 2, 0, 1, 0, 3, 4, 5, 6, 7], list(tok_node)
    assert list(node_tok) == [0, 1, 2, 9, 10, 11, 12, 13], list(node_tok)
    # brute force against the plain definition on random inputs with many repeats
    rng = np.random.default_rng(7)
    for trial in range(20):
        qs = [[tuple(rng.integers(0, 3, size=rng.integers(1, 5))) for _ in range(rng.integers(1, 7))]
              for _ in range(rng.integers(1, 4))]
        tg, co, qo = _seq_arrays(qs)
        tok_node, node_tok = jo.predictor_trie(tg, co, qo)
        hist = []
        for g, cands in enumerate(qs):
            for seq in cands:
                hist.extend((g, tuple(seq[:t])) for t in range(len(seq)))
        n = len(hist)
        for i in range(n):
            for j in range(n):
                assert (tok_node[i] == tok_node[j]) == (hist[i] == hist[j])
        firsts = [int(np.flatnonzero(tok_node == v)[0]) for v in range(len(node_tok))]
        assert firsts == sorted(firsts) and list(node_tok) == firsts


def pin_deduplicated_scoring():
    """Candidate-preserving readout (FastJEV Sec. 3.3): projecting each predictor node once
    and gathering every token's log-probability through its node gives the same outputs as
    one row per token, when equal histories have equal states (as a backbone gives them)."""
    p = wl.shared_history_problem(V=400, d=16, n_q=4, K=(3, 7), lengths=(1, 4), seed=3)
    full = jo.score(p)
    tok_node, node_tok = jo.predictor_trie(p["tok_target"], p["cand_tok_off"], p["q_cand_off"])
    assert len(node_tok) < p["n_rows"]
    dd = dict(p, H=p["H"][node_tok], n_rows=len(node_tok), tok_row=tok_node.astype(np.int32))
    red = jo.score(dd)
    for k in ("tok_logp", "cand_s", "cand_q", "q_expect", "q_confidence", "q_mass"):
        _close(red[k], full[k], 1e-12, f"dedup {k}")
    assert np.array_equal(red["q_argmax"], full["q_argmax"])
    _close(red["lse"], full["lse"][node_tok], 1e-12, "dedup lse")


def pin_decision_sensitivity():
    """FastJEV Sec. 3.4, Eq. 5-6: d = rms(ctr(delta)) / max(eps, rms(ctr(z))), J = mean d.

    By hand: z = (0, 1) has ctr (-1/2, 1/2), rms 1/2; a skip moving it to (0, 2) has
    delta (0, 1), also rms 1/2 after centring, so d = 1; a skip adding the same amount to
    every entry has d = 0 (a common shift changes no difference).  z constant has
    rms(ctr z) = 0, so the denominator is eps.  d is unchanged by a per-input shift of z or
    of the skipped logits (ctr removes it) and by scaling both by c > 0; J is the mean over
    inputs; a pure-Python brute force agrees on random ragged inputs."""
    d, J = jo.decision_sensitivity([0.0, 1.0], [[0.0, 2.0], [3.5, 4.5]], [0, 2])
    _close(d[:, 0], [1.0, 0.0], 1e-15, "hand d")
    d, _ = jo.decision_sensitivity([2.0, 2.0, 2.0], [[2.0, 2.0, 2.3]], [0, 3])
    exp_num = math.sqrt(((0.3 - 0.1) ** 2 + 2 * 0.1 ** 2) / 3)
    _close(d[0, 0], exp_num / 1e-8, 1e-6 * exp_num / 1e-8, "eps floor")
    rng = np.random.default_rng(5)
    off = np.concatenate([[0], np.cumsum(rng.integers(1, 9, size=6))])
    z = rng.normal(size=off[-1])
    zs = z + rng.normal(scale=0.3, size=(4, off[-1]))
    d, J = jo.decision_sensitivity(z, zs, off)
    shift = np.repeat(rng.normal(size=6) * 50, np.diff(off))
    d2, _ = jo.decision_sensitivity(z + shift, zs + shift + rng.normal(size=(4, 1)) * 0, off)
    _close(d2, d, 1e-9, "shift of z and skipped logits")
    d3, _ = jo.decision_sensitivity(z, zs + np.repeat(rng.normal(size=6), np.diff(off)), off)
    _close(d3, d, 1e-9, "shift of the skipped logits alone")
    d4, _ = jo.decision_sensitivity(3.7 * z, 3.7 * zs, off)
    _close(d4, d, 1e-12, "common scale")
    _close(J, d.mean(axis=1), 0.0, "J is the mean")
    for l in range(4):
        for x in range(6):
            a, b = int(off[x]), int(off[x + 1])
            m = b - a
            zm = math.fsum(z[a:b]) / m
            dl = [zs[l, i] - z[i] for i in range(a, b)]
            dm = math.fsum(dl) / m
            num = math.sqrt(math.fsum((v - dm) ** 2 for v in dl) / m)
            den = max(1e-8, math.sqrt(math.fsum((z[i] - zm) ** 2 for i in range(a, b)) / m))
            assert abs(d[l, x] - num / den) <= 1e-12 * max(1.0, num / den)


def pin_select_layers():
    """The k smallest J with ties resolved by layer index (FastJEV Sec. 3.4)."""
    J = [0.3, 0.1, 0.1, 0.5, 0.05]
    assert list(jo.select_layers(J, 3)) == [4, 1, 2]
    assert list(jo.select_layers(J, 2)) == [4, 1]
    assert list(jo.select_layers(J, 0)) == []
    assert list(jo.select_layers([1.0, 1.0, 1.0], 2)) == [0, 1]


def pin_temperature_fit():
    """Temperature fitting = the T minimising the mean gold NLL (gemma-e2b doc, "Output
    contracts"; T scales candidate scores once, nimble "V2 probability default").

    Closed form: two binary questions with gold gaps +2 and -1 have mean NLL
    f(b) = (log(1 + e^{-2b}) + log(1 + e^{b})) / 2 in b = 1/T; f'(b) = 0 gives
    x^3 - x - 2 = 0 for x = e^b, whose real root is Cardano's
    cbrt(1 + sqrt(26/27)) + cbrt(1 - sqrt(26/27)).  Scaling every score by c scales T* by c.
    Equal-text gold labels sum their probabilities; unlabelled questions are not counted."""
    s = np.array([0.0, -2.0, 0.0, 1.0])
    qo, text, gold = np.array([0, 2, 4]), np.array([0, 1, 0, 1]), np.array([0, 0])
    r = math.sqrt(26.0 / 27.0)
    x = (1 + r) ** (1 / 3) + (1 - r) ** (1 / 3)
    T_star = 1.0 / math.log(x)
    assert abs(x ** 3 - x - 2) < 1e-12
    T, f = jo.fit_temperature(s, qo, text, gold)
    assert abs(T - T_star) < 1e-7 * T_star, (T, T_star)
    for t in (0.5, 1.0, T_star, 7.0):
        want = (math.log1p(math.exp(-2 / t)) + math.log1p(math.exp(1 / t))) / 2
        assert abs(jo.mean_gold_nll(s, qo, text, gold, t)[0] - want) < 1e-14
    T3, _ = jo.fit_temperature(3.0 * s, qo, text, gold)
    assert abs(T3 - 3.0 * T_star) < 3e-7 * T_star
    # equal-text labels sum; an unlabelled question changes nothing
    s2, qo2, tx2 = np.array([1.0, 1.0, 0.0, 5.0, 2.0]), np.array([0, 3, 5]), np.array([0, 0, 1, 0, 1])
    v, n = jo.mean_gold_nll(s2, qo2, tx2, np.array([0, -1]), 1.0)
    assert n == 1 and abs(v - (math.log(2 * math.e + 1) - math.log(2 * math.e))) < 1e-14


def test_planted_temperature_recovery():
    """Statistical check of the fit (not a mutant pin): labels drawn at T0 = 2.179 by the
    Gumbel-max trick over 4096 questions give a fitted T within 5% of T0."""
    c = wl.labelled_questions(n_q=4096)
    T, _ = jo.fit_temperature(c["cand_s"], c["q_cand_off"], c["cand_text_id"], c["q_gold_text_id"])
    assert abs(T / c["T0"] - 1) < 0.05, T


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[f.__name__ for f in ALL_PINS])
def test_pin(pin):
    pin()
