"""Plain fp64 CPU oracle for teacher-forced candidate-likelihood scoring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module: only the tests, the package's smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library; the two meet only at the seeded input arrays.

What it computes, in the pages' order (citations name the page and its equation/section):

  z[r, v]   = sum_i H[r, i] W[v, i]                      projection of a predictor state
                                                         through the LM head (JET paper,
                                                         Eq. 1; FastJEV Sec. 3.3,
                                                         candidate-preserving readout)
  LSE_r     = log sum_{v in V} exp z[r, v]               full-vocabulary denominator
                                                         (JET paper, Eq. 1 and Eq. 2)
  l_k       = z[row_k, y_k] - LSE_{row_k}                token log-probability (JET Eq. 2)
  s(c)      = sum_t l_{c,t}                              chain rule (JET Eq. 3; gemma-e2b
                                                         doc, "Candidate likelihoods")
  q(c)      = exp(s(c)/T) / sum_j exp(s(c_j)/T)          candidate-set normalisation (JET
                                                         Eq. 4; gemma-e2b doc; nimble page,
                                                         Execution step 6)
  argmax    lowest index among the maxima of s/T         fixed tie order (JET Eq. 5)
  q(true)   q at the "true" candidate                    binary rule (JET, decision rules;
                                                         nimble page: booleans default to
                                                         [false, true])
  E         = sum_i i q(i)                               ordinal rule (JET, decision rules)
  NLL_gold  = -log sum_{c: text(c) = gold} q(c)          gold NLL over equal-text labels
                                                         (JET, labels vs answer text)
  restricted: softmax over a field's allowed-token logits divided by T
                                                         (nimble page, Execution steps 5-6)

Readings taken where the pages are silent:
  * T scales candidate scores only, once, before the candidate softmax; token
    log-probabilities are never tempered (JET says tokens are scored without temperature;
    the gemma-e2b doc and the nimble page apply T to candidate scores).
  * "Fixed ordering" for ties = supplied candidate order, lowest index wins.  The decision
    is taken on the exact fp64 a = s/T (a tie is exact equality there, as for candidates
    with identical inputs); top-two gaps in q are reported so that a comparison can tell
    a clear decision from a near tie.
  * Binary "true" index: per-question index if given, else 1 for K == 2 ([false, true]),
    else none (NaN).
  * Gold NLL uses the same q as the decision (so T is included), natural log; +inf when
    no candidate carries the gold text.
Floating point: inputs are widened exactly (fp32 -> fp64; bf16 bits -> fp32 -> fp64), all
arithmetic is fp64.  numpy's matmul (a library primitive) forms the dot products.
"""
from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)


# ----------------------------------------------------------------------------------------
# operand widening
# ----------------------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of an input operand to fp64.  bf16 values arrive as their 16 bits."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------
# readout: logits, full-vocabulary log-normaliser, token log-probabilities
# ----------------------------------------------------------------------------------------

def logits(H64: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """z[r, v] = <H[r], W[v]> for every predictor row r and vocabulary entry v
    (JET paper, Eq. 1: the logit of token v given the context and the candidate prefix;
    FastJEV Sec. 3.3: each predictor node is projected through the LM head)."""
    return H64 @ W64.T


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """LSE_r = m_r + log sum_v exp(z[r, v] - m_r) with m_r = max_v z[r, v]
    (JET paper, Eq. 2: the numerically stable form of the log-probability's denominator;
    the denominator runs over the full vocabulary, Eq. 1)."""
    m = z.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(z - m).sum(axis=1))


def token_logprobs(z_at_target: np.ndarray, lse_of_row: np.ndarray) -> np.ndarray:
    """l_k = z[row_k, y_k] - LSE_{row_k} (JET paper, Eq. 2)."""
    return z_at_target - lse_of_row


def candidate_scores(tok_logp: np.ndarray, cand_tok_off: np.ndarray) -> np.ndarray:
    """s(c) = sum of the candidate's token log-probabilities, in token order, with no
    length normalisation and no extra tokens (JET paper, Eq. 3 and the remarks after
    Eq. 4; gemma-e2b doc, "Candidate likelihoods")."""
    n = len(cand_tok_off) - 1
    s = np.empty(n, dtype=np.float64)
    for c in range(n):
        s[c] = float(np.sum(tok_logp[cand_tok_off[c]:cand_tok_off[c + 1]]))
    return s


# ----------------------------------------------------------------------------------------
# candidate-set decisions
# ----------------------------------------------------------------------------------------

def _lse(a: np.ndarray) -> float:
    m = float(np.max(a))
    if m == -math.inf:
        return -math.inf
    return m + math.log(float(np.sum(np.exp(a - m))))


def decide_question(s: np.ndarray, T: float, text_id=None, gold_text=None, true_idx=None) -> dict:
    """Decisions for one question from its candidates' sequence scores s.

    q = softmax(s / T) over the supplied candidates (JET Eq. 4, gemma-e2b doc, nimble
    Execution step 6 with temperature applied once to candidate scores); argmax with the
    lowest index winning ties (JET Eq. 5); q(true) (binary rule); E = sum_i i q_i with
    levels 0..K-1 (ordinal rule); gold NLL = -log of the summed q of every candidate whose
    text equals the gold text (JET, labels vs answer text), computed as
    LSE(a) - LSE(a over gold-text candidates)."""
    K = len(s)
    a = np.asarray(s, dtype=np.float64) / float(T)
    M = float(np.max(a))
    e = np.exp(a - M)
    Z = float(np.sum(e))
    q = e / Z
    argmax = int(np.flatnonzero(a == M)[0])
    qs = np.sort(q)[::-1]
    gap = float(qs[0] - qs[1]) if K >= 2 else math.inf
    if true_idx is None:
        t = 1 if K == 2 else -1
    else:
        t = int(true_idx)
    q_true = float(q[t]) if 0 <= t < K else math.nan
    expect = float(np.sum(np.arange(K, dtype=np.float64) * q))
    if text_id is None or gold_text is None:
        nll = math.nan
    else:
        g = np.asarray(text_id) == gold_text
        nll = math.inf if not g.any() else _lse(a) - _lse(a[g])
    return dict(q=q, argmax=argmax, gap=gap, q_true=q_true, expect=expect, nll=nll,
                confidence=confidence(q), mass=allowed_mass(s))


def confidence(q: np.ndarray) -> float:
    """One minus the normalised entropy of the decision distribution (gemma-e2b doc,
    "Output contracts": concentration of the distribution, not an accuracy estimate):
    1 - H(q) / ln K with H(q) = -sum q_i ln q_i and 0 ln 0 = 0.  Reading: a single choice
    (K = 1, where ln K = 0) is fully concentrated, confidence 1."""
    q = np.asarray(q, dtype=np.float64)
    K = len(q)
    if K == 1:
        return 1.0
    nz = q[q > 0]
    H = -float(np.sum(nz * np.log(nz)))
    return 1.0 - H / math.log(K)


def allowed_mass(s: np.ndarray) -> float:
    """Full-vocabulary probability of the allowed choices (gemma-e2b doc, "Output
    contracts"): the summed probabilities of the complete candidate sequences,
    sum_c exp s(c); for single-token candidates, the probability of the allowed tokens."""
    s = np.asarray(s, dtype=np.float64)
    return float(np.sum(np.exp(s)))


def decide(s: np.ndarray, q_cand_off: np.ndarray, T: float, cand_text_id=None,
           q_gold_text_id=None, q_true_idx=None) -> dict:
    """decide_question over every question; a question with any NaN candidate score (a
    candidate not computed in a sampled run) gets NaN outputs and argmax -1."""
    n_q = len(q_cand_off) - 1
    out = dict(q=np.full(len(s), np.nan), argmax=np.full(n_q, -1, np.int64),
               gap=np.full(n_q, np.nan), q_true=np.full(n_q, np.nan),
               expect=np.full(n_q, np.nan), nll=np.full(n_q, np.nan),
               confidence=np.full(n_q, np.nan), mass=np.full(n_q, np.nan))
    for g in range(n_q):
        c0, c1 = int(q_cand_off[g]), int(q_cand_off[g + 1])
        sg = s[c0:c1]
        if np.isnan(sg).any():
            continue
        r = decide_question(
            sg, T,
            None if cand_text_id is None else cand_text_id[c0:c1],
            None if q_gold_text_id is None else int(q_gold_text_id[g]),
            None if q_true_idx is None else int(q_true_idx[g]))
        out["q"][c0:c1] = r["q"]
        for k in ("argmax", "gap", "q_true", "expect", "nll", "confidence", "mass"):
            out[k][g] = r[k]
    return out


# ----------------------------------------------------------------------------------------
# full problem
# ----------------------------------------------------------------------------------------

def score(p: dict, rows=None, W64=None) -> dict:
    """Score a whole problem (a dict as built by the workloads package).

    rows: None for every row, or an index array of the predictor rows to compute (sampled
    parity at full size); tokens on other rows get NaN, and so does everything built on
    them.  W64: the head already widened to fp64 by widen() (so that repeated calls, e.g.
    when timing the scoring alone, widen it once); None widens p["W"] here.  Returns fp64
    arrays: lse (per row, NaN if not computed), tok_logp, cand_s, cand_q, q_argmax, q_gap,
    q_true, q_expect, q_nll, q_confidence, q_mass.
    """
    n_rows = int(p["n_rows"])
    tok_target = np.asarray(p["tok_target"], dtype=np.int64)
    n_tok = len(tok_target)
    tok_row = (np.arange(n_tok, dtype=np.int64) if p.get("tok_row") is None
               else np.asarray(p["tok_row"], dtype=np.int64))
    rows = np.arange(n_rows) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    if W64 is None:
        W64 = widen(p["W"], p["w_dtype"])
    H64 = widen(np.asarray(p["H"])[rows], p["h_dtype"])
    lse = np.full(n_rows, np.nan)
    z_tgt = np.full(n_tok, np.nan)
    where = np.full(n_rows, -1, dtype=np.int64)
    where[rows] = np.arange(len(rows))
    blk = 64
    for b0 in range(0, len(rows), blk):
        z = logits(H64[b0:b0 + blk], W64)
        lse[rows[b0:b0 + blk]] = logsumexp_rows(z)
        sel = np.flatnonzero((where[tok_row] >= b0) & (where[tok_row] < b0 + blk))
        z_tgt[sel] = z[where[tok_row[sel]] - b0, tok_target[sel]]
    tok_logp = token_logprobs(z_tgt, lse[tok_row])
    cand_s = candidate_scores(tok_logp, np.asarray(p["cand_tok_off"]))
    dec = decide(cand_s, np.asarray(p["q_cand_off"]), p["T"], p.get("cand_text_id"),
                 p.get("q_gold_text_id"), p.get("q_true_idx"))
    return dict(lse=lse, tok_logp=tok_logp, cand_s=cand_s, cand_q=dec["q"],
                q_argmax=dec["argmax"], q_gap=dec["gap"], q_true=dec["q_true"],
                q_expect=dec["expect"], q_nll=dec["nll"], q_confidence=dec["confidence"],
                q_mass=dec["mass"])


# ----------------------------------------------------------------------------------------
# restricted vocabulary (allowed code tokens)
# ----------------------------------------------------------------------------------------

def build_union(field_ids: np.ndarray, field_off: np.ndarray, V: int):
    """Sorted unique union of every field's allowed ids and, per slot, its index in the
    union (nimble page, Execution step 5: gather only the allowed head rows and project
    onto their union; each field then selects its own subset)."""
    ids = np.asarray(field_ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("allowed id outside [0, V)")
    union = np.unique(ids)
    slot_uidx = np.searchsorted(union, ids)
    return union.astype(np.int32), slot_uidx.astype(np.int32)


def score_restricted(rp: dict) -> dict:
    """Per field f with row r and allowed ids j: b_j = z[r, j]; q = softmax(b / T) over the
    field's allowed ids; argmax with the lowest index winning ties, decided on the
    exact fp64 b / T (nimble page, Execution step 6; scaling applied once before the
    softmax, "V2 probability default").  No full-vocabulary normaliser is involved
    ("Correctness and limits": full-vocabulary probabilities are not part of this path)."""
    fo = np.asarray(rp["field_off"])
    ids = np.asarray(rp["field_ids"], dtype=np.int64)
    rows = np.asarray(rp["field_row"], dtype=np.int64)
    H64 = widen(rp["H"], rp["h_dtype"])
    W64 = widen(np.asarray(rp["W"])[ids], rp["w_dtype"]) if ids.size else np.zeros((0, rp["d"]))
    n_f = len(fo) - 1
    logit = np.empty(len(ids))
    qv = np.empty(len(ids))
    am = np.empty(n_f, dtype=np.int64)
    gap = np.empty(n_f)
    for f in range(n_f):
        a0, a1 = int(fo[f]), int(fo[f + 1])
        b = W64[a0:a1] @ H64[rows[f]]
        logit[a0:a1] = b
        r = decide_question(b, rp["T"])
        qv[a0:a1] = r["q"]
        am[f] = r["argmax"]
        gap[f] = r["gap"]
    return dict(slot_logit=logit, slot_q=qv, field_argmax=am, field_gap=gap)


# ----------------------------------------------------------------------------------------
# predictor-row deduplication (history trie)
# ----------------------------------------------------------------------------------------

def predictor_trie(tok_target, cand_tok_off, q_cand_off):
    """History-consistent merging of candidate token sequences (FastJEV Sec. 3.3, Eq. 4).

    Token t of a candidate is predicted from the state after its preceding history: the
    question's context followed by the candidate's tokens 0 .. t-1.  Histories form a tree
    per question: the root is the context, and the child of node v by token y is keyed by
    (v, y); since every candidate starts at the same position, depth fixes the position, so
    the key carries no separate position.  Two tokens share a predictor node exactly when
    they belong to the same question and have identical preceding histories.

    Returns (tok_node, node_tok): tok_node[k] is the predictor node of token k, numbered
    0, 1, ... in order of first use over the tokens; node_tok[j] is the first token predicted
    from node j (a row of the undeduplicated layout that holds node j's state)."""
    tok_target = [int(x) for x in tok_target]
    co = [int(x) for x in cand_tok_off]
    qo = [int(x) for x in q_cand_off]
    tok_node = [-1] * len(tok_target)
    node_tok = []
    number = {}      # tree node -> predictor index (assigned at first use)
    child = {}       # (tree node, token) -> tree node
    n_tree = 0
    for g in range(len(qo) - 1):
        root = ("root", g)
        for c in range(qo[g], qo[g + 1]):
            v = root
            for k in range(co[c], co[c + 1]):
                if v not in number:
                    number[v] = len(node_tok)
                    node_tok.append(k)
                tok_node[k] = number[v]
                key = (v, tok_target[k])
                if key not in child:
                    child[key] = n_tree
                    n_tree += 1
                v = child[key]
    return np.array(tok_node, dtype=np.int64), np.array(node_tok, dtype=np.int64)


# ----------------------------------------------------------------------------------------
# decision sensitivity of layer skips
# ----------------------------------------------------------------------------------------

def decision_sensitivity(z, z_skip, seg_off, eps: float = 1e-8):
    """Layer sensitivity (FastJEV Sec. 3.4, Eq. 5-6).

    z[seg_off[x]:seg_off[x+1]] is input x's logit vector (candidates and abstention) and
    z_skip[l] the same vector with layer l skipped.  With ctr(v) = v - mean(v) and
    rms(v) = ||v|| / sqrt(m):
        d[l, x] = rms(ctr(z_skip[l] - z)) / max(eps, rms(ctr(z)))   over input x's entries
        J[l]    = mean over inputs of d[l, x].
    Returns (d [n_layers, n_inputs], J [n_layers]) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    zs = np.asarray(z_skip, dtype=np.float64).reshape(-1, len(z))
    off = [int(o) for o in seg_off]
    n_in, L = len(off) - 1, zs.shape[0]
    d = np.empty((L, n_in))
    for x in range(n_in):
        a, b = off[x], off[x + 1]
        zx = z[a:b]
        den = max(eps, float(np.sqrt(np.mean((zx - zx.mean()) ** 2))))
        for l in range(L):
            delta = zs[l, a:b] - zx
            d[l, x] = float(np.sqrt(np.mean((delta - delta.mean()) ** 2))) / den
    return d, d.mean(axis=1)


def select_layers(J, k: int):
    """The k layers with the smallest J, ties resolved by layer index (FastJEV Sec. 3.4,
    "Calibration Guided Selection"), listed in that order (smallest first)."""
    J = np.asarray(J)
    order = sorted(range(len(J)), key=lambda l: (J[l], l))
    return np.array(order[:k], dtype=np.int64)


# ----------------------------------------------------------------------------------------
# temperature fitting
# ----------------------------------------------------------------------------------------

def _labelled_matrix(s, q_cand_off, cand_text_id, q_gold_text_id):
    """Labelled questions as padded rows: scores [n, Kmax] (-inf padding) and gold masks."""
    s = np.asarray(s, dtype=np.float64)
    qo = np.asarray(q_cand_off, dtype=np.int64)
    text = np.asarray(cand_text_id)
    K = np.diff(qo)
    keep = []
    for g in range(len(K)):
        gold = int(q_gold_text_id[g])
        if gold >= 0 and (text[qo[g]:qo[g + 1]] == gold).any():
            keep.append(g)
    Kmax = int(K.max()) if len(K) else 1
    S = np.full((len(keep), Kmax), -np.inf)
    G = np.zeros((len(keep), Kmax), dtype=bool)
    for i, g in enumerate(keep):
        S[i, :K[g]] = s[qo[g]:qo[g + 1]]
        G[i, :K[g]] = text[qo[g]:qo[g + 1]] == int(q_gold_text_id[g])
    return S, G


def _row_lse(A):
    m = A.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(A - m).sum(axis=1))


def mean_gold_nll(s, q_cand_off, cand_text_id, q_gold_text_id, T: float, _mat=None):
    """Mean over labelled questions of the gold NLL at temperature T (the decision's q,
    equal-text labels summed: LSE(s/T) - LSE(s/T over gold-text candidates)).  Questions
    with no label (gold id < 0) or no candidate of the gold text are not counted.
    Returns (mean, number of questions counted)."""
    S, G = _mat if _mat is not None else _labelled_matrix(s, q_cand_off, cand_text_id, q_gold_text_id)
    if len(S) == 0:
        return math.nan, 0
    A = S / float(T)
    nll = _row_lse(A) - _row_lse(np.where(G, A, -np.inf))
    return float(nll.mean()), len(S)


def fit_temperature(s, q_cand_off, cand_text_id, q_gold_text_id, T_min: float = 1e-2,
                    T_max: float = 1e2):
    """The temperature minimising the mean gold NLL over [T_min, T_max] (gemma-e2b doc,
    "Output contracts": temperature fitting; nimble "V2 probability default": T scales the
    candidate scores once before the softmax).  The pages name the fit but not its method;
    this is the plain minimiser: an 801-point log grid locates the basin, then a bounded
    scalar minimisation in log T refines it.  Returns (T*, mean NLL at T*)."""
    from scipy.optimize import minimize_scalar

    mat = _labelled_matrix(s, q_cand_off, cand_text_id, q_gold_text_id)
    f = lambda u: mean_gold_nll(None, None, None, None, math.exp(u), _mat=mat)[0]  # noqa: E731
    lo, hi = math.log(T_min), math.log(T_max)
    grid = np.linspace(lo, hi, 801)
    vals = np.array([f(u) for u in grid])
    if not np.isfinite(vals).any():
        return math.nan, math.nan
    i = int(np.nanargmin(vals))
    a, b = grid[max(i - 1, 0)], grid[min(i + 1, len(grid) - 1)]
    r = minimize_scalar(f, bounds=(a, b), method="bounded", options=dict(xatol=1e-12))
    best_u, best_f = (r.x, r.fun) if r.fun <= vals[i] else (grid[i], vals[i])
    return math.exp(best_u), float(best_f)
