"""Seeded synthetic inputs shaped like the pages' candidate-scoring workloads.

Every array here is input construction only: normal draws, bf16 rounding of those draws,
and index bookkeeping (which predictor row scores which target token, which tokens form a
candidate, which candidates form a question).  No logit, log-probability or softmax is
computed in this module.

Shapes follow the pages:
  * enum fields with 1-26 distinct single-token choices and boolean fields ordered
    [false, true] (nimble "Parallel constrained scoring in MLX", Run section);
  * up to 32 named fields per request (gemma-e2b architecture doc, "Media and limits");
  * a 248,320-token vocabulary whose head is bf16 (nimble page, Execution step 5 and
    "Correctness and limits");
  * 64-candidate choice sets and multi-token candidates scored teacher-forced
    (FastJEV, Section 3.3; gemma-e2b doc, "Candidate likelihoods");
  * the first token of every candidate scored from the shared prefix's last state
    (JET paper, Section 3 on hybrid execution: the prefix output supplies first-token
    probabilities).
The pages measured on public benchmarks (MMLU, BoolQ, AI2D, ...); these synthetic inputs
stand in for them.  No benchmark item is reproduced.

A problem is a plain dict:
  H (float32 [rows,d] or uint16 bf16 bits), h_dtype ('f32'|'bf16'),
  W (float32 [V,d] or uint16 bf16 bits), w_dtype,
  tok_row (int32 [n_tok] or None = token k uses row k), tok_target (int32 [n_tok]),
  cand_tok_off (int32 [n_cand+1]), q_cand_off (int32 [n_q+1]),
  cand_text_id (int32 [n_cand] or None), q_gold_text_id (int32 [n_q] or None),
  q_true_idx (int32 [n_q] or None), T (float), V, d, n_rows, name.
A restricted problem is a dict with H, h_dtype, W, w_dtype, field_ids (int32, the allowed
ids of all fields concatenated), field_off (int32 [n_fields+1]), field_row (int32
[n_fields]), T, V, d, n_rows, name.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CONFIG_NAMES = ("tiny", "binary_enum", "multi_token", "restricted", "large_batch")

# Stream tags: every array draws from its own counter-free PCG64 stream keyed by
# (seed, tag[, chunk]) so that arrays can be regenerated independently and in parallel.
_TAG_STRUCT = 1
_TAG_H = 2
_TAG_W = 3

_CHUNK_ELEMS = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits.

    Inputs are finite draws, so the NaN special case of the rounding rule never arises.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_matrix(rows: int, d: int, seed: int, tag: int, std: float, dtype: str) -> np.ndarray:
    """[rows, d] draws of N(0, std^2), float32 (or bf16 bits), generated in fixed row chunks.

    Chunk i uses the stream (seed, tag, i); the chunk size is fixed, so the values never
    depend on the thread count.
    """
    rows_per_chunk = max(1, _CHUNK_ELEMS // d)
    n_chunks = (rows + rows_per_chunk - 1) // rows_per_chunk
    out = np.empty((rows, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    s = np.float32(std)

    def fill(i: int) -> None:
        r0 = i * rows_per_chunk
        r1 = min(rows, r0 + rows_per_chunk)
        g = np.random.default_rng([seed, tag, i])
        x = g.standard_normal((r1 - r0, d), dtype=np.float32)
        if s != np.float32(1.0):
            x *= s
        out[r0:r1] = bf16_bits(x) if dtype == "bf16" else x

    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def head_weights(V: int, d: int, seed: int, dtype: str = "bf16", std: float | None = None) -> np.ndarray:
    """LM head W[V, d] ~ N(0, 1/d) unless std is given; bf16 = RNE of the float32 draw."""
    return _normal_matrix(V, d, seed, _TAG_W, (1.0 / np.sqrt(d)) if std is None else std, dtype)


def hidden_states(rows: int, d: int, seed: int, dtype: str = "f32") -> np.ndarray:
    """Predictor hidden states H[rows, d] ~ N(0, 1)."""
    return _normal_matrix(rows, d, seed, _TAG_H, 1.0, dtype)


class _Builder:
    """Accumulates the token -> candidate -> question CSR structure."""

    def __init__(self) -> None:
        self.tok_row: list[int] = []
        self.tok_target: list[int] = []
        self.cand_off = [0]
        self.q_off = [0]
        self.text: list[int] = []
        self.gold: list[int] = []
        self.true_idx: list[int] = []

    def candidate(self, rows, targets, text_id: int) -> None:
        rows = [int(r) for r in rows]
        targets = [int(t) for t in targets]
        assert len(rows) == len(targets) and len(rows) >= 1
        self.tok_row += rows
        self.tok_target += targets
        self.cand_off.append(len(self.tok_row))
        self.text.append(int(text_id))

    def end_question(self, gold_text: int, true_idx: int = -1) -> None:
        assert len(self.text) > self.q_off[-1], "a question needs at least one candidate"
        self.q_off.append(len(self.text))
        self.gold.append(int(gold_text))
        self.true_idx.append(int(true_idx))

    def arrays(self) -> dict:
        i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
        return dict(
            tok_row=i32(self.tok_row),
            tok_target=i32(self.tok_target),
            cand_tok_off=i32(self.cand_off),
            q_cand_off=i32(self.q_off),
            cand_text_id=i32(self.text),
            q_gold_text_id=i32(self.gold),
            q_true_idx=i32(self.true_idx),
        )


def _finish(name, V, d, n_rows, arrays, H, h_dtype, W, w_dtype, T, identity_rows=False,
            with_true_idx=True) -> dict:
    p = dict(name=name, V=int(V), d=int(d), n_rows=int(n_rows), H=H, h_dtype=h_dtype, W=W,
             w_dtype=w_dtype, T=float(T), **arrays)
    if identity_rows:
        assert np.array_equal(p["tok_row"], np.arange(len(p["tok_row"]), dtype=np.int32))
        p["tok_row"] = None
    if not with_true_idx:
        p["q_true_idx"] = None
    return p


# ----------------------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------------------

def tiny(seed: int = 101, tie: bool = False, with_weights: bool = True) -> dict:
    """V=4096, d=256, fp32 H and W; one question of K=4 candidates.

    Row 0 is the shared prefix's last state and scores every candidate's first token; each
    later token has its own predictor row.  Lengths are a seeded permutation of (2,3,3,3),
    the only multiset of four lengths in 1..3 giving 8 rows (1 + sum(m_c - 1) = 8) and
    11 tokens.  tie=True makes candidate 3 re-reference candidate 2's rows and targets
    with candidate 2's text id: an exact duplicate.
    """
    V, d = 4096, 256
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    lengths = rng.permutation(np.array([2, 3, 3, 3]))
    cands = []
    nxt = 1
    for m in lengths:
        rows = [0] + list(range(nxt, nxt + int(m) - 1))
        nxt += int(m) - 1
        cands.append((rows, rng.integers(0, V, size=int(m))))
    gold = int(rng.integers(0, 4))
    texts = [0, 1, 2, 3]
    if tie:
        cands[3] = cands[2]
        texts[3] = texts[2]
    b = _Builder()
    for c, (rows, tg) in enumerate(cands):
        b.candidate(rows, tg, texts[c])
    b.end_question(texts[gold], -1)
    H = hidden_states(8, d, seed, "f32") if with_weights else None
    W = head_weights(V, d, seed, "f32") if with_weights else None
    return _finish("tiny_tie" if tie else "tiny", V, d, 8, b.arrays(), H, "f32", W, "f32", 1.0,
                   with_true_idx=False)


def _field_sizes(rng, n_fields=32, n_binary=8, kmin=3, kmax=26):
    return [2] * n_binary + [int(k) for k in rng.integers(kmin, kmax + 1, size=n_fields - n_binary)]


def binary_enum(seed: int = 202, with_weights: bool = True, V: int = 248320, d: int = 2560) -> dict:
    """32 single-token fields, one scored row each: fields 0-7 boolean (K=2, order
    [false, true]), fields 8-31 enums with K ~ U{3..26}; targets distinct within a field;
    fp32 H, bf16 W, T=1."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    Ks = _field_sizes(rng)
    b = _Builder()
    for f, K in enumerate(Ks):
        tg = rng.choice(V, size=K, replace=False)
        for c in range(K):
            b.candidate([f], [tg[c]], c)
        b.end_question(int(rng.integers(0, K)), -1)
    H = hidden_states(32, d, seed, "f32") if with_weights else None
    W = head_weights(V, d, seed, "bf16") if with_weights else None
    return _finish("binary_enum", V, d, 32, b.arrays(), H, "f32", W, "bf16", 1.0,
                   with_true_idx=False)


def multi_token(seed: int = 303, with_weights: bool = True, V: int = 262144, d: int = 1536,
                n_main: int = 8, K: int = 64, n_dup: int = 4, max_len: int = 12) -> dict:
    """8 choice questions x 64 candidates with lengths ~U{1..12}; every primary token has
    its own predictor row.  Per question, 4 candidates are exact duplicates of 4 others
    (same targets, H rows copied bitwise, same text id).  Per question there is also an
    ordinal subset (K=5 distinct-text candidates, levels 0..4) and a binary subset
    (2 distinct-text candidates, [false, true]) whose candidates re-reference the same
    (row, target) pairs: new token entries, no new rows."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    b = _Builder()
    n_orig = K - n_dup
    nrow = 0
    dup_rows = []  # (dst_rows, src_rows) pairs, copied after H is drawn
    per_q = []
    for q in range(n_main):
        lengths = rng.integers(1, max_len + 1, size=n_orig)
        targets = [rng.integers(0, V, size=int(m)) for m in lengths]
        src = rng.choice(n_orig, size=n_dup, replace=False)
        order = rng.permutation(K)  # slot i holds logical candidate order[i]
        logical = list(range(n_orig)) + [int(s) for s in src]  # index into originals
        rows_of_orig = {}
        for i in range(K):
            lc = int(order[i])
            o = logical[lc]
            m = len(targets[o])
            rows = list(range(nrow, nrow + m))
            nrow += m
            if lc < n_orig:
                rows_of_orig[o] = rows
            else:
                dup_rows.append((rows, o, q))
            b.candidate(rows, targets[o], q * K + o)
        gold_o = int(rng.integers(0, n_orig))
        b.end_question(q * K + gold_o, -1)
        per_q.append((targets, rows_of_orig))
    # resolve duplicate source rows now that every original has rows
    dup_pairs = [(dst, per_q[q][1][o]) for (dst, o, q) in dup_rows]
    n_rows = nrow
    # ordinal subsets (K=5, levels 0..4), then binary subsets ([false, true])
    for q in range(n_main):
        targets, rows_of_orig = per_q[q]
        pick = rng.choice(n_orig, size=5, replace=False)
        for o in pick:
            b.candidate(rows_of_orig[int(o)], targets[int(o)], q * K + int(o))
        b.end_question(q * K + int(pick[int(rng.integers(0, 5))]), -1)
    for q in range(n_main):
        targets, rows_of_orig = per_q[q]
        pick = rng.choice(n_orig, size=2, replace=False)
        for o in pick:
            b.candidate(rows_of_orig[int(o)], targets[int(o)], q * K + int(o))
        b.end_question(q * K + int(pick[int(rng.integers(0, 2))]), 1)
    H = None
    if with_weights:
        H = hidden_states(n_rows, d, seed, "f32")
        for dst, src in dup_pairs:
            H[dst] = H[src]
    W = head_weights(V, d, seed, "bf16") if with_weights else None
    p = _finish("multi_token", V, d, n_rows, b.arrays(), H, "f32", W, "bf16", 1.0)
    p["n_primary_tok"] = n_rows
    p["n_primary_cand"] = n_main * K
    p["dup_row_pairs"] = dup_pairs
    return p


def large_batch(seed: int = 505, with_weights: bool = True, V: int = 248320, d: int = 2560,
                n_q: int = 512, K: int = 8, max_len: int = 12) -> dict:
    """512 questions x 8 candidates with lengths ~U{1..12}; every token has its own row
    (tok_row = identity, passed as None); bf16 H and W; random targets; T=1."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    b = _Builder()
    nrow = 0
    for q in range(n_q):
        lengths = rng.integers(1, max_len + 1, size=K)
        for c in range(K):
            m = int(lengths[c])
            b.candidate(range(nrow, nrow + m), rng.integers(0, V, size=m), c)
            nrow += m
        b.end_question(int(rng.integers(0, K)), -1)
    H = hidden_states(nrow, d, seed, "bf16") if with_weights else None
    W = head_weights(V, d, seed, "bf16") if with_weights else None
    return _finish("large_batch", V, d, nrow, b.arrays(), H, "bf16", W, "bf16", 1.0,
                   identity_rows=True, with_true_idx=False)


def restricted(seed: int = 404, max_variant: bool = False, with_weights: bool = True,
               V: int = 248320, d: int = 2560, w_seed: int = 202) -> dict:
    """Restricted-vocabulary fields: 32 fields of allowed code tokens, one row each, T=2.

    The head is the binary/enum workload's W (seed 202), so this is that problem through
    the allowed-token path.  Default: the same K structure (8 boolean fields, 24 enums
    with K ~ U{3..26}), ids distinct within a field.  max_variant: every field has 26
    allowed ids and all 832 ids are distinct (union of 832 rows).
    """
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    if max_variant:
        Ks = [26] * 32
        ids = rng.choice(V, size=832, replace=False)
        groups = [ids[26 * f: 26 * (f + 1)] for f in range(32)]
    else:
        Ks = _field_sizes(rng)
        groups = [rng.choice(V, size=K, replace=False) for K in Ks]
    field_ids = np.concatenate(groups).astype(np.int32)
    field_off = np.concatenate([[0], np.cumsum(Ks)]).astype(np.int32)
    H = hidden_states(32, d, seed, "f32") if with_weights else None
    W = head_weights(V, d, w_seed, "bf16") if with_weights else None
    return dict(name="restricted_max" if max_variant else "restricted", V=V, d=d, n_rows=32,
                H=H, h_dtype="f32", W=W, w_dtype="bf16", field_ids=field_ids,
                field_off=field_off, field_row=np.arange(32, dtype=np.int32), T=2.0)


def restricted_as_full(rp: dict) -> dict:
    """The same fields as single-token candidates of a full-vocabulary problem: field f is
    a question whose candidates are its allowed ids, each scored from field_row[f]."""
    fo = rp["field_off"]
    n_f = len(fo) - 1
    tok_row = np.repeat(rp["field_row"], np.diff(fo)).astype(np.int32)
    n = int(fo[-1])
    return dict(name=rp["name"] + "_as_full", V=rp["V"], d=rp["d"], n_rows=rp["n_rows"],
                H=rp["H"], h_dtype=rp["h_dtype"], W=rp["W"], w_dtype=rp["w_dtype"],
                tok_row=tok_row, tok_target=rp["field_ids"].astype(np.int32),
                cand_tok_off=np.arange(n + 1, dtype=np.int32), q_cand_off=fo.astype(np.int32),
                cand_text_id=np.arange(n, dtype=np.int32) - np.repeat(fo[:-1], np.diff(fo)).astype(np.int32),
                q_gold_text_id=np.zeros(n_f, dtype=np.int32), q_true_idx=None, T=rp["T"])


# ----------------------------------------------------------------------------------------
# Generic builder for edge cases and ragged parity shapes
# ----------------------------------------------------------------------------------------

def make_problem(V: int, d: int, n_q: int, K=(1, 8), lengths=(1, 4), layout: str = "prefix",
                 h_dtype: str = "f32", w_dtype: str = "bf16", T: float = 1.0, seed: int = 1,
                 dups: int = 0, w_std: float | None = None, n_extra_rows: int = 0,
                 name: str = "custom") -> dict:
    """A seeded problem of arbitrary size.

    layout:
      'prefix' - each question has a prefix row scoring every candidate's first token;
                 later tokens get their own rows (the tiny workload's layout);
      'field'  - single-token candidates, all scored from one row per question;
      'own'    - every token has its own row (tok_row = identity, passed as None).
    K and lengths are inclusive (lo, hi) ranges or ints.  dups > 0 appends that many exact
    duplicates (same rows and targets, same text id) of earlier candidates per question
    (when the question has one).  n_extra_rows adds unreferenced rows at the end.
    """
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    rint = lambda r: int(r) if np.isscalar(r) else int(rng.integers(r[0], r[1] + 1))  # noqa: E731
    b = _Builder()
    nrow = 0
    for q in range(n_q):
        Kq = rint(K)
        prefix_row = None
        if layout in ("prefix", "field"):
            prefix_row = nrow
            nrow += 1
        made = []
        for c in range(Kq):
            m = 1 if layout == "field" else rint(lengths)
            tg = rng.integers(0, V, size=m)
            if layout == "field":
                rows = [prefix_row]
            elif layout == "prefix":
                rows = [prefix_row] + list(range(nrow, nrow + m - 1))
                nrow += m - 1
            else:
                rows = list(range(nrow, nrow + m))
                nrow += m
            b.candidate(rows, tg, c)
            made.append((rows, tg))
        for j in range(dups if Kq >= 1 else 0):
            src = int(rng.integers(0, Kq))
            b.candidate(made[src][0], made[src][1], src)
        b.end_question(int(rng.integers(0, Kq)), -1)
    n_rows = nrow + n_extra_rows
    hseed = seed * 7919 + 17
    H = hidden_states(n_rows, d, hseed, h_dtype) if n_rows > 0 else np.zeros((0, d), np.float32 if h_dtype == "f32" else np.uint16)
    W = head_weights(V, d, seed, w_dtype, std=w_std)
    return _finish(name, V, d, n_rows, b.arrays(), H, h_dtype, W, w_dtype, T,
                   identity_rows=(layout == "own" and n_extra_rows == 0 and dups == 0),
                   with_true_idx=False)


def shared_history_problem(V: int, d: int, n_q: int, K=(2, 8), lengths=(1, 5), alphabet: int = 3,
                           h_dtype: str = "f32", w_dtype: str = "bf16", T: float = 1.0,
                           seed: int = 1, name: str = "shared_history") -> dict:
    """Every token on its own row (tok_row = identity), with candidates that share leading
    tokens: each question draws its candidates' tokens from `alphabet` ids of its own, so
    histories repeat.  A row is the state after the token's preceding history within its
    question, as a backbone would produce it: tokens with equal histories get bitwise-equal
    rows (one seeded draw per distinct history)."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    rint = lambda r: int(r) if np.isscalar(r) else int(rng.integers(r[0], r[1] + 1))  # noqa: E731
    b = _Builder()
    state_of_tok = []
    states = {}
    nrow = 0
    for q in range(n_q):
        ids = rng.choice(V, size=min(alphabet, V), replace=False)
        Kq = rint(K)
        for c in range(Kq):
            m = rint(lengths)
            tg = ids[rng.integers(0, len(ids), size=m)]
            b.candidate(list(range(nrow, nrow + m)), tg, c)
            nrow += m
            for t in range(m):
                key = (q, tuple(int(x) for x in tg[:t]))
                state_of_tok.append(states.setdefault(key, len(states)))
        b.end_question(int(rng.integers(0, Kq)), -1)
    hseed = seed * 7919 + 29
    Hs = hidden_states(len(states), d, hseed, h_dtype)
    H = np.ascontiguousarray(Hs[np.asarray(state_of_tok, dtype=np.int64)])
    W = head_weights(V, d, seed, w_dtype)
    return _finish(name, V, d, nrow, b.arrays(), H, h_dtype, W, w_dtype, T, identity_rows=True,
                   with_true_idx=False)


def calibration_logits(n_inputs: int = 32, K=(2, 65), n_layers: int = 28, seed: int = 707,
                       tie=(4, 9)) -> dict:
    """A calibration set for layer-skip sensitivity: per input a logit vector of K entries
    (candidates and abstention; 32 inputs of up to 64 candidates + 1 by default, the pages'
    calibration size and candidate-set size), with a common offset per input, and per layer
    the same vectors perturbed by a common shift plus layer noise of log-uniform scale in
    [1e-2, 1].  Layer tie[1] is an exact copy of layer tie[0] (an exact tie)."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    m = rng.integers(K[0], K[1] + 1, size=n_inputs)
    off = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
    n = int(off[-1])
    z = (rng.normal(scale=3.0, size=n) + np.repeat(rng.normal(scale=20.0, size=n_inputs), m))
    scale = 10.0 ** rng.uniform(-2.0, 0.0, size=n_layers)
    zs = np.empty((n_layers, n))
    for l in range(n_layers):
        zs[l] = z + np.repeat(rng.normal(scale=5.0, size=n_inputs), m) + scale[l] * rng.normal(size=n)
    if tie is not None:
        zs[tie[1]] = zs[tie[0]]
    return dict(z=z.astype(np.float32), z_skip=zs.astype(np.float32), seg_off=off,
                n_layers=int(n_layers), n_inputs=int(n_inputs))


def labelled_questions(n_q: int = 4096, K=(2, 26), T0: float = 2.179078721266035,
                       seed: int = 808, dup_text: float = 0.1, score_std: float = 3.0) -> dict:
    """Candidate scores with gold labels drawn at a planted temperature T0 (default: the
    fitted temperature one of the pages quotes).  Scores ~ N(0, score_std) per candidate;
    the gold is argmax(s / T0 + Gumbel noise), which has the distribution softmax(s / T0)
    (the Gumbel-max property), so no softmax is computed here.  With probability dup_text a
    question has one candidate re-using another's text id (an equal-text label)."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    Ks = rng.integers(K[0], K[1] + 1, size=n_q)
    qo = np.concatenate([[0], np.cumsum(Ks)]).astype(np.int32)
    s = rng.normal(scale=score_std, size=int(qo[-1]))
    text = np.concatenate([np.arange(k) for k in Ks]).astype(np.int32)
    gold = np.empty(n_q, np.int32)
    for g in range(n_q):
        a, b = int(qo[g]), int(qo[g + 1])
        if b - a >= 2 and rng.random() < dup_text:
            text[b - 1] = text[a]
        pick = int(np.argmax(s[a:b] / T0 + rng.gumbel(size=b - a)))
        gold[g] = text[a + pick]
    return dict(cand_s=s.astype(np.float32), q_cand_off=qo, cand_text_id=text,
                q_gold_text_id=gold, T0=float(T0))


def stress(kind: str = "wide", seed: int = 606, V: int = 248320, d: int = 2560) -> dict:
    """The binary/enum shape with peaked logits.

    'wide'    - W ~ N(0, 16/d): logit standard deviation about 4;
    'planted' - as the default head, plus for every row r one vocabulary entry v_r whose
                head row is bf16(40 * h_r / |h_r|^2), giving that row a logit near +40.
    """
    p = binary_enum(seed=seed, with_weights=False, V=V, d=d)
    p["H"] = hidden_states(32, d, seed, "f32")
    if kind == "wide":
        p["W"] = head_weights(V, d, seed, "bf16", std=4.0 / np.sqrt(d))
    elif kind == "planted":
        W = head_weights(V, d, seed, "bf16")
        rng = np.random.default_rng([seed, 99])
        vs = rng.choice(V, size=32, replace=False)
        for r in range(32):
            h = p["H"][r].astype(np.float64)
            W[vs[r]] = bf16_bits((40.0 * h / np.dot(h, h)).astype(np.float32))
        p["W"] = W
        p["planted_vocab"] = vs.astype(np.int32)
    else:
        raise ValueError(kind)
    p["name"] = f"stress_{kind}"
    return p


def make_config(name: str, **kw) -> dict:
    if name == "tiny":
        return tiny(**kw)
    if name == "tiny_tie":
        return tiny(tie=True, **kw)
    if name == "binary_enum":
        return binary_enum(**kw)
    if name == "multi_token":
        return multi_token(**kw)
    if name == "restricted":
        return restricted(**kw)
    if name == "restricted_max":
        return restricted(max_variant=True, **kw)
    if name == "large_batch":
        return large_batch(**kw)
    raise KeyError(name)


def make_restricted(n_fields: int, V: int, d: int, K=(1, 26), T: float = 2.0, seed: int = 1,
                    h_dtype: str = "f32", w_dtype: str = "bf16", n_rows: int | None = None,
                    shared_rows: bool = False) -> dict:
    """A seeded restricted problem of arbitrary size (fields may share rows when
    shared_rows, so that several fields read one row)."""
    rng = np.random.default_rng([seed, _TAG_STRUCT])
    Ks = [int(K) if np.isscalar(K) else int(rng.integers(K[0], K[1] + 1)) for _ in range(n_fields)]
    groups = [rng.choice(V, size=k, replace=False) for k in Ks]
    rows = n_rows if n_rows is not None else n_fields
    field_row = (rng.integers(0, rows, size=n_fields) if shared_rows
                 else np.arange(n_fields) % max(rows, 1)).astype(np.int32)
    return dict(name="restricted_custom", V=V, d=d, n_rows=rows,
                H=hidden_states(rows, d, seed * 31 + 5, h_dtype), h_dtype=h_dtype,
                W=head_weights(V, d, seed, w_dtype), w_dtype=w_dtype,
                field_ids=np.concatenate(groups).astype(np.int32) if groups else np.zeros(0, np.int32),
                field_off=np.concatenate([[0], np.cumsum(Ks)]).astype(np.int32),
                field_row=field_row, T=float(T))
