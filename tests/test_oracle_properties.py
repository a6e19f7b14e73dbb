"""Property tests of the fp64 oracle on random small problems (hypothesis): random
vocabulary sizes, widths, question/candidate/token structures, layouts, temperatures and
operand types, each checked against the exact-summation brute force of the definitions and
against structural invariants that hold for every input."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle as jo  # noqa: E402
import workloads as wl  # noqa: E402
from tests.test_oracle_pins import _close, brute_force  # noqa: E402

problems = st.fixed_dictionaries(dict(
    seed=st.integers(0, 2**31 - 1),
    layout=st.sampled_from(["prefix", "field", "own"]),
    V=st.integers(1, 48),
    d=st.sampled_from([4, 8, 16]),
    n_q=st.integers(1, 4),
    K=st.tuples(st.integers(1, 3), st.integers(3, 7)),
    lengths=st.tuples(st.integers(1, 2), st.integers(2, 4)),
    T=st.sampled_from([0.5, 1.0, 1.7, 4.0]),
    dups=st.integers(0, 2),
    h_dtype=st.sampled_from(["f32", "bf16"]),
    w_dtype=st.sampled_from(["f32", "bf16"]),
))


def _make(c):
    if c["w_dtype"] == "f32":
        c = dict(c, h_dtype="f32")  # an fp32 head takes fp32 hidden states only
    return wl.make_problem(n_extra_rows=1 if c["layout"] != "own" else 0, **c)


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(problems)
def test_oracle_matches_brute_force(c):
    p = _make(c)
    r = jo.score(p)
    b = brute_force(p)
    _close(r["lse"], b["lse"], 1e-11, "lse")
    _close(r["tok_logp"], b["tok_logp"], 1e-11, "l")
    _close(r["cand_s"], b["cand_s"], 1e-10, "s")
    _close(r["cand_q"], b["cand_q"], 1e-11, "q")
    _close(r["q_expect"], b["q_expect"], 1e-10, "E")
    # argmax: equal where the top two scaled scores are apart by more than rounding
    qo = p["q_cand_off"]
    for g in range(len(qo) - 1):
        a = np.sort(np.asarray(b["cand_s"][qo[g]:qo[g + 1]]) / p["T"])[::-1]
        if len(a) == 1 or a[0] - a[1] > 1e-9:
            assert r["q_argmax"][g] == b["q_argmax"][g]


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(problems)
def test_oracle_invariants(c):
    p = _make(c)
    r = jo.score(p)
    qo = p["q_cand_off"]
    co = p["cand_tok_off"]
    q = np.asarray(r["cand_q"])
    for g in range(len(qo) - 1):
        qg = q[qo[g]:qo[g + 1]]
        K = len(qg)
        # a distribution over the question's candidates
        assert np.all(qg >= 0) and abs(qg.sum() - 1.0) < 1e-12
        # expected index inside [0, K - 1]
        assert -1e-12 <= r["q_expect"][g] <= K - 1 + 1e-12
        # the decision is a candidate of maximal probability
        assert qg[r["q_argmax"][g]] == qg.max()
    # log-probabilities are <= 0 and candidate sums add them in token order
    assert np.all(np.asarray(r["tok_logp"]) <= 1e-12)
    for cc in range(len(co) - 1):
        assert abs(r["cand_s"][cc] - sum(r["tok_logp"][co[cc]:co[cc + 1]])) < 1e-12
