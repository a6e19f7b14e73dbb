"""fp64 CPU oracle for candidate-likelihood scoring.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package's smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  Parity status of every function
is pinned by tests/test_oracle_pins.py (worked example, closed forms, invariants, brute
force); none is "parity unpinned".
"""
from .jet_oracle import (  # noqa: F401
    build_union,
    candidate_scores,
    decide,
    allowed_mass,
    confidence,
    decide_question,
    decision_sensitivity,
    fit_temperature,
    logits,
    logsumexp_rows,
    mean_gold_nll,
    predictor_trie,
    score,
    score_restricted,
    select_layers,
    token_logprobs,
    widen,
)
