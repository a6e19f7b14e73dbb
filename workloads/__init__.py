"""Seeded synthetic workloads for candidate-likelihood scoring.

This package only builds inputs (hidden states, head weights, token/candidate/question
index structure).  It performs none of the scoring arithmetic, so both the CPU oracle and
the HIP path can consume the same arrays without sharing any of the method's code.
"""
from .synth import (  # noqa: F401
    CONFIG_NAMES,
    bf16_bits,
    head_weights,
    hidden_states,
    make_config,
    make_restricted,
    make_problem,
    tiny,
    binary_enum,
    multi_token,
    restricted,
    restricted_as_full,
    large_batch,
    stress,
    shared_history_problem,
    calibration_logits,
    labelled_questions,
)
