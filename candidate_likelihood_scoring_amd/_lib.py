"""ctypes mirror of include/jet.h and the loader of libjet.so.

Argument marshalling only: every step of the scoring path runs in the HIP library.  There
is no fallback: if libjet.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjet.so")

JET_F32 = 0
JET_BF16 = 1

STATUS = {
    0: "JET_OK", -1: "JET_E_NULL", -2: "JET_E_SHAPE", -3: "JET_E_DTYPE", -4: "JET_E_INDEX",
    -5: "JET_E_TEMP", -6: "JET_E_WORKSPACE", -7: "JET_E_HIP",
}
NOALLOC_MAX_WORKSPACE = 64 << 20  # JET_NOALLOC_MAX_WORKSPACE
FLAG_BAD_ROW = 1
FLAG_BAD_TARGET = 2
FLAG_BAD_OFFSETS = 4
FLAG_BAD_TRUE_IDX = 8
FLAG_BAD_UNION = 16


class JetProblem(ctypes.Structure):
    _fields_ = [
        ("H", c_void_p), ("h_dtype", c_int), ("n_rows", c_int32),
        ("W", c_void_p), ("w_dtype", c_int), ("V", c_int32), ("d", c_int32),
        ("tok_row", c_void_p), ("tok_target", c_void_p), ("n_tok", c_int32),
        ("cand_tok_off", c_void_p), ("n_cand", c_int32),
        ("q_cand_off", c_void_p), ("n_q", c_int32),
        ("cand_text_id", c_void_p), ("q_gold_text_id", c_void_p), ("q_true_idx", c_void_p),
        ("T", c_float),
    ]


class JetOutputs(ctypes.Structure):
    _fields_ = [
        ("tok_logp", c_void_p), ("row_lse", c_void_p), ("cand_s", c_void_p), ("cand_q", c_void_p),
        ("q_argmax", c_void_p), ("q_true", c_void_p), ("q_expect", c_void_p),
        ("q_gold_nll", c_void_p), ("q_confidence", c_void_p), ("q_mass", c_void_p),
        ("dev_flags", c_void_p),
    ]


class JetRestrictedProblem(ctypes.Structure):
    _fields_ = [
        ("H", c_void_p), ("h_dtype", c_int), ("n_rows", c_int32),
        ("W", c_void_p), ("w_dtype", c_int), ("V", c_int32), ("d", c_int32),
        ("union_ids", c_void_p), ("n_union", c_int32),
        ("field_row", c_void_p), ("field_slot_off", c_void_p), ("slot_uidx", c_void_p),
        ("n_fields", c_int32), ("n_slots", c_int32), ("T", c_float),
    ]


class JetRestrictedOutputs(ctypes.Structure):
    _fields_ = [("slot_logit", c_void_p), ("slot_q", c_void_p), ("field_argmax", c_void_p),
                ("dev_flags", c_void_p)]


EXPORTS = {
    "jet_score_workspace_size": (c_size_t, [POINTER(JetProblem)]),
    "jet_score": (c_int, [POINTER(JetProblem), POINTER(JetOutputs), c_void_p, c_size_t, c_void_p]),
    "jet_score_profiled": (c_int, [POINTER(JetProblem), POINTER(JetOutputs), c_void_p, c_size_t,
                                   c_void_p, c_void_p, c_void_p]),
    "jet_score_noalloc": (c_int, [POINTER(JetProblem), POINTER(JetOutputs), c_void_p]),
    "jet_projection_kernel": (c_char_p, [POINTER(JetProblem)]),
    "jet_stream_read": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "jet_fit_temperature_workspace_size": (c_size_t, [c_int32]),
    "jet_fit_temperature": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                    c_float, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_size_t, c_void_p]),
    "jet_decision_sensitivity": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                         c_float, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p]),
    "jet_build_predictor_trie": (c_int, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                                         c_void_p, POINTER(c_int32)]),
    "jet_validate_host": (c_int, [POINTER(JetProblem)]),
    "jet_build_union": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, POINTER(c_int32),
                                c_void_p]),
    "jet_restricted_workspace_size": (c_size_t, [POINTER(JetRestrictedProblem)]),
    "jet_score_restricted": (c_int, [POINTER(JetRestrictedProblem), POINTER(JetRestrictedOutputs),
                                     c_void_p, c_size_t, c_void_p]),
    "jet_validate_restricted_host": (c_int, [POINTER(JetRestrictedProblem)]),
    "jet_status_string": (c_char_p, [c_int]),
}

_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libjet.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libjet.so is not built ({p}); run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


class JetError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().jet_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")
        self.status = status
