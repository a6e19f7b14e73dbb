"""Marshalling of problem dicts (numpy arrays, as the workloads package builds them) onto the
device and through the C ABI.  No scoring arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import api


def _operand(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def _i32(a, device):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def to_device(p: dict, device="cuda") -> dict:
    """Upload a full-vocabulary problem; returns the keyword arguments of api.score."""
    return dict(
        H=_operand(p["H"], p["h_dtype"], device), W=_operand(p["W"], p["w_dtype"], device),
        tok_target=_i32(p["tok_target"], device), cand_tok_off=_i32(p["cand_tok_off"], device),
        q_cand_off=_i32(p["q_cand_off"], device), T=p["T"], tok_row=_i32(p.get("tok_row"), device),
        cand_text_id=_i32(p.get("cand_text_id"), device),
        q_gold_text_id=_i32(p.get("q_gold_text_id"), device),
        q_true_idx=_i32(p.get("q_true_idx"), device))


def restricted_to_device(rp: dict, device="cuda") -> dict:
    """Build the allowed-id union on the host (jet_build_union) and upload a restricted
    problem; returns the keyword arguments of api.score_restricted plus the host union."""
    union, slot = api.build_union(rp["field_ids"], rp["field_off"], rp["V"])
    return dict(
        H=_operand(rp["H"], rp["h_dtype"], device), W=_operand(rp["W"], rp["w_dtype"], device),
        union_ids=_i32(union, device), field_row=_i32(rp["field_row"], device),
        field_slot_off=_i32(rp["field_off"], device), slot_uidx=_i32(slot, device), T=rp["T"],
        host_union=union, host_slot_uidx=slot)


def score_problem(pd: dict, **kw) -> dict:
    return api.score(**pd, **kw)


def score_restricted_problem(rd: dict, **kw) -> dict:
    args = {k: v for k, v in rd.items() if not k.startswith("host_")}
    return api.score_restricted(**args, **kw)


def to_numpy(out: dict) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in out.items()}
