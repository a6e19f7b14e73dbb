"""Thin torch-facing binding of libjet (argument marshalling only).

PyTorch supplies device memory and the stream; every computation runs in the HIP library.
Function names follow the C ABI: score -> jet_score, score_restricted ->
jet_score_restricted, build_union -> jet_build_union, validate -> jet_validate_host.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import _lib
from ._lib import JetError, JetOutputs, JetProblem, JetRestrictedOutputs, JetRestrictedProblem

__all__ = ["score", "score_noalloc", "score_restricted", "build_union", "validate", "validate_restricted",
           "score_workspace_size", "restricted_workspace_size", "Workspace"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.JET_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return _lib.JET_BF16  # bf16 values or their raw 16-bit patterns
    raise TypeError(f"unsupported operand dtype {t.dtype}")


def _check_i32(name: str, t, dev) -> None:
    if t is None:
        return
    if t.dtype != torch.int32 or not t.is_contiguous() or t.device != dev:
        raise TypeError(f"{name} must be a contiguous int32 tensor on {dev}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def debug_validate() -> bool:
    """True when JET_DEBUG_VALIDATE=1: before each scoring call the index arrays are copied
    to the host and checked with jet_validate_host / jet_validate_restricted_host, and a
    failure raises JetError (JET_E_INDEX) with nothing enqueued.  The copies synchronise
    with the device, so this is a debugging mode; without it out-of-range indices are only
    reported through the device flag word."""
    return os.environ.get("JET_DEBUG_VALIDATE", "") == "1"


def _host_i32(t):
    return None if t is None else np.ascontiguousarray(t.detach().cpu().numpy(), dtype=np.int32)


def _validate_score_on_host(prob: JetProblem, tok_row, tok_target, cand_tok_off, q_cand_off,
                            q_true_idx, where: str) -> None:
    h = {k: _host_i32(v) for k, v in dict(tok_row=tok_row, tok_target=tok_target,
                                         cand_tok_off=cand_tok_off, q_cand_off=q_cand_off,
                                         q_true_idx=q_true_idx).items()}
    st = validate(h["tok_target"] if h["tok_target"] is not None else np.zeros(0, np.int32),
                  h["cand_tok_off"] if h["cand_tok_off"] is not None else np.zeros(1, np.int32),
                  h["q_cand_off"] if h["q_cand_off"] is not None else np.zeros(1, np.int32),
                  prob.n_rows, prob.V, prob.d, prob.T, tok_row=h["tok_row"],
                  q_true_idx=h["q_true_idx"], h_dtype=prob.h_dtype, w_dtype=prob.w_dtype)
    if st != 0:
        raise JetError(st, f"{where} (JET_DEBUG_VALIDATE)")


def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _enter_stream(stream, *tensors) -> None:
    """Before enqueueing library work on `stream` (a torch stream or a raw hipStream_t):
    when it is not the current stream, order it after the current stream's work (where the
    tensors handed to the library were allocated and initialised) and record the tensors'
    use on it, so that torch neither overwrites them early nor frees them before it ends."""
    if stream is None:
        return
    cur = torch.cuda.current_stream()
    if not isinstance(stream, torch.cuda.Stream):
        h = int(stream)
        if h == 0 or h == cur.cuda_stream:
            return
        stream = torch.cuda.ExternalStream(h)
    elif stream == cur:
        return
    stream.wait_stream(cur)
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(stream)


class Workspace:
    """A reusable device workspace (grown on demand, 256-byte aligned)."""

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None
        self.base = 0
        self.size = 0

    def get(self, nbytes: int) -> tuple[int, int]:
        if nbytes > self.size:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
            addr = self.buf.data_ptr()
            self.base = (addr + 255) & ~255
            self.size = nbytes
        return self.base, self.size


# Default workspaces, one per (device, stream): the library's calls on one stream run in
# order and may share scratch memory, while calls on different streams may overlap, so
# each stream gets its own.
_default_ws: dict = {}


def _workspace(ws, device, stream=None) -> Workspace:
    if ws is not None:
        return ws
    key = (str(torch.device(device)), _stream_handle(stream) or 0)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def make_problem(H, W, tok_target, cand_tok_off, q_cand_off, T=1.0, tok_row=None,
                 cand_text_id=None, q_gold_text_id=None, q_true_idx=None) -> JetProblem:
    dev = W.device
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [n_rows, d] and W [V, d]")
    if not H.is_contiguous() or not W.is_contiguous() or H.device != dev:
        raise TypeError("H and W must be contiguous tensors on one device")
    for name, t in (("tok_target", tok_target), ("cand_tok_off", cand_tok_off),
                    ("q_cand_off", q_cand_off), ("tok_row", tok_row), ("cand_text_id", cand_text_id),
                    ("q_gold_text_id", q_gold_text_id), ("q_true_idx", q_true_idx)):
        _check_i32(name, t, dev)
    p = JetProblem()
    p.H, p.h_dtype, p.n_rows = _ptr(H), _dtype_code(H), H.shape[0]
    p.W, p.w_dtype, p.V, p.d = _ptr(W), _dtype_code(W), W.shape[0], W.shape[1]
    p.tok_row, p.tok_target, p.n_tok = _ptr(tok_row), _ptr(tok_target), tok_target.numel()
    p.cand_tok_off, p.n_cand = _ptr(cand_tok_off), cand_tok_off.numel() - 1
    p.q_cand_off, p.n_q = _ptr(q_cand_off), q_cand_off.numel() - 1
    p.cand_text_id, p.q_gold_text_id, p.q_true_idx = (_ptr(cand_text_id), _ptr(q_gold_text_id),
                                                      _ptr(q_true_idx))
    p.T = float(T)
    return p


def build_predictor_trie(tok_target, cand_tok_off, q_cand_off):
    """Host history trie (see jet_build_predictor_trie): returns (tok_node, node_tok) as
    int32 numpy arrays; raises JetError on malformed input."""
    tg = np.ascontiguousarray(np.asarray(tok_target), dtype=np.int32)
    co = np.ascontiguousarray(np.asarray(cand_tok_off), dtype=np.int32)
    qo = np.ascontiguousarray(np.asarray(q_cand_off), dtype=np.int32)
    n_tok = int(co[-1]) if len(co) else 0
    tok_node = np.empty(max(n_tok, 1), np.int32)
    node_tok = np.empty(max(n_tok, 1), np.int32)
    nn = ctypes.c_int32(0)
    st = _lib.load().jet_build_predictor_trie(tg.ctypes.data, co.ctypes.data, len(co) - 1,
                                              qo.ctypes.data, len(qo) - 1, tok_node.ctypes.data,
                                              node_tok.ctypes.data, ctypes.byref(nn))
    if st != 0:
        raise _lib.JetError(st, "jet_build_predictor_trie")
    return tok_node[:n_tok].copy(), node_tok[:nn.value].copy()


def decision_sensitivity(z: torch.Tensor, z_skip: torch.Tensor, seg_off: torch.Tensor, k: int,
                         eps: float = 1e-8, stream=None) -> dict:
    """Layer-skip sensitivity on the device (see jet_decision_sensitivity): z [n_values] and
    z_skip [n_layers, n_values] float32, seg_off [n_inputs + 1] int32, all on one device.
    Returns d [n_layers, n_inputs], J [n_layers], selected [k] and dev_flags [1]."""
    dev = z.device
    if z.dtype != torch.float32 or z_skip.dtype != torch.float32 or z.dim() != 1 or \
            z_skip.dim() != 2 or z_skip.shape[1] != z.shape[0] or not z.is_contiguous() or \
            not z_skip.is_contiguous() or z_skip.device != dev:
        raise TypeError("z [n_values] and z_skip [n_layers, n_values]: contiguous float32, one device")
    _check_i32("seg_off", seg_off, dev)
    L, n_in = int(z_skip.shape[0]), int(seg_off.numel()) - 1
    out = dict(d=torch.empty(L, max(n_in, 0), dtype=torch.float32, device=dev),
               J=torch.empty(L, dtype=torch.float32, device=dev),
               selected=torch.empty(max(k, 1), dtype=torch.int32, device=dev),
               dev_flags=torch.empty(1, dtype=torch.int32, device=dev))
    _enter_stream(stream, z, z_skip, seg_off, *out.values())
    sh = _stream_handle(stream)
    st = _lib.load().jet_decision_sensitivity(
        _ptr(z), _ptr(z_skip), _ptr(seg_off), n_in, int(z.numel()), L, float(eps), int(k),
        _ptr(out["d"]), _ptr(out["J"]), _ptr(out["selected"]), _ptr(out["dev_flags"]), sh)
    if st != 0:
        raise JetError(st, "jet_decision_sensitivity")
    out["selected"] = out["selected"][:k]
    return out


def fit_temperature(cand_s: torch.Tensor, q_cand_off: torch.Tensor, cand_text_id: torch.Tensor,
                    q_gold_text_id: torch.Tensor, T_min: float = 1e-2, T_max: float = 1e2,
                    stream=None) -> dict:
    """Fit the candidate-score temperature on the device (see jet_fit_temperature).
    Returns T [1], nll [1] and dev_flags [1] (device tensors)."""
    dev = cand_s.device
    if cand_s.dtype != torch.float32 or not cand_s.is_contiguous():
        raise TypeError("cand_s must be a contiguous float32 tensor")
    for name, t in (("q_cand_off", q_cand_off), ("cand_text_id", cand_text_id),
                    ("q_gold_text_id", q_gold_text_id)):
        _check_i32(name, t, dev)
    out = dict(T=torch.empty(1, dtype=torch.float32, device=dev),
               nll=torch.empty(1, dtype=torch.float32, device=dev),
               dev_flags=torch.empty(1, dtype=torch.int32, device=dev))
    lib = _lib.load()
    n_q = int(q_cand_off.numel()) - 1
    need = int(lib.jet_fit_temperature_workspace_size(max(n_q, 1)))
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    base = (ws.data_ptr() + 255) & ~255
    _enter_stream(stream, cand_s, q_cand_off, cand_text_id, q_gold_text_id, ws, *out.values())
    st = lib.jet_fit_temperature(
        _ptr(cand_s), _ptr(q_cand_off), n_q, int(cand_s.numel()),
        _ptr(cand_text_id), _ptr(q_gold_text_id), float(T_min), float(T_max), _ptr(out["T"]),
        _ptr(out["nll"]), _ptr(out["dev_flags"]), base, need, _stream_handle(stream))
    out["_workspace"] = ws  # keeps the workspace alive until the caller drops the result
    if st != 0:
        raise JetError(st, "jet_fit_temperature")
    return out


def projection_kernel(prob: JetProblem) -> str | None:
    """Name of the projection kernel jet_score launches for this problem (None if invalid)."""
    r = _lib.load().jet_projection_kernel(ctypes.byref(prob))
    return r.decode() if r else None


def stream_read(buf, out, stream=None) -> None:
    """Read every byte of the device tensor buf once (jet_stream_read); XOR a checksum of its
    words into out (a one-element int32 device tensor).  Measurement helper."""
    nbytes = buf.numel() * buf.element_size()
    _enter_stream(stream, buf, out)
    st = _stream_handle(stream)
    rc = _lib.load().jet_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), st)
    if rc != 0:
        raise JetError(rc, "jet_stream_read")


def score_workspace_size(prob: JetProblem) -> int:
    return int(_lib.load().jet_score_workspace_size(ctypes.byref(prob)))


def alloc_outputs(prob: JetProblem, device, optional: bool = True) -> dict:
    f = lambda n: torch.empty(max(n, 0), dtype=torch.float32, device=device)  # noqa: E731
    out = dict(tok_logp=f(prob.n_tok), cand_s=f(prob.n_cand), cand_q=f(prob.n_cand),
               q_argmax=torch.empty(max(prob.n_q, 0), dtype=torch.int32, device=device))
    if optional:
        out.update(row_lse=f(prob.n_rows), q_true=f(prob.n_q), q_expect=f(prob.n_q),
                   q_gold_nll=f(prob.n_q), q_confidence=f(prob.n_q), q_mass=f(prob.n_q),
                   dev_flags=torch.zeros(1, dtype=torch.int32, device=device))
    return out


def _outputs_struct(out: dict) -> JetOutputs:
    o = JetOutputs()
    for name, _ in JetOutputs._fields_:
        setattr(o, name, _ptr(out.get(name)))
    return o


def score(H, W, tok_target, cand_tok_off, q_cand_off, T=1.0, tok_row=None, cand_text_id=None,
          q_gold_text_id=None, q_true_idx=None, *, out=None, workspace=None, stream=None,
          events=None, optional=True) -> dict:
    """jet_score on device tensors.  Returns a dict of output tensors (allocated unless
    `out` is given).  events: optional (before, after) raw hipEvent_t handles recorded
    around the projection kernel.  Without `workspace` the call uses this module's
    workspace for its (device, stream): calls on different streams never share scratch
    memory; a caller-supplied workspace must not be used by two streams at once."""
    prob = make_problem(H, W, tok_target, cand_tok_off, q_cand_off, T, tok_row, cand_text_id,
                        q_gold_text_id, q_true_idx)
    lib = _lib.load()
    need = int(lib.jet_score_workspace_size(ctypes.byref(prob)))
    if out is None:
        out = alloc_outputs(prob, W.device, optional)
    o = _outputs_struct(out)
    sh = _stream_handle(stream)
    if need == 0:  # invalid scalars: jet_score reports which check failed, enqueuing nothing
        raise JetError(lib.jet_score(ctypes.byref(prob), ctypes.byref(o), None, 0, sh), "jet_score")
    if debug_validate():
        _validate_score_on_host(prob, tok_row, tok_target, cand_tok_off, q_cand_off, q_true_idx,
                                "jet_score")
    ws = _workspace(workspace, W.device, stream)
    base, size = ws.get(need)
    _enter_stream(stream, H, W, tok_target, cand_tok_off, q_cand_off, tok_row, cand_text_id,
                  q_gold_text_id, q_true_idx, ws.buf, *out.values())
    if events is None:
        st = lib.jet_score(ctypes.byref(prob), ctypes.byref(o), base, size, sh)
    else:
        st = lib.jet_score_profiled(ctypes.byref(prob), ctypes.byref(o), base, size, sh,
                                    events[0], events[1])
    if st != 0:
        raise JetError(st, "jet_score")
    return out


def score_noalloc(H, W, tok_target, cand_tok_off, q_cand_off, T=1.0, tok_row=None,
                  cand_text_id=None, q_gold_text_id=None, q_true_idx=None, *, out,
                  stream=None) -> dict:
    """jet_score_noalloc on device tensors: jet_score with the library's static workspace
    (no workspace argument; nothing allocated here either, so `out` must be given, e.g.
    from alloc_outputs ahead of time).  Calls that overlap on one GPU race on that
    workspace; calls ordered on one stream do not."""
    prob = make_problem(H, W, tok_target, cand_tok_off, q_cand_off, T, tok_row, cand_text_id,
                        q_gold_text_id, q_true_idx)
    o = _outputs_struct(out)
    if debug_validate():
        _validate_score_on_host(prob, tok_row, tok_target, cand_tok_off, q_cand_off, q_true_idx,
                                "jet_score_noalloc")
    _enter_stream(stream, H, W, tok_target, cand_tok_off, q_cand_off, tok_row, cand_text_id,
                  q_gold_text_id, q_true_idx, *out.values())
    st = _lib.load().jet_score_noalloc(ctypes.byref(prob), ctypes.byref(o), _stream_handle(stream))
    if st != 0:
        raise JetError(st, "jet_score_noalloc")
    return out


def validate(tok_target: np.ndarray, cand_tok_off: np.ndarray, q_cand_off: np.ndarray, n_rows: int,
             V: int, d: int, T: float = 1.0, tok_row=None, q_true_idx=None, h_dtype: int = 0,
             w_dtype: int = 1) -> int:
    """jet_validate_host on HOST index arrays (numpy int32).  Returns the status code."""
    keep = []

    def hp(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.int32)
        keep.append(a)
        return a.ctypes.data

    dummy = np.zeros(4, dtype=np.float32)  # H, W are not read; non-NULL, aligned stand-ins
    keep.append(dummy)
    p = JetProblem()
    p.H, p.h_dtype, p.n_rows = dummy.ctypes.data, h_dtype, n_rows
    p.W, p.w_dtype, p.V, p.d = dummy.ctypes.data, w_dtype, V, d
    p.tok_row, p.tok_target, p.n_tok = hp(tok_row), hp(tok_target), len(tok_target)
    p.cand_tok_off, p.n_cand = hp(cand_tok_off), len(cand_tok_off) - 1
    p.q_cand_off, p.n_q = hp(q_cand_off), len(q_cand_off) - 1
    p.q_true_idx = hp(q_true_idx)
    p.T = float(T)
    return int(_lib.load().jet_validate_host(ctypes.byref(p)))


def build_union(field_ids: np.ndarray, field_off: np.ndarray, V: int):
    """jet_build_union on the host: (union_ids, slot_uidx) as numpy int32 arrays."""
    ids = np.ascontiguousarray(field_ids, dtype=np.int32)
    off = np.ascontiguousarray(field_off, dtype=np.int32)
    n = int(off[-1]) if len(off) else 0
    union = np.zeros(max(n, 1), dtype=np.int32)
    slot = np.zeros(max(n, 1), dtype=np.int32)
    nu = ctypes.c_int32(0)
    st = _lib.load().jet_build_union(ids.ctypes.data if n else None, off.ctypes.data, len(off) - 1,
                                     int(V), union.ctypes.data, ctypes.byref(nu), slot.ctypes.data)
    if st != 0:
        raise JetError(st, "jet_build_union")
    return union[:nu.value].copy(), slot[:n].copy()


def make_restricted_problem(H, W, union_ids, field_row, field_slot_off, slot_uidx,
                            T=1.0) -> JetRestrictedProblem:
    dev = W.device
    for name, t in (("union_ids", union_ids), ("field_row", field_row),
                    ("field_slot_off", field_slot_off), ("slot_uidx", slot_uidx)):
        _check_i32(name, t, dev)
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [n_rows, d] and W [V, d]")
    p = JetRestrictedProblem()
    p.H, p.h_dtype, p.n_rows = _ptr(H), _dtype_code(H), H.shape[0]
    p.W, p.w_dtype, p.V, p.d = _ptr(W), _dtype_code(W), W.shape[0], W.shape[1]
    p.union_ids, p.n_union = _ptr(union_ids), union_ids.numel()
    p.field_row, p.field_slot_off, p.slot_uidx = _ptr(field_row), _ptr(field_slot_off), _ptr(slot_uidx)
    p.n_fields, p.n_slots = field_slot_off.numel() - 1, slot_uidx.numel()
    p.T = float(T)
    return p


def score_restricted(H, W, union_ids, field_row, field_slot_off, slot_uidx, T=1.0, *, out=None,
                     workspace=None, stream=None) -> dict:
    """jet_score_restricted on device tensors: slot_logit, slot_q, field_argmax, dev_flags.
    Without `workspace` the call uses this module's workspace for its (device, stream)."""
    prob = make_restricted_problem(H, W, union_ids, field_row, field_slot_off, slot_uidx, T)
    lib = _lib.load()
    need = int(lib.jet_restricted_workspace_size(ctypes.byref(prob)))
    dev = W.device
    if out is None:
        out = dict(slot_logit=torch.empty(prob.n_slots, dtype=torch.float32, device=dev),
                   slot_q=torch.empty(prob.n_slots, dtype=torch.float32, device=dev),
                   field_argmax=torch.empty(prob.n_fields, dtype=torch.int32, device=dev),
                   dev_flags=torch.zeros(1, dtype=torch.int32, device=dev))
    o = JetRestrictedOutputs()
    for name, _ in JetRestrictedOutputs._fields_:
        setattr(o, name, _ptr(out.get(name)))
    if need == 0:  # invalid scalars: the entry point reports which check failed
        raise JetError(lib.jet_score_restricted(ctypes.byref(prob), ctypes.byref(o), None, 0,
                                                _stream_handle(stream)), "jet_score_restricted")
    if debug_validate():
        hv = [_host_i32(t) for t in (union_ids, field_row, field_slot_off, slot_uidx)]
        st = validate_restricted(*hv, n_rows=prob.n_rows, V=prob.V, d=prob.d, T=prob.T,
                                 h_dtype=prob.h_dtype, w_dtype=prob.w_dtype)
        if st != 0:
            raise JetError(st, "jet_score_restricted (JET_DEBUG_VALIDATE)")
    ws = _workspace(workspace, dev, stream)
    base, size = ws.get(need)
    _enter_stream(stream, H, W, union_ids, field_row, field_slot_off, slot_uidx, ws.buf,
                  *out.values())
    st = lib.jet_score_restricted(ctypes.byref(prob), ctypes.byref(o), base, size,
                                  _stream_handle(stream))
    if st != 0:
        raise JetError(st, "jet_score_restricted")
    return out


def restricted_workspace_size(prob: JetRestrictedProblem) -> int:
    return int(_lib.load().jet_restricted_workspace_size(ctypes.byref(prob)))


def validate_restricted(union_ids, field_row, field_slot_off, slot_uidx, n_rows: int, V: int, d: int,
                        T: float = 1.0, h_dtype: int = 0, w_dtype: int = 1) -> int:
    """jet_validate_restricted_host on HOST arrays.  Returns the status code."""
    keep = []

    def hp(a):
        a = np.ascontiguousarray(a, dtype=np.int32)
        keep.append(a)
        return a.ctypes.data

    dummy = np.zeros(4, dtype=np.float32)
    p = JetRestrictedProblem()
    p.H, p.h_dtype, p.n_rows = dummy.ctypes.data, h_dtype, n_rows
    p.W, p.w_dtype, p.V, p.d = dummy.ctypes.data, w_dtype, V, d
    p.union_ids, p.n_union = hp(union_ids), len(union_ids)
    p.field_row, p.field_slot_off, p.slot_uidx = hp(field_row), hp(field_slot_off), hp(slot_uidx)
    p.n_fields, p.n_slots = len(field_slot_off) - 1, len(slot_uidx)
    p.T = float(T)
    return int(_lib.load().jet_validate_restricted_host(ctypes.byref(p)))
