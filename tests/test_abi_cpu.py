"""C ABI checks that need no GPU: the library loads, exports every declared symbol, the
ctypes structs match the C layout, host validation and the union builder behave, and
invalid scalars are rejected before anything touches the device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as jo
import workloads as wl
from candidate_likelihood_scoring_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jet.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"JET_API\s+[\w\s\*]+?\b(jet_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (jet_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(_lib.EXPORTS), "ctypes table out of sync with include/jet.h"
    for n in names:
        assert getattr(lib, n) is not None


_STRUCTS = {
    "jet_problem": _lib.JetProblem, "jet_outputs": _lib.JetOutputs,
    "jet_restricted_problem": _lib.JetRestrictedProblem,
    "jet_restricted_outputs": _lib.JetRestrictedOutputs,
}


def test_struct_layout_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in _STRUCTS.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-o", str(exe), str(src)], check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    for line in got:
        if not line:
            continue
        cname, field, val = line.split()
        cls = _STRUCTS[cname]
        want = ctypes.sizeof(cls) if field == "sizeof" else getattr(cls, field).offset
        assert int(val) == want, (cname, field, val, want)


def test_status_strings(lib):
    for code in range(-7, 1):
        assert lib.jet_status_string(code)


def _p(**kw):
    p = wl.make_problem(V=50, d=32, n_q=3, K=(1, 4), lengths=(1, 3), layout="prefix", seed=3, **kw)
    return p


def _validate(p, **over):
    args = dict(tok_target=p["tok_target"], cand_tok_off=p["cand_tok_off"], q_cand_off=p["q_cand_off"],
                n_rows=p["n_rows"], V=p["V"], d=p["d"], T=p["T"], tok_row=p["tok_row"],
                q_true_idx=p.get("q_true_idx"), h_dtype=0, w_dtype=1)
    args.update(over)
    return api.validate(**args)


def test_validate_host_accepts_generated_problems():
    for name in ("tiny", "tiny_tie", "binary_enum", "multi_token", "large_batch"):
        p = wl.make_config(name, with_weights=False)
        w_dtype = 0 if p["w_dtype"] == "f32" else 1
        h_dtype = 0 if p["h_dtype"] == "f32" else 1
        assert _validate(p, h_dtype=h_dtype, w_dtype=w_dtype) == 0, name


def test_validate_host_rejects_bad_indices():
    p = _p()
    E_INDEX, E_SHAPE, E_TEMP, E_DTYPE = -4, -2, -5, -3
    t = p["tok_target"].copy(); t[0] = p["V"]
    assert _validate(p, tok_target=t) == E_INDEX
    t = p["tok_target"].copy(); t[-1] = -1
    assert _validate(p, tok_target=t) == E_INDEX
    r = p["tok_row"].copy(); r[1] = p["n_rows"]
    assert _validate(p, tok_row=r) == E_INDEX
    c = p["cand_tok_off"].copy(); c[1] = c[0]
    assert _validate(p, cand_tok_off=c) == E_INDEX  # empty candidate (m_c = 0)
    c = p["cand_tok_off"].copy(); c[-1] += 1
    assert _validate(p, cand_tok_off=c, tok_target=np.append(p["tok_target"], 0),
                     tok_row=np.append(p["tok_row"], 0)) == 0
    q = p["q_cand_off"].copy(); q[1] = 0
    assert _validate(p, q_cand_off=q) == E_INDEX  # empty question (K = 0)
    K = np.diff(p["q_cand_off"])
    assert _validate(p, q_true_idx=np.full(len(K), -1, np.int32)) == 0
    assert _validate(p, q_true_idx=K.astype(np.int32)) == E_INDEX
    assert _validate(p, T=0.0) == E_TEMP
    assert _validate(p, T=float("nan")) == E_TEMP
    assert _validate(p, T=float("inf")) == E_TEMP
    assert _validate(p, d=48) == E_SHAPE
    assert _validate(p, V=0) == E_SHAPE
    assert _validate(p, h_dtype=1, w_dtype=0) == E_DTYPE


def test_build_union_matches_oracle():
    rng = np.random.default_rng(2)
    for trial in range(5):
        n_f = int(rng.integers(1, 40))
        K = rng.integers(1, 27, size=n_f)
        off = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
        ids = rng.integers(0, 1000, size=int(off[-1])).astype(np.int32)
        u, s = api.build_union(ids, off, 1000)
        ou, os_ = jo.build_union(ids, off, 1000)
        assert np.array_equal(u, ou) and np.array_equal(s, os_)
    for name in ("restricted", "restricted_max"):
        rp = wl.make_config(name, with_weights=False)
        u, s = api.build_union(rp["field_ids"], rp["field_off"], rp["V"])
        ou, os_ = jo.build_union(rp["field_ids"], rp["field_off"], rp["V"])
        assert np.array_equal(u, ou) and np.array_equal(s, os_)
    assert len(api.build_union(wl.make_config("restricted_max", with_weights=False)["field_ids"],
                               wl.make_config("restricted_max", with_weights=False)["field_off"],
                               248320)[0]) == 832
    with pytest.raises(_lib.JetError):
        api.build_union(np.array([1, 1000], np.int32), np.array([0, 2], np.int32), 1000)
    with pytest.raises(_lib.JetError):
        api.build_union(np.array([1, 2], np.int32), np.array([0, 0, 2], np.int32), 1000)


def test_validate_restricted_host():
    union = np.array([2, 5, 9], np.int32)
    ok = dict(union_ids=union, field_row=np.array([0, 1], np.int32),
              field_slot_off=np.array([0, 2, 3], np.int32), slot_uidx=np.array([0, 2, 1], np.int32),
              n_rows=2, V=10, d=32)
    assert api.validate_restricted(**ok) == 0
    assert api.validate_restricted(**{**ok, "union_ids": np.array([2, 2, 9], np.int32)}) == -4
    assert api.validate_restricted(**{**ok, "slot_uidx": np.array([0, 3, 1], np.int32)}) == -4
    assert api.validate_restricted(**{**ok, "field_row": np.array([0, 2], np.int32)}) == -4
    assert api.validate_restricted(**{**ok, "T": -1.0}) == -5


def test_score_rejects_invalid_scalars_without_a_device(lib):
    """Scalar and workspace checks return before any device call, so they run here."""
    h = np.zeros(64, np.float32)
    p = _lib.JetProblem()
    p.H, p.h_dtype, p.n_rows = h.ctypes.data, 0, 1
    p.W, p.w_dtype, p.V, p.d = h.ctypes.data, 1, 2, 32
    tgt = np.zeros(1, np.int32)
    off = np.array([0, 1], np.int32)
    p.tok_target, p.n_tok = tgt.ctypes.data, 1
    p.cand_tok_off, p.n_cand = off.ctypes.data, 1
    p.q_cand_off, p.n_q = off.ctypes.data, 1
    p.T = 1.0
    o = _lib.JetOutputs()
    f = np.zeros(4, np.float32)
    o.tok_logp = o.cand_s = o.cand_q = o.q_argmax = f.ctypes.data
    assert lib.jet_score_workspace_size(ctypes.byref(p)) > 0
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -6
    p.T = -1.0
    assert lib.jet_score_workspace_size(ctypes.byref(p)) == 0
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -5
    p.T = 1.0
    p.d = 40
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -2
    p.d = 32
    p.w_dtype, p.h_dtype = 0, 1
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -3
    p.w_dtype, p.h_dtype = 1, 0
    o.cand_q = None
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -1
    o.cand_q = f.ctypes.data
    p.n_cand = 0  # fewer candidates than questions: a question would be empty
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -2
    p.n_cand = 1
    # the offset arrays end at n_cand and n_tok: candidates without a question, or tokens
    # without a candidate, are a shape error
    p.n_q = 0
    assert lib.jet_score_workspace_size(ctypes.byref(p)) == 0
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -2
    p.n_cand = 0
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), None, 0, None) == -2
    p.n_tok = 0
    assert lib.jet_score_workspace_size(ctypes.byref(p)) > 0  # rows only: LSE per row
    p.n_tok, p.n_cand, p.n_q = 1, 1, 1
    ws = np.zeros(1 << 20, np.uint8)
    mis = ws.ctypes.data + 1
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), mis, 1 << 19, None) == -6


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="launches on fake pointers only where no GPU exists")
def test_failed_launch_returns_hip_status(lib):
    """A problem that passes every host check reaches its first launch; with no GPU present
    that launch fails, and each device entry point reports JET_E_HIP (the status that may
    follow work the same call already enqueued) rather than crashing."""
    h = np.zeros(64, np.float32)
    p = _lib.JetProblem()
    p.H, p.h_dtype, p.n_rows = h.ctypes.data, 0, 1
    p.W, p.w_dtype, p.V, p.d = h.ctypes.data, 1, 2, 32
    tgt = np.zeros(1, np.int32)
    off = np.array([0, 1], np.int32)
    p.tok_target, p.n_tok = tgt.ctypes.data, 1
    p.cand_tok_off, p.n_cand = off.ctypes.data, 1
    p.q_cand_off, p.n_q = off.ctypes.data, 1
    p.T = 1.0
    o = _lib.JetOutputs()
    f = np.zeros(4, np.float32)
    o.tok_logp = o.cand_s = o.cand_q = o.q_argmax = f.ctypes.data
    need = lib.jet_score_workspace_size(ctypes.byref(p))
    ws = np.zeros(need + 512, np.uint8)
    base = (ws.ctypes.data + 255) & ~255
    assert lib.jet_score(ctypes.byref(p), ctypes.byref(o), base, need, None) == -7
    assert lib.jet_score_profiled(ctypes.byref(p), ctypes.byref(o), base, need, None, None, None) == -7
    rp = _lib.JetRestrictedProblem()
    rp.H, rp.h_dtype, rp.n_rows = h.ctypes.data, 0, 1
    rp.W, rp.w_dtype, rp.V, rp.d = h.ctypes.data, 1, 2, 32
    uid = np.zeros(1, np.int32)
    rp.union_ids, rp.n_union = uid.ctypes.data, 1
    rp.field_row, rp.field_slot_off, rp.slot_uidx = uid.ctypes.data, off.ctypes.data, uid.ctypes.data
    rp.n_fields, rp.n_slots, rp.T = 1, 1, 1.0
    ro = _lib.JetRestrictedOutputs()
    ro.slot_logit = ro.slot_q = ro.field_argmax = f.ctypes.data
    rneed = lib.jet_restricted_workspace_size(ctypes.byref(rp))
    rws = np.zeros(rneed + 512, np.uint8)
    rbase = (rws.ctypes.data + 255) & ~255
    assert lib.jet_score_restricted(ctypes.byref(rp), ctypes.byref(ro), rbase, rneed, None) == -7


def test_debug_validate_checks_host_copies(monkeypatch):
    """JET_DEBUG_VALIDATE=1 copies the index arrays to the host and validates them before
    a call (here on CPU tensors, nothing is launched): a good problem passes, an
    out-of-range target, row or true index raises JetError with JET_E_INDEX."""
    import torch

    p = wl.make_problem(V=300, d=32, n_q=5, K=(2, 4), lengths=(1, 3), layout="prefix", seed=44)
    t = {k: torch.from_numpy(np.asarray(p[k])) for k in ("tok_target", "cand_tok_off", "q_cand_off", "tok_row")}
    H = torch.zeros(p["n_rows"], 32, dtype=torch.float32)
    W = torch.zeros(300, 32, dtype=torch.bfloat16)
    monkeypatch.setenv("JET_DEBUG_VALIDATE", "1")
    assert api.debug_validate()
    prob = api.make_problem(H, W, t["tok_target"], t["cand_tok_off"], t["q_cand_off"], tok_row=t["tok_row"])
    api._validate_score_on_host(prob, t["tok_row"], t["tok_target"], t["cand_tok_off"], t["q_cand_off"],
                                None, "test")
    for name, idx, val in (("tok_target", 2, 300), ("tok_row", 1, p["n_rows"])):
        bad = t[name].clone()
        bad[idx] = val
        args = dict(t, **{name: bad})
        with pytest.raises(_lib.JetError) as e:
            api._validate_score_on_host(prob, args["tok_row"], args["tok_target"], args["cand_tok_off"],
                                        args["q_cand_off"], None, "test")
        assert e.value.status == -4
    K = np.diff(p["q_cand_off"])
    with pytest.raises(_lib.JetError):
        api._validate_score_on_host(prob, t["tok_row"], t["tok_target"], t["cand_tok_off"], t["q_cand_off"],
                                    torch.from_numpy((K + 1).astype(np.int32)), "test")
    monkeypatch.setenv("JET_DEBUG_VALIDATE", "0")
    assert not api.debug_validate()


def test_workspace_size_is_monotone_in_problem_size(lib):
    sizes = []
    for n_rows in (1, 32, 33, 1000):
        p = _lib.JetProblem()
        h = np.zeros(16, np.float32)
        p.H, p.h_dtype, p.n_rows = h.ctypes.data, 0, n_rows
        p.W, p.w_dtype, p.V, p.d = h.ctypes.data, 1, 248320, 2560
        p.T = 1.0
        sizes.append(lib.jet_score_workspace_size(ctypes.byref(p)))
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)


def test_restricted_one_launch_limits(lib):
    """The restricted plan (host-only call): d <= 16384 and at most 4096 slots take the
    one-launch per-field kernel, whose only workspace is the flag word (256 bytes), for
    either head dtype; past either limit the projection keeps its partial sums (bf16 head,
    one [n_union][n_rows] plane per 512-wide k group) or its gathered rows and logits (fp32
    head) in the workspace."""
    h = np.zeros(16, np.float32)

    def need(d, n_slots, w_dtype=1, n_union=100, n_rows=32):
        rp = _lib.JetRestrictedProblem()
        rp.H, rp.h_dtype, rp.n_rows = h.ctypes.data, 0, n_rows
        rp.W, rp.w_dtype, rp.V, rp.d = h.ctypes.data, w_dtype, 248320, d
        rp.union_ids, rp.n_union = h.ctypes.data, n_union
        rp.field_row = rp.field_slot_off = rp.slot_uidx = h.ctypes.data
        rp.n_fields, rp.n_slots, rp.T = 32, n_slots, 2.0
        return lib.jet_restricted_workspace_size(ctypes.byref(rp))

    for w_dtype in (1, 0):
        for d in (32, 1024, 2560, 2592, 4096, 16384):
            assert need(d, 832, w_dtype) == 256, (d, w_dtype)
        assert need(16384, 4096, w_dtype) == 256
    # past the limits: 256-byte aligned partial planes (or gathered rows and logits), then
    # the flag word
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need(16416, 832) == al(33 * 100 * 32 * 4) + 256
    assert need(2560, 4097) == al(5 * 100 * 32 * 4) + 256
    assert need(16416, 832, w_dtype=0) == al(100 * 16416 * 4) + al(100 * 32 * 4) + 256
    assert need(64, 4097, w_dtype=0) == al(100 * 64 * 4) + al(100 * 32 * 4) + 256


def test_restricted_slots_without_fields_rejected(lib):
    """The field offsets end at n_slots, so slots without a field are a shape error (host
    check, no device needed); no slots and no fields is a valid empty problem."""
    h = np.zeros(16, np.float32)
    rp = _lib.JetRestrictedProblem()
    rp.H, rp.h_dtype, rp.n_rows = h.ctypes.data, 0, 4
    rp.W, rp.w_dtype, rp.V, rp.d = h.ctypes.data, 1, 1000, 64
    rp.union_ids, rp.n_union = h.ctypes.data, 3
    rp.field_row = rp.field_slot_off = rp.slot_uidx = h.ctypes.data
    rp.n_fields, rp.n_slots, rp.T = 0, 3, 1.0
    assert lib.jet_restricted_workspace_size(ctypes.byref(rp)) == 0
    ro = _lib.JetRestrictedOutputs()
    assert lib.jet_score_restricted(ctypes.byref(rp), ctypes.byref(ro), None, 0, None) == -2
    rp.n_slots = 0
    assert lib.jet_restricted_workspace_size(ctypes.byref(rp)) > 0


def test_projection_kernel_choice(lib):
    """The plan's kernel choice depends only on the problem's scalars (host-only call)."""
    from candidate_likelihood_scoring_amd import api

    h = np.zeros(16, np.float32)

    def pick(n_rows, V, d, h_dtype, w_dtype, T=1.0):
        p = _lib.JetProblem()
        p.H, p.h_dtype, p.n_rows = h.ctypes.data, h_dtype, n_rows
        p.W, p.w_dtype, p.V, p.d = h.ctypes.data, w_dtype, V, d
        p.T = T
        return api.projection_kernel(p)

    F32, BF16 = 0, 1
    assert pick(26546, 248320, 2560, BF16, BF16) == "k_project_tiled_m16"
    assert pick(3330, 262144, 1536, F32, BF16) == "k_project_tiled_m16x2"
    assert pick(3330, 262144, 192, F32, BF16) == "k_project_tiled_m16x2"  # three 64-wide stages
    assert pick(3330, 49152, 960, BF16, BF16) == "k_project_tiled_m16"      # 15 stages (d % 128 = 64)
    # one pass of the streaming kernel takes up to 64 rows of fp32 H or 128 of bf16 H
    assert pick(32, 248320, 2560, F32, BF16) == "k_project_wg_bf16"
    assert pick(64, 248320, 2560, F32, BF16) == "k_project_wg_bf16"
    assert pick(65, 248320, 2560, F32, BF16) == "k_project_tiled_m16x2"  # one padded row tile
    assert pick(128, 248320, 2560, BF16, BF16) == "k_project_wg_bf16"
    assert pick(129, 248320, 2560, BF16, BF16) == "k_project_tiled_m16"  # one padded row tile
    assert pick(255, 5000, 256, BF16, BF16) == "k_project_tiled_m16"
    assert pick(40, 5000, 192, F32, BF16) == "k_project_wg_bf16"        # a 64-wide last stage
    assert pick(65, 5000, 192, F32, BF16) == "k_project_tiled_m16x2"
    assert pick(128, 49152, 960, BF16, BF16) == "k_project_wg_bf16"
    assert pick(129, 49152, 960, BF16, BF16) == "k_project_tiled_m16"
    assert pick(32, 5000, 160, BF16, BF16) == "k_project_small_bf16"    # d not whole 64-wide stages
    assert pick(1000, 5000, 160, BF16, BF16) == "k_project_small_bf16"
    assert pick(300, 255, 256, BF16, BF16) == "k_project_wg_bf16"       # vocabulary below one tile
    assert pick(33, 255, 256, F32, BF16) == "k_project_wg_bf16"
    # fp32 head: streaming with at least 256 (256-entry group, row tile) pairs
    assert pick(32, 1000, 64, F32, F32) == "k_project_small_f32"
    assert pick(8, 32768, 256, F32, F32) == "k_project_small_f32"   # 128 groups
    assert pick(16, 65536, 96, F32, F32) == "k_project_wg_f32"      # 256 groups, one 16-row tile
    assert pick(17, 65280, 96, F32, F32) == "k_project_small_f32"   # 255 groups, one 32-row tile
    assert pick(33, 32768, 256, F32, F32) == "k_project_wg_f32"     # 128 groups x 2 row tiles
    assert pick(5000, 1000, 96, F32, F32) == "k_project_wg_f32"     # 4 groups x 157 row tiles
    # operands past 4 GiB keep the matrix-core kernels (offsets local to each workgroup)
    assert pick(300, 262144, 8192, BF16, BF16) == "k_project_tiled_m16"   # head of 4 GiB
    assert pick(300, 300007, 8192, BF16, BF16) == "k_project_tiled_m16"   # 4.9 GB head
    assert pick(300, 262144, 8192, F32, BF16) == "k_project_tiled_m16x2"
    assert pick(270000, 4099, 8192, BF16, BF16) == "k_project_tiled_m16"  # 4.4 GB of H
    assert pick(2 ** 21, 262144, 8192, F32, BF16) == "k_project_tiled_m16x2"
    assert pick(32, 1000, 64, F32, BF16, T=-1.0) is None


def test_predictor_trie_matches_oracle():
    """The library's history trie (host call) equals the oracle's, bit for bit."""
    import oracle as jo
    from candidate_likelihood_scoring_amd import api

    rng = np.random.default_rng(11)
    for trial in range(30):
        n_q = int(rng.integers(1, 6))
        tg, co, qo = [], [0], [0]
        for g in range(n_q):
            for c in range(int(rng.integers(1, 9))):
                m = int(rng.integers(1, 6))
                tg.extend(int(x) for x in rng.integers(0, 1 + trial % 4, size=m))
                co.append(len(tg))
            qo.append(len(co) - 1)
        tn, nt = api.build_predictor_trie(tg, co, qo)
        rtn, rnt = jo.predictor_trie(tg, co, qo)
        assert np.array_equal(tn, rtn) and np.array_equal(nt, rnt)
    p = wl.multi_token()
    tn, nt = api.build_predictor_trie(p["tok_target"], p["cand_tok_off"], p["q_cand_off"])
    rtn, rnt = jo.predictor_trie(p["tok_target"], p["cand_tok_off"], p["q_cand_off"])
    assert np.array_equal(tn, rtn) and np.array_equal(nt, rnt)


def test_predictor_trie_rejects_malformed_input():
    from candidate_likelihood_scoring_amd import api

    with pytest.raises(_lib.JetError) as e:
        api.build_predictor_trie([1, 2], [0, 2], [0, 2])      # question end != n_cand
    assert e.value.status == -2
    with pytest.raises(_lib.JetError) as e:
        api.build_predictor_trie([1, 2], [0, 2, 2], [0, 2])   # empty candidate
    assert e.value.status == -2
    with pytest.raises(_lib.JetError) as e:
        api.build_predictor_trie([1, -2], [0, 2], [0, 1])     # negative target
    assert e.value.status == -4
    lib = _lib.load()
    off = (ctypes.c_int32 * 2)(0, 0)
    n = ctypes.c_int32(0)
    assert lib.jet_build_predictor_trie(None, off, -1, off, 0, None, None, ctypes.byref(n)) == -2
    assert lib.jet_build_predictor_trie(None, off, 0, off, -1, None, None, ctypes.byref(n)) == -2
    assert lib.jet_build_predictor_trie(None, None, 0, off, 0, None, None, ctypes.byref(n)) == -1


def test_decision_sensitivity_host_checks(lib):
    """Scalar checks return before anything is enqueued, so they run without a device."""
    buf = np.zeros(64, np.float32)
    off = np.array([0, 4], np.int32)
    a = buf.ctypes.data

    def call(n_in=1, n_val=4, L=2, eps=1e-8, k=1, sel=a, z=a):
        return lib.jet_decision_sensitivity(z, a, off.ctypes.data, n_in, n_val, L, eps, k, a, a, sel,
                                            None, None)

    assert call(n_in=0) == -2
    assert call(n_val=0) == -2
    assert call(L=0) == -2 and call(L=4097) == -2
    assert call(k=3) == -2 and call(k=-1) == -2
    assert call(eps=0.0) == -2 and call(eps=float("nan")) == -2 and call(eps=float("inf")) == -2
    assert call(sel=None) == -1 and call(z=None) == -1


def test_fit_temperature_host_checks(lib):
    """Scalar checks return before anything is enqueued, so they run without a device."""
    buf = np.zeros(16, np.float32)
    a = buf.ctypes.data

    ws = np.zeros(1 << 20, np.uint8)
    w = (ws.ctypes.data + 255) & ~255

    def call(n_q=1, n_c=2, lo=0.01, hi=100.0, s=a, wsp=w, wsb=1 << 19):
        return lib.jet_fit_temperature(s, a, n_q, n_c, a, a, lo, hi, a, a, None, wsp, wsb, None)

    assert call(s=None) == -1
    assert call(n_q=0) == -2 and call(n_c=0) == -2
    assert call(lo=0.0) == -5 and call(lo=2.0, hi=1.0) == -5 and call(hi=float("inf")) == -5
    assert call(lo=float("nan")) == -5
    assert call(wsp=None) == -6 and call(wsp=w + 1) == -6 and call(wsb=16) == -6
    assert lib.jet_fit_temperature_workspace_size(0) == 0
    assert 0 < lib.jet_fit_temperature_workspace_size(10) <= lib.jet_fit_temperature_workspace_size(10 ** 6)


def test_stream_read_host_checks(lib):
    """The measurement helper rejects bad arguments before anything is enqueued."""
    E_NULL, E_SHAPE = -1, -2
    out = ctypes.c_uint32(0)
    assert lib.jet_stream_read(None, 1024, ctypes.addressof(out), None) == E_NULL
    assert lib.jet_stream_read(16, 1024, None, None) == E_NULL
    assert lib.jet_stream_read(17, 1024, ctypes.addressof(out), None) == E_SHAPE  # misaligned
    assert lib.jet_stream_read(16, 1000, ctypes.addressof(out), None) == E_SHAPE  # not 16 B whole
    assert lib.jet_stream_read(16, 0, ctypes.addressof(out), None) == 0            # nothing to read


def test_profile_digest_ignores_comments_only():
    """The counter-traffic digest changes with the kernel code, not with its comments."""
    import bench
    code = "int f(int a) {\n  return a + 1;  // one\n}\n"
    assert bench._code_only(code) == bench._code_only("/* header\n note */\n" + code.replace("// one", "// two") + "\n\n")
    assert bench._code_only(code) != bench._code_only(code.replace("a + 1", "a + 2"))
    for files in bench.KERNEL_SOURCES.values():
        assert "candidate_likelihood_scoring_amd/csrc/jet_api.hip" in files
