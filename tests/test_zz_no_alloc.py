"""jet_score_noalloc (workspace in the library's static device array) against jet_score
with a caller workspace: four calls in a row on one stream, each on a smaller problem,
each bitwise equal to jet_score's outputs and within the oracle's tolerances; a problem
whose workspace exceeds the array is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle as jo
import workloads as wl
from tests.parity import compare, log

torch = pytest.importorskip("torch")
from candidate_likelihood_scoring_amd import _lib, api, problem  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # matrix-core path (bf16 H, 15 row tiles): the larger call first
    dict(V=20011, d=256, n_q=60, K=(2, 8), lengths=(1, 6), layout="own", seed=901,
         h_dtype="bf16", n_extra_rows=2500),
    # matrix-core path with fewer rows than one row tile (fp32 H planes zero-padded)
    dict(V=6151, d=128, n_q=4, K=(1, 12), layout="field", seed=902, dups=2, n_extra_rows=96),
    # fp32 head on its streaming kernel (256 vocabulary groups, one 16-row tile)
    dict(V=65536, d=96, n_q=9, K=(1, 12), layout="field", seed=904, w_dtype="f32"),
    # streaming path, fp32 H, one row per field: smallest workspace, same array
    dict(V=6151, d=128, n_q=9, K=(1, 12), layout="field", seed=903, dups=2),
]


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def test_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available(), "needs a GPU"
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream or None
    sizes = []
    for case in CASES:
        p = wl.make_problem(**case)
        dp = problem.to_device(p, "cuda")
        prob = api.make_problem(**dp)
        need = api.score_workspace_size(prob)
        sizes.append(need)
        assert 0 < need <= _lib.NOALLOC_MAX_WORKSPACE
        ref = api.score(**dp)  # jet_score with a caller workspace
        out = api.alloc_outputs(prob, "cuda")
        for v in out.values():
            v.fill_(-3)  # stale values must not survive
        torch.cuda.synchronize()
        log(f"[gpu] noalloc {api.projection_kernel(prob)} rows={p['n_rows']} ws={need}")
        st = lib.jet_score_noalloc(ctypes.byref(prob), ctypes.byref(api._outputs_struct(out)), sh)
        assert st == 0, st
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(_bits(ref[k]), _bits(out[k])), k
        errs = compare(p, {k: v.cpu().numpy() for k, v in out.items()}, jo.score(p), f"noalloc {case}")
        log(f"[gpu] noalloc errs {errs}")
    assert all(b < a for a, b in zip(sizes, sizes[1:])), sizes


def test_noalloc_rejects_a_workspace_beyond_the_array():
    """About 400 MB of partials for 200,000 rows of a 248,320-entry head: JET_E_WORKSPACE,
    decided on the host from the scalars (the pointers are never read)."""
    lib = _lib.load()
    h = np.zeros(64, np.float32)
    p = _lib.JetProblem()
    p.H, p.h_dtype, p.n_rows = h.ctypes.data, _lib.JET_BF16, 200000
    p.W, p.w_dtype, p.V, p.d = h.ctypes.data, _lib.JET_BF16, 248320, 2560
    p.T = 1.0
    assert lib.jet_score_workspace_size(ctypes.byref(p)) > _lib.NOALLOC_MAX_WORKSPACE
    o = _lib.JetOutputs()
    assert lib.jet_score_noalloc(ctypes.byref(p), ctypes.byref(o), None) == -6
