"""HIP path vs the fp64 oracle on the same seeded inputs (needs an MI355X).

Small and ragged problems are compared element by element on every output.  The five
workloads run at their full sizes in the configuration the benchmark times; the large ones
are compared on sampled rows the oracle computes one by one, plus properties that hold at
any size (flags clear, q sums to one, duplicates bitwise equal, run-to-run determinism).
"""
import numpy as np
import pytest

import oracle as jo
import workloads as wl
from tests.parity import Q_TOL, check_decisions, compare, log, tol_logp

torch = pytest.importorskip("torch")
from candidate_likelihood_scoring_amd import api  # noqa: E402
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jet():
    from candidate_likelihood_scoring_amd import problem

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return problem


def _run(jet, p, **kw):
    out = jet.to_numpy(jet.score_problem(jet.to_device(p, "cuda"), **kw))
    torch.cuda.synchronize()
    return out


# ----------------------------------------------------------------------------------------
# small problems: full element-by-element parity
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "tiny_tie"])
def test_tiny(jet, name):
    p = wl.make_config(name)
    log(f"[gpu] {name}")
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] {name} errs {compare(p, out, ref, name)}")
    if name == "tiny_tie":
        co = p["cand_tok_off"]
        assert out["cand_s"][2] == out["cand_s"][3]  # identical inputs: bitwise equal
        assert out["cand_q"][2] == out["cand_q"][3]
        assert np.array_equal(out["tok_logp"][co[2]:co[3]], out["tok_logp"][co[3]:co[4]])
        # the duplicated pair is the best: an exact tie on both sides, the lowest index wins
        assert ref["q_argmax"][0] == 2 and ref["q_gap"][0] == 0.0
        assert out["q_argmax"][0] == 2


RAGGED = [
    dict(V=4099, d=64, n_q=7, K=(1, 9), lengths=(1, 5), layout="prefix", seed=11),
    dict(V=10007, d=256, n_q=12, K=(2, 20), lengths=(1, 4), layout="own", seed=12),
    dict(V=6151, d=96, n_q=40, K=(1, 26), layout="field", seed=13, T=2.0),
    dict(V=5003, d=128, n_q=9, K=(1, 12), lengths=(1, 6), layout="prefix", seed=14, h_dtype="bf16",
         dups=2),
    dict(V=3001, d=64, n_q=6, K=(1, 8), lengths=(1, 7), layout="own", seed=15, w_dtype="f32"),
    dict(V=2053, d=32, n_q=30, K=(1, 70), lengths=(1, 3), layout="prefix", seed=16, T=0.7),
    dict(V=33, d=32, n_q=3, K=(1, 5), lengths=(1, 3), layout="prefix", seed=17),
    dict(V=1, d=32, n_q=2, K=(1, 3), lengths=(1, 2), layout="own", seed=18),
    dict(V=64, d=32, n_q=1, K=1, lengths=1, layout="field", seed=19),
    dict(V=4096, d=256, n_q=8, K=(2, 5), lengths=(1, 3), layout="own", seed=20, w_dtype="f32",
         n_extra_rows=0, w_std=0.5),
    # streaming kernel, 1,843 single-token candidates scored from 100 field rows
    dict(V=5003, d=128, n_q=100, K=(10, 26), layout="field", seed=21),
    # streaming kernel, 200 rows in 7 row tiles
    dict(V=65536, d=128, n_q=100, K=(2, 6), lengths=1, layout="prefix", seed=22,
         n_extra_rows=100),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"ragged{i}" for i in range(len(RAGGED))])
def test_ragged(jet, case):
    p = wl.make_problem(**case)
    log(f"[gpu] ragged {case} rows={p['n_rows']} tok={len(p['tok_target'])}")
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] errs {compare(p, out, ref, str(case))}")


MANY_CANDIDATES = [
    # one question of 20,000 single-token candidates, with exact duplicates
    dict(V=30011, d=64, n_q=1, K=20000, layout="field", seed=31, T=1.3, dups=3),
    # questions of 1 to 200 candidates side by side (64 and fewer on their own wave, the
    # others on the whole workgroup)
    dict(V=30011, d=64, n_q=30, K=(1, 200), layout="field", seed=32),
    # multi-token candidates, 40 to 400 per question, bf16 H
    dict(V=2053, d=32, n_q=6, K=(40, 400), lengths=(1, 3), layout="prefix", seed=33,
         h_dtype="bf16", dups=2),
    # 40 to 130 candidates (on either side of one wave's 64), fp32 head
    dict(V=1000, d=32, n_q=20, K=(40, 130), lengths=(1, 2), layout="own", seed=34, w_dtype="f32"),
]


@pytest.mark.parametrize("case", MANY_CANDIDATES, ids=["one_20000", "mixed_200", "multi_token_400",
                                                       "around_64"])
def test_many_candidates(jet, case):
    """Questions with more than 64 candidates are decided by a whole workgroup (on problems
    where one could have more than 1,024): every output against the oracle, the tie rule on
    exact duplicates, and the same bits on a second call."""
    p = wl.make_problem(**case)
    Ks = np.diff(p["q_cand_off"])
    assert int(p["q_cand_off"][-1]) - (len(Ks) - 1) > 1024 and Ks.max() > 64  # the case's premise
    # a true index per question, last candidate or one past 64 (q_true of the thread that
    # holds it)
    p["q_true_idx"] = np.where(Ks > 70, 70, Ks - 1).astype(np.int32)
    log(f"[gpu] many candidates {case}: K per question {Ks.tolist()[:12]}")
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] errs {compare(p, out, ref, str(case))}")
    again = _run(jet, p)
    for k in out:
        assert np.array_equal(out[k], again[k], equal_nan=True), k


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [384, 640, 192, 960, 64])
def test_stream_odd_stage_count(jet, d, h_dtype):
    """The streaming kernel with an odd number of 128-wide stages (3 and 5; with d % 128 =
    64 the last one 64 wide: 2 stages at d = 192, 8 at 960, 1 at 64): with one row tile its
    H stage buffers alternate by pairs of stages (2, 3, 1, 4 and 1 pairs here), so with an
    odd pair count the last stage of one vocabulary group and the first of the next share a
    buffer.  513 groups over 256 workgroups give every workgroup two or three groups in a
    row; every output against the oracle (30 field rows: one row tile)."""
    p = wl.make_problem(V=131101, d=d, n_q=30, K=(2, 6), layout="field", seed=95,
                        h_dtype=h_dtype)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] stream odd stages d={d} {h_dtype} rows={p['n_rows']} ({kern})")
    assert kern == "k_project_wg_bf16" and p["n_rows"] <= 32
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] errs {compare(p, out, ref, f'odd_stages_{d}_{h_dtype}')}")


# (d, H dtype, rows): the streaming kernel carrying 2 (fp32 H) or 4 (bf16 H) 32-row tiles
# per workgroup, with full and ragged last tiles and odd stage counts (d = 384, 640; a
# 64-wide last stage at d = 320, 960)
_STREAM_MULTI = [(256, "f32", 64), (384, "f32", 41), (256, "bf16", 128), (640, "bf16", 97),
                 (128, "bf16", 70), (384, "bf16", 33), (320, "f32", 50), (960, "bf16", 111)]


@pytest.mark.parametrize("d,h_dtype,rows", _STREAM_MULTI,
                         ids=[f"d{d}_{h}_{r}" for d, h, r in _STREAM_MULTI])
def test_stream_row_tiles_per_workgroup(jet, d, h_dtype, rows):
    """The streaming kernel with several 32-row tiles of H per workgroup: each head fragment
    is multiplied into every row tile's accumulators, so the head is read once for up to 64
    (fp32 H) or 128 (bf16 H) rows.  One question per row (single-token fields), so every
    row carries tokens; every output against the oracle."""
    p = wl.make_problem(V=131101, d=d, n_q=rows, K=(2, 8), layout="field", seed=300 + rows,
                        h_dtype=h_dtype)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] stream row tiles d={d} {h_dtype} rows={p['n_rows']} ({kern})")
    assert kern == "k_project_wg_bf16" and p["n_rows"] == rows
    out = _run(jet, p)
    log(f"[gpu] errs {compare(p, out, jo.score(p), f'stream_multi_{d}_{h_dtype}_{rows}')}")


# fp32 head (V, d, rows), each with at least 256 (vocabulary group, row tile) pairs so that
# the streaming kernel takes it: last stage 32 wide (d % 64 = 32) or whole; 1 to 16 stages
# (odd and even counts, each remainder of the 3-slot pipeline; odd counts also with several
# groups per workgroup, V > 65,536); the 16-row tile (1 to 16 rows) and 32-row tiles, the
# last ragged; vocabularies of one entry, below one 256-entry group and with a one-entry
# last group; a head past the last-level cache (non-temporal loads)
_F32_STREAM = [(1, 32, 8200), (255, 96, 8192), (70001, 96, 1), (131101, 320, 16),
               (65537, 64, 17), (30011, 160, 70), (100003, 1024, 5), (128000, 1024, 4),
               (3001, 64, 2100), (257, 256, 4100), (140000, 192, 40), (90001, 64, 9)]


@pytest.mark.parametrize("V,d,rows", _F32_STREAM, ids=[f"V{v}_d{d}_{r}" for v, d, r in _F32_STREAM])
def test_f32_head_stream(jet, V, d, rows):
    """fp32 head and fp32 H: the streaming kernel (one row tile per workgroup, 16 rows with
    v_mfma_f32_16x16x4f32 up to 16 rows, else 32 with v_mfma_f32_32x32x2f32; 64 k per stage
    through LDS), one question per row (single-token fields); every output against the
    oracle at the fp32 tolerance, on every row."""
    p = wl.make_problem(V=V, d=d, n_q=rows, K=1 if V == 1 else (1, 6), layout="field",
                        seed=500 + d + rows, w_dtype="f32")
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] f32 head V={V} d={d} rows={p['n_rows']} ({kern})")
    assert kern == "k_project_wg_f32" and p["n_rows"] == rows
    out = _run(jet, p)
    log(f"[gpu] errs {compare(p, out, jo.score(p), f'f32_stream_{V}_{d}_{rows}')}")


@pytest.mark.parametrize("h_dtype,rows", [("f32", 150), ("bf16", 300)])
def test_stream_small_vocab_many_rows(jet, h_dtype, rows):
    """A vocabulary below one tiled tile (V = 200) keeps many rows on the streaming kernel:
    several passes of 2 (fp32 H) or 4 (bf16 H) row tiles, the last one ragged; every
    output against the oracle."""
    p = wl.make_problem(V=200, d=256, n_q=rows, K=(2, 8), layout="field", seed=400 + rows,
                        h_dtype=h_dtype)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] stream small vocab {h_dtype} rows={p['n_rows']} ({kern})")
    assert kern == "k_project_wg_bf16" and p["n_rows"] == rows
    out = _run(jet, p)
    log(f"[gpu] errs {compare(p, out, jo.score(p), f'stream_small_vocab_{h_dtype}')}")


@pytest.mark.parametrize("h_dtype,rows", [("f32", 64), ("bf16", 128)])
def test_stream_row_tiles_large_head(jet, h_dtype, rows):
    """The most rows one pass of the streaming kernel takes (64 of fp32 H, 128 of bf16 H) on
    binary_enum's head shape (V = 248,320, d = 2560, non-temporal head loads): every output of
    16 sampled questions (one row each) against the oracle, properties on all."""
    p = wl.make_problem(V=248320, d=2560, n_q=rows, K=(2, 8), layout="field", seed=77,
                        h_dtype=h_dtype)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] stream row tiles, large head, {h_dtype} rows={p['n_rows']} ({kern})")
    assert kern == "k_project_wg_bf16" and p["n_rows"] == rows
    out = _run(jet, p)
    _full_size_properties(p, out)
    qs = np.random.default_rng(6).choice(rows, 16, replace=False)
    ref = jo.score(p, rows=_rows_of_questions(p, qs))
    log(f"[gpu] errs {compare(p, out, ref, 'stream_multi_large_' + h_dtype, sampled=True)}")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
def test_stream_target_logit_dominates(jet, h_dtype):
    """Streaming path, where each target logit is a dot product of its own, summed in
    another order than the projection's: every row gets one planted vocabulary entry
    (head row bf16(40 h / |h|^2), logit near +40, every other logit about N(0, 1)) and all
    its tokens target it, so l_k is about -1e-14 and a rounding apart from 0.  l_k must stay
    <= 0 and match the oracle, and no output may depend on whether row_lse is requested
    (without it the launch has no row waves)."""
    p = wl.make_problem(V=8192, d=256, n_q=5, K=(2, 5), lengths=(1, 2), layout="prefix",
                        seed=71, h_dtype=h_dtype)
    H = np.asarray(p["H"])
    H64 = ((H.astype(np.uint32) << 16).view(np.float32) if h_dtype == "bf16" else H).astype(np.float64)
    rng = np.random.default_rng(72)
    planted = rng.choice(p["V"], size=p["n_rows"], replace=False).astype(np.int32)
    W = np.array(p["W"], copy=True)
    for r in range(p["n_rows"]):
        W[planted[r]] = wl.bf16_bits((40.0 * H64[r] / np.dot(H64[r], H64[r])).astype(np.float32))
    rows = np.arange(len(p["tok_target"])) if p["tok_row"] is None else np.asarray(p["tok_row"])
    p = dict(p, W=W, tok_target=planted[rows])
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] stream dominant targets {h_dtype} rows={p['n_rows']} tokens={len(rows)} ({kern})")
    assert kern == "k_project_wg_bf16"
    out = _run(jet, p)
    ref = jo.score(p)
    assert np.max(ref["tok_logp"]) > -1e-6
    log(f"[gpu] errs {compare(p, out, ref, f'dominant_{h_dtype}')}")
    assert np.all(out["tok_logp"] <= 0)
    lean = _run(jet, p, optional=False)
    for k in lean:
        assert np.array_equal(lean[k], out[k]), k


@pytest.mark.parametrize("h_dtype", ["f32", "bf16"])
def test_mid_rows_large_head(jet, h_dtype):
    """Between one streaming row tile and one whole tiled row tile, on binary_enum's head
    shape (V = 248,320, d = 2560): 207 rows run on the tiled kernel, with fp32 H as two
    128-row tiles (XCD-aware blocks padded with empty row tiles) and with bf16 H as one
    256-row tile of zero-padded H.  fp32 H against the full oracle, bf16 H on every row of
    10 sampled questions."""
    p = wl.make_problem(V=248320, d=2560, n_q=40, K=(2, 6), lengths=(1, 3), layout="prefix",
                        seed=99, h_dtype=h_dtype, n_extra_rows=0)
    n = p["n_rows"]
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] mid rows, large head, {n} rows {h_dtype} ({kern})")
    assert 128 < n < 256
    assert kern == ("k_project_tiled_m16x2" if h_dtype == "f32" else "k_project_tiled_m16")
    out = _run(jet, p)
    _full_size_properties(p, out)
    qs = np.random.default_rng(5).choice(len(p["q_cand_off"]) - 1, 10, replace=False)
    rows = None if h_dtype == "f32" else _rows_of_questions(p, qs)
    ref = jo.score(p, rows=rows)
    log(f"[gpu] mid rows errs {compare(p, out, ref, 'mid_rows_' + h_dtype, sampled=rows is not None)}")


# (V, extra rows, rows before -> after): the streaming kernel (a vocabulary below one tiled
# tile) going from two 32-row tiles to three; the tiled kernel from one zero-padded row tile
# to one exact one (bf16 H: 256 rows) and from one to two (fp32 H: 128-row tiles)
_ROW_TILE_STEPS = {
    "stream_f32": (250, "f32", 4, 64), "stream_bf16": (250, "bf16", 4, 64),
    "tiled_bf16": (20011, "bf16", 196, 256), "tiled_f32": (20011, "f32", 68, 128),
}


@pytest.mark.parametrize("case", list(_ROW_TILE_STEPS))
def test_extra_row_tile_keeps_every_bit(jet, case):
    """The same questions in a problem with one more, unreferenced row: a kernel's
    partials, the merge and the decisions do not depend on how many rows or row tiles the
    problem has (nor on zero padding rows), so every output keeps its bits; both against
    the oracle."""
    V, h_dtype, extra, n0 = _ROW_TILE_STEPS[case]
    p = wl.make_problem(V=V, d=256, n_q=12, K=(2, 5), lengths=(1, 3), layout="prefix",
                        seed=98, h_dtype=h_dtype, n_extra_rows=extra)
    q = wl.make_problem(V=V, d=256, n_q=12, K=(2, 5), lengths=(1, 3), layout="prefix",
                        seed=98, h_dtype=h_dtype, n_extra_rows=extra + 1)
    assert p["n_rows"] == n0 and q["n_rows"] == n0 + 1
    assert np.array_equal(p["H"], q["H"][:n0]) and np.array_equal(p["tok_target"], q["tok_target"])
    kp = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    kq = api.projection_kernel(api.make_problem(**jet.to_device(q, "cuda")))
    log(f"[gpu] extra row {case}: {n0} rows ({kp}) -> {n0 + 1} ({kq})")
    assert kp == kq and (kp == "k_project_wg_bf16") == case.startswith("stream")
    a, b = _run(jet, p), _run(jet, q)
    log(f"[gpu] extra row {case}: errs {compare(p, a, jo.score(p), 'row_tiles_' + case)}")
    for k in a:
        x, y = (a[k], b[k][:n0]) if k == "row_lse" else (a[k], b[k])
        assert np.array_equal(x.view(np.int32), y.view(np.int32)), k


# Large-row (matrix-core) path: at least 256 rows and 256 entries, d a multiple of two
# K stages (128 for bf16 hidden states, 64 for fp32).  Ragged row and vocabulary tails
# exercise the shifted last tiles; the medium case gives every workgroup several
# vocabulary tiles, so the stage stream runs across tile boundaries.
TILED = [
    dict(V=3001, d=128, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=61, h_dtype="bf16",
         n_extra_rows=300),
    dict(V=1283, d=256, n_q=25, K=(1, 12), lengths=(1, 5), layout="prefix", seed=62,
         h_dtype="bf16", n_extra_rows=211),
    dict(V=256, d=128, n_q=10, K=(2, 4), lengths=(1, 3), layout="own", seed=65, h_dtype="bf16",
         n_extra_rows=256),
    dict(V=2500, d=64, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=63, n_extra_rows=250),
    dict(V=4099, d=192, n_q=20, K=(1, 10), lengths=(1, 4), layout="field", seed=64,
         n_extra_rows=400, T=1.7),
    # fp32 H: the 16 x 16 kernel's two-plane form, 128-row tiles
    dict(V=3001, d=128, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=68, n_extra_rows=300),
    dict(V=1283, d=256, n_q=25, K=(1, 12), lengths=(1, 5), layout="prefix", seed=69,
         n_extra_rows=211),
    dict(V=256, d=128, n_q=10, K=(2, 4), lengths=(1, 3), layout="own", seed=70, n_extra_rows=256),
    # an odd number of 64-wide stages (the extra stage after the stage-pair loop), with two
    # vocabulary tiles per workgroup so the odd stage is followed by the next tile's stages
    dict(V=30011, d=192, n_q=40, K=(2, 8), lengths=(1, 6), layout="own", seed=71, h_dtype="bf16",
         n_extra_rows=300),
    dict(V=20011, d=320, n_q=30, K=(2, 8), lengths=(1, 6), layout="prefix", seed=72,
         n_extra_rows=200, T=0.8),
    dict(V=5003, d=64, n_q=20, K=(2, 8), lengths=(1, 5), layout="field", seed=73, h_dtype="bf16",
         n_extra_rows=256),
]


@pytest.mark.parametrize("case", TILED, ids=[f"tiled{i}" for i in range(len(TILED))])
def test_tiled(jet, case):
    p = wl.make_problem(**case)
    log(f"[gpu] tiled {case} rows={p['n_rows']} tok={len(p['tok_target'])}")
    assert p["n_rows"] >= 256 and p["V"] >= 256
    from candidate_likelihood_scoring_amd import api
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    assert kern.startswith("k_project_tiled"), kern
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] errs {compare(p, out, ref, str(case))}")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
def test_tiled_stream(jet, h_dtype):
    p = wl.make_problem(V=131101, d=128, n_q=40, K=(2, 6), lengths=(1, 4), layout="prefix",
                        seed=66, h_dtype=h_dtype, n_extra_rows=3000)
    log(f"[gpu] tiled stream {h_dtype} rows={p['n_rows']} V={p['V']}")
    from candidate_likelihood_scoring_amd import api
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    assert kern.startswith("k_project_tiled"), kern
    out = _run(jet, p)
    _full_size_properties(p, out)
    # oracle on every referenced row plus the rows at each 256-row tile boundary and the tail
    n = p["n_rows"]
    edges = [r for b in range(0, n, 128) for r in (b, b + 1, b + 127) if r < n]
    rows = np.unique(np.concatenate([np.asarray(p["tok_row"]), edges, np.arange(n - 3, n)]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] errs {compare(p, out, ref, 'tiled_stream', sampled=True)} on {len(rows)} rows")


@pytest.mark.parametrize("operand", ["head", "hidden"])
def test_tiled_operands_past_4gib(jet, operand):
    """Operands larger than 4 GiB stay on the matrix-core kernel, whose buffer offsets are
    local to each workgroup's tiles: a 4.9 GB head (V = 300,007, d = 8192: 37,863 head rows
    lie past 4 GiB, and targets are planted there) or 4.4 GB of hidden states (270,000
    rows of d = 8192; rows past 4 GiB sampled).  Sampled rows against the oracle."""
    if operand == "head":
        p = wl.make_problem(V=300007, d=8192, n_q=12, K=(2, 5), lengths=(1, 3), layout="own",
                            seed=96, h_dtype="bf16", n_extra_rows=230)
        edge = (1 << 32) // (8192 * 2)  # first head row past 4 GiB
        tg = p["tok_target"].copy()
        tg[:6] = [edge, edge + 1, p["V"] - 1, p["V"] - 2, p["V"] - 300, edge - 1]
        p["tok_target"] = tg
    else:
        p = wl.make_problem(V=4099, d=8192, n_q=12, K=(2, 5), lengths=(1, 3), layout="prefix",
                            seed=97, h_dtype="bf16", n_extra_rows=270000)
    n = p["n_rows"]
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] past 4 GiB ({operand}): V={p['V']} rows={n} head={p['V'] * p['d'] * 2} "
        f"H={n * p['d'] * 2} bytes ({kern})")
    assert kern == "k_project_tiled_m16"
    assert max(p["V"], n) * p["d"] * 2 > (1 << 32)
    out = _run(jet, p)
    _full_size_properties(p, out)
    tok_row = np.arange(len(p["tok_target"])) if p["tok_row"] is None else np.asarray(p["tok_row"])
    edge_r = (1 << 32) // (p["d"] * 2)
    rows = np.unique(np.concatenate([tok_row, np.arange(0, 8), np.arange(n - 300, n),
                                     [r for r in (edge_r - 1, edge_r, edge_r + 1) if r < n]]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] past 4 GiB ({operand}) errs {compare(p, out, ref, f'past4g_{operand}', sampled=True)}"
        f" on {len(rows)} rows")


def test_tiled_padded_row_groups(jet):
    """bf16 H in 31 row tiles of 256 over 513 vocabulary tiles (136 splits): the launch
    places 8 row tiles x 4 splits per XCD and pads the last row group with one empty row
    tile, whose workgroups exit at once.  Every row of the last two row groups and the
    tile boundaries are checked."""
    p = wl.make_problem(V=131101, d=128, n_q=40, K=(2, 6), lengths=(1, 4), layout="prefix",
                        seed=71, h_dtype="bf16", n_extra_rows=7611)
    n = p["n_rows"]
    log(f"[gpu] padded row groups rows={n} V={p['V']}")
    assert 30 * 256 < n <= 31 * 256
    out = _run(jet, p)
    _full_size_properties(p, out)
    edges = [r for b in range(0, n, 256) for r in (b, b + 255) if r < n]
    rows = np.unique(np.concatenate([np.asarray(p["tok_row"]), edges, np.arange(16 * 256, n)]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] errs {compare(p, out, ref, 'padded_row_groups', sampled=True)} on {len(rows)} rows")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("R", [8, 9, 15, 16, 17, 24, 31, 33, 40])
def test_tiled_placement_sweep(jet, h_dtype, R):
    """Row-tile counts on both sides of the XCD block-shape rule (8 x 4 blocks for bf16 H
    when padding to a multiple of 8 costs at most R/16 row tiles, else 4 x 8, padded), over
    129 vocabulary tiles (40 splits): the sampled rows cover every tile boundary and the
    last two row tiles."""
    tile = 256 if h_dtype == "bf16" else 128
    p = wl.make_problem(V=33001, d=128, n_q=40, K=(2, 6), lengths=(1, 4), layout="prefix",
                        seed=71, h_dtype=h_dtype, n_extra_rows=R * tile - 7 - 289)
    n = p["n_rows"]
    log(f"[gpu] placement sweep {h_dtype} R={R} rows={n}")
    assert -(-n // tile) == R
    out = _run(jet, p)
    _full_size_properties(p, out)
    edges = [r for b in range(0, n, tile) for r in (b, b + tile - 1) if r < n]
    rows = np.unique(np.concatenate([np.asarray(p["tok_row"]), edges, np.arange(n - 2 * tile, n)]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] errs {compare(p, out, ref, f'placement_{h_dtype}_{R}', sampled=True)}")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
def test_tiled_bad_indices_many_tiles(jet, h_dtype):
    """The tiled kernel over many (row tile, vocabulary tile) pairs (about 36 x 1,025) with
    its tokens spread over the row tiles; an out-of-range target and an out-of-range row
    raise their flags and leave only their own tokens NaN, every other output bit and the
    row LSEs unchanged."""
    p = wl.make_problem(V=262147, d=128, n_q=40, K=(2, 6), lengths=(1, 4), layout="prefix",
                        seed=67, h_dtype=h_dtype, n_extra_rows=9000)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] tiled bad indices {h_dtype} rows={p['n_rows']} V={p['V']} ({kern})")
    assert kern in ("k_project_tiled_m16", "k_project_tiled_m16x2")
    out = _run(jet, p)
    _full_size_properties(p, out)
    rows = np.unique(np.asarray(p["tok_row"]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] errs {compare(p, out, ref, 'tiled_bad_indices', sampled=True)} on {len(rows)} rows")
    q = dict(p)
    q["tok_target"] = p["tok_target"].copy()
    q["tok_row"] = p["tok_row"].copy()
    q["tok_target"][3] = p["V"] + 5
    q["tok_row"][7] = p["n_rows"] + 9
    bad = _run(jet, q)
    assert int(bad["dev_flags"][0]) & 1 and int(bad["dev_flags"][0]) & 2
    assert np.isnan(bad["tok_logp"][3]) and np.isnan(bad["tok_logp"][7])
    good = np.ones(len(p["tok_target"]), bool)
    good[[3, 7]] = False
    assert np.array_equal(bad["tok_logp"][good], out["tok_logp"][good])
    assert np.array_equal(bad["row_lse"], out["row_lse"])


@pytest.mark.parametrize("h_dtype", ["f32", "bf16"])
def test_deduplicated_rows(jet, h_dtype):
    """Predictor-row deduplication (history trie built by the library on the host): scoring
    one row per predictor node gives the full problem's outputs (FastJEV Sec. 3.3)."""
    from candidate_likelihood_scoring_amd import api

    p = wl.shared_history_problem(V=5003, d=128, n_q=40, K=(4, 12), lengths=(1, 6), alphabet=3,
                                  h_dtype=h_dtype, seed=71)
    tok_node, node_tok = api.build_predictor_trie(p["tok_target"], p["cand_tok_off"], p["q_cand_off"])
    pd = dict(p, H=p["H"][node_tok], n_rows=len(node_tok), tok_row=tok_node)
    log(f"[gpu] dedup {h_dtype}: {p['n_rows']} rows -> {pd['n_rows']} predictor nodes")
    assert pd["n_rows"] < p["n_rows"]
    ref = jo.score(p)
    out_full = _run(jet, p)
    out_dd = _run(jet, pd)
    log(f"[gpu] full errs {compare(p, out_full, ref, 'dedup full')}")
    ref_dd = dict(ref, lse=ref["lse"][node_tok])
    log(f"[gpu] dedup errs {compare(pd, out_dd, ref_dd, 'dedup nodes')}")


@pytest.mark.parametrize("case", [dict(), dict(n_inputs=300, K=(1, 130), n_layers=61, seed=708),
                                  dict(n_inputs=1, K=(1, 1), n_layers=3, seed=709, tie=None)],
                         ids=["calib32", "ragged", "single"])
def test_decision_sensitivity(jet, case):
    """Layer-skip sensitivity (FastJEV Sec. 3.4, Eq. 5-6) against the oracle.  Tolerance per
    d: fp32 centring loses u * (|mean| / rms of the centred values) for both vectors, with
    u = 2^-24, plus the sums' own rounding; J within the mean of those; the selection must
    match wherever the oracle's J separates the k-th and (k+1)-th layers by more than that."""
    from candidate_likelihood_scoring_amd import api

    c = wl.calibration_logits(**case)
    L, n_in = c["n_layers"], c["n_inputs"]
    z64, zs64, off = c["z"].astype(np.float64), c["z_skip"].astype(np.float64), c["seg_off"]
    d_ref, J_ref = jo.decision_sensitivity(c["z"], c["z_skip"], off)
    dev = "cuda"
    for k in sorted({0, 1, min(6, L), L}):
        out = api.decision_sensitivity(torch.from_numpy(c["z"]).to(dev),
                                       torch.from_numpy(c["z_skip"]).to(dev),
                                       torch.from_numpy(off).to(dev), k)
        torch.cuda.synchronize()
        assert int(out["dev_flags"][0]) == 0
        d = out["d"].cpu().numpy().astype(np.float64)
        J = out["J"].cpu().numpy().astype(np.float64)
        sel = out["selected"].cpu().numpy()
        u = 2.0 ** -24
        tol = np.empty((L, n_in))
        for x in range(n_in):
            a, b = int(off[x]), int(off[x + 1])
            zx = z64[a:b]
            rz = max(1e-8, float(np.sqrt(np.mean((zx - zx.mean()) ** 2))))
            for l in range(L):
                dl = zs64[l, a:b] - zx
                rd = float(np.sqrt(np.mean((dl - dl.mean()) ** 2)))
                cm = abs(dl.mean()) / max(rd, 1e-30) + abs(zx.mean()) / rz
                tol[l, x] = 8 * u * (4 + (b - a) ** 0.5 + cm) * d_ref[l, x] + 1e-30
        err = np.abs(d - d_ref)
        assert np.all(err <= tol), ("d", float((err / tol).max()))
        tol_J = tol.mean(axis=1) + 4 * u * J_ref
        assert np.all(np.abs(J - J_ref) <= tol_J), ("J", float(np.abs(J - J_ref).max()))
        if c.get("n_layers") and case.get("tie", (4, 9)) is not None and L > 9:
            assert J[4] == J[9] and np.array_equal(d[4], d[9])  # exact copies tie exactly
        ref_sel = jo.select_layers(J_ref, k)
        order = sorted(range(L), key=lambda l: (J_ref[l], l))
        if k == 0 or k == L or J_ref[order[k]] - J_ref[order[k - 1]] > tol_J[order[k]] + tol_J[order[k - 1]]:
            assert set(sel) == set(ref_sel), (k, sel, ref_sel)
        # whatever the band, the selection is sorted by (J, index) in the kernel's own values
        assert list(sel) == sorted(sel, key=lambda l: (J[l], l))
        assert len(set(sel)) == k and all(J[s] <= J[o] for s in sel for o in set(range(L)) - set(sel))
        log(f"[gpu] sensitivity {case} k={k}: max d err/tol {float((err / tol).max()):.3f}")


def test_decision_sensitivity_bad_offsets_flag(jet):
    """A segment outside [0, n_values) raises the offsets flag; its d is NaN and ranks last."""
    from candidate_likelihood_scoring_amd import api

    c = wl.calibration_logits(n_inputs=4, K=(3, 6), n_layers=5, seed=710, tie=None)
    off = c["seg_off"].copy()
    off[3] = off[4] + 7  # input 2 runs past the end, input 3 is inverted
    out = api.decision_sensitivity(torch.from_numpy(c["z"]).cuda(), torch.from_numpy(c["z_skip"]).cuda(),
                                   torch.from_numpy(off).cuda(), 5)
    torch.cuda.synchronize()
    assert int(out["dev_flags"][0]) & 4
    d = out["d"].cpu().numpy()
    assert np.all(np.isnan(d[:, 2])) and np.all(np.isnan(d[:, 3])) and np.all(np.isfinite(d[:, :2]))
    assert sorted(out["selected"].cpu().numpy().tolist()) == [0, 1, 2, 3, 4]


def _fit_tolerance(s, qo, text, gold, T):
    """fp32 error bound of the mean gold NLL at T: each question's two log-sum-exps over K
    terms carry at most (2K + 8) u of their magnitude (u = 2^-24); 4x that, averaged."""
    u = 2.0 ** -24
    tot, n = 0.0, 0
    for g in range(len(qo) - 1):
        a = np.asarray(s[qo[g]:qo[g + 1]], np.float64) / T
        m = np.asarray(text[qo[g]:qo[g + 1]]) == gold[g]
        if gold[g] < 0 or not m.any():
            continue
        l1 = a.max() + np.log(np.exp(a - a.max()).sum())
        l2 = a[m].max() + np.log(np.exp(a[m] - a[m].max()).sum())
        tot += (2 * len(a) + 8) * u * (abs(l1) + abs(l2))
        n += 1
    return 4 * tot / max(n, 1)


def _check_fit(s, qo, text, gold, out, T_min=1e-2, T_max=1e2, what="", ds=0.0):
    """ds: bound on |GPU scores - oracle scores| when the fit ran on the GPU's own scores;
    each log-sum-exp is 1-Lipschitz in its arguments, so the NLL moves by <= 2 ds / T."""
    T_ref, f_ref = jo.fit_temperature(s, qo, text, gold, T_min, T_max)
    T = float(out["T"][0])
    nll = float(out["nll"][0])
    assert int(out["dev_flags"][0]) == 0
    f_at = jo.mean_gold_nll(s, qo, text, gold, T)[0]
    tol = _fit_tolerance(s, qo, text, gold, T_ref)
    shift = 2.0 * ds / min(T, T_ref)
    assert f_at - f_ref <= 2 * tol + 2 * shift, (what, T, T_ref, f_at - f_ref, tol, shift)
    assert abs(nll - f_at) <= tol + shift, (what, nll, f_at, tol, shift)
    log(f"[gpu] fit {what}: T {T:.6f} (oracle {T_ref:.6f}), excess NLL {f_at - f_ref:.2e} "
        f"(tol {2 * tol:.1e})")


@pytest.mark.parametrize("case", ["planted", "closed_form", "partly_unlabelled", "wide", "many"])
def test_fit_temperature(jet, case):
    """Temperature fitting against the oracle's minimiser, compared by the NLL it attains."""
    from candidate_likelihood_scoring_amd import api

    if case == "planted":
        c = wl.labelled_questions(n_q=4096)
        s, qo, text, gold = c["cand_s"], c["q_cand_off"], c["cand_text_id"], c["q_gold_text_id"]
    elif case == "closed_form":
        s = np.array([0.0, -2.0, 0.0, 1.0], np.float32)
        qo, text, gold = (np.array([0, 2, 4], np.int32), np.array([0, 1, 0, 1], np.int32),
                          np.array([0, 0], np.int32))
    elif case == "many":
        # more questions than the 4096 waves of a full launch: waves take one or two each
        c = wl.labelled_questions(n_q=5001, K=(2, 8), seed=811)
        s, qo, text, gold = c["cand_s"], c["q_cand_off"], c["cand_text_id"], c["q_gold_text_id"]
    elif case == "wide":
        # 60-150 candidates per question: scores arrive in chunks of 64 (one per lane)
        c = wl.labelled_questions(n_q=200, K=(60, 150), seed=810)
        s, qo, text, gold = c["cand_s"], c["q_cand_off"], c["cand_text_id"], c["q_gold_text_id"]
    else:
        c = wl.labelled_questions(n_q=300, K=(1, 9), seed=809)
        s, qo, text = c["cand_s"], c["q_cand_off"], c["cand_text_id"]
        gold = c["q_gold_text_id"].copy()
        gold[::7] = -1          # unlabelled
        gold[3::11] = 999       # no candidate of that text
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    for T_min, T_max in ((1e-2, 1e2), (0.5, 4.0)):
        out = api.fit_temperature(t(s), t(qo), t(text), t(gold), T_min, T_max)
        torch.cuda.synchronize()
        _check_fit(s, qo, text, gold, out, T_min, T_max, f"{case} [{T_min}, {T_max}]")


def test_fit_temperature_after_scoring(jet):
    """The calibration chain: jet_score's candidate scores (on the device) feed the fit."""
    from candidate_likelihood_scoring_amd import api

    p = wl.make_problem(V=3001, d=64, n_q=60, K=(2, 7), lengths=(1, 3), layout="prefix", seed=81)
    pdv = jet.to_device(p, "cuda")
    out = jet.score_problem(pdv)
    torch.cuda.synchronize()
    ref = jo.score(p)
    fit = api.fit_temperature(out["cand_s"], pdv["q_cand_off"], pdv["cand_text_id"],
                              pdv["q_gold_text_id"])
    torch.cuda.synchronize()
    ds = float(np.max(np.abs(out["cand_s"].cpu().numpy().astype(np.float64) - ref["cand_s"])))
    _check_fit(ref["cand_s"], p["q_cand_off"], p["cand_text_id"], p["q_gold_text_id"], fit,
               what="after scoring", ds=ds)


def test_true_index_and_gold(jet):
    p = wl.make_problem(V=3000, d=64, n_q=10, K=(2, 6), lengths=(1, 3), layout="prefix", seed=31, dups=1)
    K = np.diff(p["q_cand_off"])
    rng = np.random.default_rng(0)
    p["q_true_idx"] = np.array([rng.integers(-1, k) for k in K], dtype=np.int32)
    p["q_gold_text_id"][0] = 999  # gold text absent -> +inf
    out = _run(jet, p)
    ref = jo.score(p)
    compare(p, out, ref, "true_idx")
    assert np.isinf(out["q_gold_nll"][0])


def test_side_stream_matches_current_stream(jet):
    """Scoring on a stream other than the current one (outputs and workspace allocated, and
    the flag word zeroed, on the current stream) gives the same bits as on the current one."""
    from candidate_likelihood_scoring_amd import api
    p = wl.make_problem(V=6151, d=128, n_q=12, K=(2, 6), lengths=(1, 4), layout="prefix", seed=71)
    dp = jet.to_device(p, "cuda")
    ref = api.score(**dp)
    side = torch.cuda.Stream()
    got = api.score(**dp, workspace=api.Workspace("cuda"), stream=side)
    torch.cuda.synchronize()
    for k in ref:  # bit patterns: q_true is NaN for non-binary questions
        assert torch.equal(ref[k].view(torch.int32), got[k].view(torch.int32)), k
    assert int(got["dev_flags"][0]) == 0


def test_stream_read_checksum(jet):
    """The plain-read helper the bench times reads every word once: its XOR checksum
    matches the host's, for a buffer that is not a multiple of the grid's stride."""
    from candidate_likelihood_scoring_amd import api
    rng = np.random.default_rng(12)
    host = rng.integers(0, 2**32, size=(1 << 22) + 12, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.stream_read(buf, out)
    torch.cuda.synchronize()
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host))


@pytest.mark.parametrize("d", [32, 128])
def test_empty_problem(jet, d):
    p = wl.make_problem(V=100, d=d, n_q=0, seed=2, n_extra_rows=3)
    out = _run(jet, p)
    ref = jo.score(p)
    assert out["dev_flags"][0] == 0
    assert np.max(np.abs(out["row_lse"] - ref["lse"])) < 2e-3


@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
def test_no_rows_clears_the_flag_word(jet, w_dtype):
    """A problem without rows (hence without tokens, candidates or questions) runs no
    projection; the call still clears a caller's stale flag word."""
    p = wl.make_problem(V=300, d=128, n_q=0, seed=3, w_dtype=w_dtype)
    assert p["n_rows"] == 0
    dp = jet.to_device(p, "cuda")
    buf = api.alloc_outputs(api.make_problem(**dp), "cuda")
    buf["dev_flags"].fill_(7)
    jet.score_problem(dp, out=buf)
    torch.cuda.synchronize()
    assert int(buf["dev_flags"][0]) == 0


@pytest.mark.parametrize("d", [32, 128])
def test_bad_indices_set_flags_without_faulting(jet, d):
    """Out-of-range rows/targets and malformed offsets are bounds-checked on the device
    (d = 32: the register-staged kernel; d = 128: the streaming kernel)."""
    p = wl.make_problem(V=500, d=d, n_q=4, K=(2, 4), lengths=(1, 3), layout="prefix", seed=41)
    q = dict(p)
    q["tok_target"] = p["tok_target"].copy()
    q["tok_target"][0] = p["V"] + 7
    out = _run(jet, q)
    assert out["dev_flags"][0] & 2
    assert np.isnan(out["tok_logp"][0])
    # the same output buffers again with valid indices: the call clears the flag word
    # itself; the other tokens' values do not depend on the bad one
    dq = jet.to_device(q, "cuda")
    buf = api.alloc_outputs(api.make_problem(**dq), "cuda")
    jet.score_problem(dq, out=buf)
    torch.cuda.synchronize()
    assert int(buf["dev_flags"][0]) & 2
    clean = jet.to_numpy(jet.score_problem(jet.to_device(p, "cuda"), out=buf))
    assert clean["dev_flags"][0] == 0
    assert np.array_equal(out["tok_logp"][1:], clean["tok_logp"][1:])
    assert np.array_equal(out["row_lse"], clean["row_lse"])
    q = dict(p)
    q["tok_row"] = p["tok_row"].copy()
    q["tok_row"][1] = p["n_rows"] + 100
    out = _run(jet, q)
    assert out["dev_flags"][0] & 1
    q = dict(p)
    q["cand_tok_off"] = p["cand_tok_off"].copy()
    q["cand_tok_off"][2] = q["cand_tok_off"][1]  # an empty candidate
    out = _run(jet, q)
    assert out["dev_flags"][0] & 4
    q = dict(p)
    K = np.diff(p["q_cand_off"])
    q["q_true_idx"] = (K + 3).astype(np.int32)
    out = _run(jet, q)
    assert out["dev_flags"][0] & 8
    # offset arrays that do not start at 0 or end at n_cand / n_tok, every question and
    # candidate well formed in itself: a candidate outside every question, or a token outside
    # every candidate, raises the flag too
    p2 = wl.make_problem(V=500, d=d, n_q=4, K=(2, 4), lengths=(2, 3), layout="own", seed=43)
    for key, pos, delta in (("q_cand_off", 0, 1), ("q_cand_off", -1, -1),
                            ("cand_tok_off", 0, 1), ("cand_tok_off", -1, -1)):
        q = dict(p2)
        q[key] = p2[key].copy()
        q[key][pos] += delta
        out = _run(jet, q)
        assert out["dev_flags"][0] == 4, (key, pos, out["dev_flags"][0])


def test_debug_validate_rejects_before_launch(jet, monkeypatch):
    """With JET_DEBUG_VALIDATE=1 the binding validates host copies of the index arrays: a
    bad target (jet_score) or union id (jet_score_restricted) raises JET_E_INDEX and the
    outputs are left untouched; valid calls still score."""
    from candidate_likelihood_scoring_amd import _lib
    p = wl.make_problem(V=500, d=128, n_q=4, K=(2, 4), lengths=(1, 3), layout="prefix", seed=42)
    monkeypatch.setenv("JET_DEBUG_VALIDATE", "1")
    good = _run(jet, p)
    assert int(good["dev_flags"][0]) == 0
    q = dict(p, tok_target=p["tok_target"].copy())
    q["tok_target"][0] = p["V"] + 7
    dq = jet.to_device(q, "cuda")
    out = {k: torch.full_like(v, -5) for k, v in api.score(**jet.to_device(p, "cuda")).items()}
    torch.cuda.synchronize()
    with pytest.raises(_lib.JetError) as e:
        api.score(**dq, out=out)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert all(bool((v == -5).all()) for v in out.values())
    rp = wl.make_restricted(n_fields=5, V=1000, d=64, K=(1, 9), seed=3)
    rd = {k: v for k, v in jet.restricted_to_device(rp, "cuda").items() if not k.startswith("host_")}
    rd["union_ids"][0] = rp["V"] + 3
    with pytest.raises(_lib.JetError) as e:
        api.score_restricted(**rd)
    assert e.value.status == -4


def test_deterministic(jet):
    p = wl.make_problem(V=20011, d=256, n_q=20, K=(2, 10), lengths=(1, 5), layout="prefix", seed=51)
    a = _run(jet, p)
    b = _run(jet, p)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


# ----------------------------------------------------------------------------------------
# the five workloads at full size
# ----------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def binary_enum():
    return wl.binary_enum()


def test_binary_enum_full(jet, binary_enum):
    p = binary_enum
    log("[gpu] binary_enum full")
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] binary_enum errs {compare(p, out, ref, 'binary_enum')}")


@pytest.mark.parametrize("kind", ["wide", "planted"])
def test_stress(jet, kind):
    p = wl.stress(kind)
    log(f"[gpu] stress {kind}")
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] stress {kind} errs {compare(p, out, ref, kind)}")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
def test_stress_tiled(jet, h_dtype):
    """Peaked logits (W ~ N(0, 16/d), logit standard deviation about 4) through the
    matrix-core kernels, whose epilogue rescales each row's running sum tile by tile."""
    p = wl.make_problem(V=5003, d=256, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=85,
                        h_dtype=h_dtype, n_extra_rows=300, w_std=4.0 / 16.0)
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    assert kern.startswith("k_project_tiled"), kern
    out = _run(jet, p)
    ref = jo.score(p)
    log(f"[gpu] stress tiled {h_dtype} ({kern}) errs {compare(p, out, ref, 'stress_tiled')}")


@pytest.mark.parametrize("h_dtype", ["bf16", "f32"])
def test_many_rows(jet, h_dtype):
    """300,050 rows (2,345 tiles of 128 or 1,173 of 256) of which most score no token: the
    full-vocabulary LSE of every row (row_lse) on sampled rows across the whole range,
    including the shifted last row tile, against the oracle."""
    p = wl.make_problem(V=4099, d=128, n_q=50, K=(2, 6), layout="field", seed=91,
                        h_dtype=h_dtype, n_extra_rows=300000)
    n = p["n_rows"]
    kern = api.projection_kernel(api.make_problem(**jet.to_device(p, "cuda")))
    log(f"[gpu] many rows {h_dtype} rows={n} ({kern})")
    assert kern.startswith("k_project_tiled"), kern
    out = _run(jet, p)
    _full_size_properties(p, out)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.asarray(p["tok_row"]), rng.choice(n, 200, replace=False),
                                     np.arange(n - 300, n), np.arange(0, 40)]))
    ref = jo.score(p, rows=rows)
    log(f"[gpu] many rows errs {compare(p, out, ref, 'many_rows', sampled=True)}")


def _rows_of_questions(p, qs):
    co, qo = p["cand_tok_off"], p["q_cand_off"]
    tok_row = np.arange(len(p["tok_target"])) if p["tok_row"] is None else p["tok_row"]
    rows = []
    for g in qs:
        t0, t1 = co[qo[g]], co[qo[g + 1]]
        rows.append(tok_row[t0:t1])
    return np.unique(np.concatenate(rows))


def _full_size_properties(p, out):
    qo = p["q_cand_off"]
    assert out["dev_flags"][0] == 0
    assert np.all(np.isfinite(out["tok_logp"])) and np.all(out["tok_logp"] < 0)
    sums = np.add.reduceat(out["cand_q"].astype(np.float64), qo[:-1])
    assert np.max(np.abs(sums - 1.0)) < 1e-5
    co = p["cand_tok_off"]
    s_from_l = np.add.reduceat(out["tok_logp"].astype(np.float64), co[:-1])
    assert np.max(np.abs(s_from_l - out["cand_s"])) < 1e-3
    K = np.diff(qo)
    assert np.all((out["q_argmax"] >= 0) & (out["q_argmax"] < K))


def test_multi_token_full_sampled(jet):
    p = wl.multi_token()
    log(f"[gpu] multi_token rows={p['n_rows']} tok={len(p['tok_target'])}")
    out = _run(jet, p)
    _full_size_properties(p, out)
    # duplicates: bitwise-equal log-probs for bitwise-equal rows at other positions
    for dst, src in p["dup_row_pairs"]:
        assert np.array_equal(out["row_lse"][dst], out["row_lse"][src])
    # full parity: every row, so every main question and every ordinal/binary subset
    log(f"[gpu] multi_token oracle on all {p['n_rows']} rows")
    ref = jo.score(p)
    errs = compare(p, out, ref, "multi_token")
    log(f"[gpu] multi_token errs {errs}")
    n_q = len(p["q_cand_off"]) - 1
    assert errs["argmax_checked"] + errs["argmax_in_band"] == n_q


def _one_question_per_row_tile(p, tile):
    """Questions whose rows cover, for every row tile, a row inside it (rows follow tokens,
    so each question owns a contiguous run of rows): the question holding the row 100 rows
    into each tile, plus the last question (the shifted last tile)."""
    co, qo = np.asarray(p["cand_tok_off"]), np.asarray(p["q_cand_off"])
    tok_row = np.arange(len(p["tok_target"])) if p["tok_row"] is None else np.asarray(p["tok_row"])
    first_row = tok_row[co[qo[:-1]]]
    n = p["n_rows"]
    qs = {len(qo) - 2}
    for t0 in range(0, n, tile):
        r = min(t0 + 100, n - 1)
        qs.add(int(np.searchsorted(first_row, r, side="right") - 1))
    return sorted(qs)


def test_large_batch_full_sampled(jet):
    """The headline workload in the benchmark's launch configuration; the oracle computes
    one question in every 256-row tile of the matrix-core kernel (104 of 512 questions),
    so every row tile's partials and captured targets are checked."""
    p = wl.large_batch()
    log(f"[gpu] large_batch rows={p['n_rows']}")
    out = _run(jet, p)
    _full_size_properties(p, out)
    qs = _one_question_per_row_tile(p, 256)
    rows = _rows_of_questions(p, qs)
    tiles = np.unique(rows // 256)
    log(f"[gpu] large_batch oracle on {len(qs)} questions, {len(rows)} rows, {len(tiles)} row tiles")
    assert len(tiles) == -(-p["n_rows"] // 256)
    ref = jo.score(p, rows=rows)
    errs = compare(p, out, ref, "large_batch", sampled=True)
    log(f"[gpu] large_batch errs {errs}")
    assert errs["argmax_checked"] + errs["argmax_in_band"] == len(qs)


def test_large_batch_deduplicated_full_sampled(jet):
    """The large workload with one row per predictor node of the history trie (the layout
    the bench's --dedup line times): 22,962 rows instead of 26,546, a different ragged
    last row tile; parity on sampled questions."""
    p = wl.large_batch()
    tok_node, node_tok = api.build_predictor_trie(p["tok_target"], p["cand_tok_off"], p["q_cand_off"])
    tok_row = np.arange(len(p["tok_target"])) if p.get("tok_row") is None else np.asarray(p["tok_row"])
    q = dict(p, H=np.ascontiguousarray(p["H"][tok_row[node_tok]]), n_rows=len(node_tok),
             tok_row=tok_node.astype(np.int32))
    log(f"[gpu] large_batch dedup rows={q['n_rows']}")
    out = _run(jet, q)
    _full_size_properties(q, out)
    qs = _one_question_per_row_tile(q, 256)
    rows = _rows_of_questions(q, qs)
    log(f"[gpu] large_batch dedup oracle on {len(qs)} questions, {len(rows)} rows")
    assert len(np.unique(rows // 256)) == -(-q["n_rows"] // 256)
    ref = jo.score(q, rows=rows)
    log(f"[gpu] large_batch dedup errs {compare(q, out, ref, 'large_batch_dedup', sampled=True)}")


@pytest.mark.parametrize("max_variant", [False, True])
def test_restricted(jet, max_variant):
    rp = wl.restricted(max_variant=max_variant)
    log(f"[gpu] restricted max={max_variant}")
    rd = jet.restricted_to_device(rp, "cuda")
    ou, os_ = jo.build_union(rp["field_ids"], rp["field_off"], rp["V"])
    assert np.array_equal(rd["host_union"], ou) and np.array_equal(rd["host_slot_uidx"], os_)
    out = jet.to_numpy(jet.score_restricted_problem(rd))
    torch.cuda.synchronize()
    assert out["dev_flags"][0] == 0
    ref = jo.score_restricted(rp)
    dl = np.max(np.abs(out["slot_logit"] - ref["slot_logit"]))
    dq = np.max(np.abs(out["slot_q"] - ref["slot_q"]))
    assert dl <= 2e-3 and dq <= Q_TOL, (dl, dq)
    dec = ref["field_gap"] > Q_TOL
    nd = check_decisions(out["field_argmax"], out["slot_logit"], rp["field_off"], rp["T"],
                         ref["field_argmax"], ref["field_gap"], ref["slot_q"], "restricted")
    # against the full-vocabulary path on the same inputs (LSE cancels in the field softmax)
    full = _run(jet, wl.restricted_as_full(rp))
    assert np.max(np.abs(full["cand_q"] - out["slot_q"])) <= Q_TOL
    assert np.array_equal(full["q_argmax"][dec], out["field_argmax"][dec])
    log(f"[gpu] restricted decisions {nd}")
    log(f"[gpu] restricted errs logit={dl:.2e} q={dq:.2e}")


@pytest.mark.parametrize("case", [
    dict(n_fields=5, V=1000, d=64, K=(1, 9), seed=3),
    dict(n_fields=70, V=30011, d=256, K=(1, 26), seed=4, shared_rows=True, n_rows=9),
    dict(n_fields=3, V=500, d=32, K=(2, 4), seed=5, h_dtype="bf16"),
    dict(n_fields=4, V=700, d=64, K=(1, 5), seed=6, w_dtype="f32"),
    # an fp32 head in one launch over two batches of four chunks
    dict(n_fields=7, V=3000, d=2560, K=(1, 26), seed=16, w_dtype="f32"),
    # several union tiles, two row tiles with a ragged tail, d = 512 + 96 (a partial k group)
    dict(n_fields=45, V=20000, d=608, K=(1, 26), seed=7),
    dict(n_fields=40, V=3000, d=1056, K=(1, 26), seed=8, h_dtype="bf16", n_rows=33),
    # the one-launch path with the hidden row in registers at its widest (five 512-wide
    # chunks), bf16 hidden states
    dict(n_fields=8, V=9000, d=2560, K=(2, 26), seed=12, h_dtype="bf16"),
    # the one-launch path with the hidden row in LDS: just past the registers; nine chunks
    # (a second batch of head loads with one chunk); at its widest
    dict(n_fields=6, V=5000, d=2592, K=(1, 26), seed=10),
    dict(n_fields=9, V=4000, d=4608, K=(1, 26), seed=13, h_dtype="bf16"),
    dict(n_fields=5, V=2000, d=16384, K=(2, 26), seed=14),
    # past its limits, the two-launch path: d above 16384, and more than 4096 slots; with
    # an fp32 head, gather, projection and field softmax
    dict(n_fields=4, V=1500, d=16416, K=(2, 26), seed=15),
    dict(n_fields=200, V=30011, d=128, K=(20, 26), seed=11),
    dict(n_fields=170, V=9000, d=64, K=(25, 26), seed=17, w_dtype="f32"),
])
def test_restricted_ragged(jet, case):
    rp = wl.make_restricted(T=1.7, **case)
    one_launch = rp["d"] <= 16384 and len(rp["field_ids"]) <= 4096
    log(f"[gpu] restricted d={rp['d']} slots={len(rp['field_ids'])} W {rp['w_dtype']} "
        f"H {rp['h_dtype']} ({'one launch' if one_launch else 'projection + field softmax'})")
    rd = jet.restricted_to_device(rp, "cuda")
    out = jet.to_numpy(jet.score_restricted_problem(rd))
    torch.cuda.synchronize()
    ref = jo.score_restricted(rp)
    tl = 1e-4 if rp["w_dtype"] == "f32" else 2e-3
    assert out["dev_flags"][0] == 0
    assert np.max(np.abs(out["slot_logit"] - ref["slot_logit"])) <= tl
    assert np.max(np.abs(out["slot_q"] - ref["slot_q"])) <= Q_TOL
    check_decisions(out["field_argmax"], out["slot_logit"], rp["field_off"], rp["T"],
                    ref["field_argmax"], ref["field_gap"], ref["slot_q"], f"restricted {case}")


def test_restricted_bad_union_id(jet):
    """A union id outside [0, V) on the device reads as a zero head row and raises
    JET_FLAG_BAD_UNION; fields that do not use it are scored as usual."""
    rp = wl.make_restricted(n_fields=12, V=4000, d=256, K=(2, 6), seed=9)
    rd = jet.restricted_to_device(rp, "cuda")
    bad = len(rd["host_union"]) - 1
    rd["union_ids"][bad] = rp["V"] + 7
    out = jet.to_numpy(jet.score_restricted_problem(rd))
    torch.cuda.synchronize()
    assert out["dev_flags"][0] & 16
    ref = jo.score_restricted(rp)
    fo = rp["field_off"]
    uses = np.array([bad in rd["host_slot_uidx"][fo[f]:fo[f + 1]] for f in range(len(fo) - 1)])
    assert uses.any() and not uses.all()
    slot_bad = rd["host_slot_uidx"] == bad
    assert np.all(out["slot_logit"][slot_bad] == 0.0)
    keep = np.repeat(~uses, np.diff(fo))
    assert np.max(np.abs(out["slot_logit"][keep] - ref["slot_logit"][keep])) <= 2e-3
    assert np.max(np.abs(out["slot_q"][keep] - ref["slot_q"][keep])) <= Q_TOL


@pytest.mark.parametrize("case", [
    dict(n_fields=12, V=3000, d=256, K=(3, 6), seed=21),                   # one launch, registers
    dict(n_fields=12, V=3000, d=2048, K=(3, 6), seed=22, h_dtype="bf16"),  # one launch, registers
    dict(n_fields=12, V=3000, d=4096, K=(3, 6), seed=23),                  # one launch, LDS
    dict(n_fields=170, V=9000, d=128, K=(25, 26), seed=24),                # > 4096 slots
    dict(n_fields=12, V=3000, d=96, K=(3, 6), seed=25, w_dtype="f32"),     # one launch, LDS
    dict(n_fields=170, V=9000, d=64, K=(25, 26), seed=26, w_dtype="f32"),  # > 4096 slots
], ids=["fields_nc2", "fields_nc5", "fields_lds", "two_launch", "f32_lds", "f32_gather"])
def test_restricted_bad_device_indices(jet, case):
    """Malformed indices met on the device, the same on every restricted kernel: a field
    row outside [0, n_rows) gives NaN logits and argmax -1 for its field; a slot index
    outside [0, n_union) gives that slot a NaN logit (the field's softmax is then NaN, and
    its argmax is taken over the other slots); an empty field (malformed offsets) gets
    argmax -1.  Flags: JET_FLAG_BAD_UNION | JET_FLAG_BAD_OFFSETS.  Every other field is
    scored as usual."""
    rp = wl.make_restricted(T=1.3, **case)
    rd = jet.restricted_to_device(rp, "cuda")
    fo = np.asarray(rp["field_off"])
    f_row, f_slot, f_empty = 2, 5, 8
    rd["field_row"][f_row] = rp["n_rows"] + 5
    bad_j = int(fo[f_slot]) + 1
    rd["slot_uidx"][bad_j] = len(rd["host_union"]) + 3
    rd["field_slot_off"][f_empty + 1] = int(fo[f_empty])  # field 8 empty, field 9 widened
    out = jet.to_numpy(jet.score_restricted_problem(rd))
    torch.cuda.synchronize()
    log(f"[gpu] restricted bad indices d={rp['d']} slots={len(rp['field_ids'])} W {rp['w_dtype']}: "
        f"flags {out['dev_flags'][0]}")
    assert out["dev_flags"][0] == 16 | 4
    ref = jo.score_restricted(rp)
    tl = 1e-4 if rp["w_dtype"] == "f32" else 2e-3
    # bad row: every logit and q NaN, no decision
    sl = slice(fo[f_row], fo[f_row + 1])
    assert np.all(np.isnan(out["slot_logit"][sl])) and np.all(np.isnan(out["slot_q"][sl]))
    assert out["field_argmax"][f_row] == -1
    # bad slot index: that logit NaN, the others exact; q NaN; argmax over the others
    sl = slice(fo[f_slot], fo[f_slot + 1])
    lg = out["slot_logit"][sl].copy()
    good = np.arange(lg.size) != bad_j - fo[f_slot]
    assert np.isnan(lg[~good]).all() and not np.isnan(lg[good]).any()
    assert np.max(np.abs(lg[good] - ref["slot_logit"][sl][good])) <= tl
    assert np.all(np.isnan(out["slot_q"][sl]))
    b = ref["slot_logit"][sl] / rp["T"]
    b[~good] = -np.inf
    top = np.sort(b)[::-1]
    if top[0] - top[1] > 1e-3:
        assert out["field_argmax"][f_slot] == int(np.argmax(b))
    # empty field: no decision
    assert out["field_argmax"][f_empty] == -1
    # every other field as the oracle has it
    others = [f for f in range(len(fo) - 1) if f not in (f_row, f_slot, f_empty, f_empty + 1)]
    keep = np.repeat(np.isin(np.arange(len(fo) - 1), others), np.diff(fo))
    assert np.max(np.abs(out["slot_logit"][keep] - ref["slot_logit"][keep])) <= tl
    assert np.max(np.abs(out["slot_q"][keep] - ref["slot_q"][keep])) <= Q_TOL
    sub_off = np.concatenate([[0], np.cumsum(np.diff(fo)[others])])
    check_decisions(out["field_argmax"][others], out["slot_logit"][keep], sub_off, rp["T"],
                    ref["field_argmax"][others], ref["field_gap"][others], ref["slot_q"][keep],
                    f"restricted bad indices {case}")


@pytest.mark.parametrize("case", [
    dict(n_fields=12, V=3000, d=256, K=(3, 6), seed=21),
    dict(n_fields=12, V=3000, d=4096, K=(3, 6), seed=23),
    dict(n_fields=170, V=9000, d=128, K=(25, 26), seed=24),
    dict(n_fields=170, V=9000, d=64, K=(25, 26), seed=26, w_dtype="f32"),
], ids=["fields_nc2", "fields_lds", "two_launch", "f32_gather"])
def test_restricted_offset_ends_flagged(jet, case):
    """Field offsets that do not start at 0 or end at n_slots, every field well formed in
    itself (a slot outside every field): JET_FLAG_BAD_OFFSETS alone, on every restricted
    kernel."""
    rp = wl.make_restricted(**case)
    for pos, delta in ((0, 1), (-1, -1)):
        rd = jet.restricted_to_device(rp, "cuda")
        rd["field_slot_off"][pos] += delta
        out = jet.to_numpy(jet.score_restricted_problem(rd))
        torch.cuda.synchronize()
        assert out["dev_flags"][0] == 4, (case, pos, out["dev_flags"][0])


# ----------------------------------------------------------------------------------------
# no stray writes: outputs and workspace padded with a canary that must survive the call
# ----------------------------------------------------------------------------------------

_CANARY = 0x7FA5A5A5  # a NaN bit pattern that no kernel writes
_PAD = 64


def _padded_outputs(names_sizes, dev):
    full, views = {}, {}
    for name, (n, dtype) in names_sizes.items():
        buf = torch.full((n + _PAD,), _CANARY, dtype=torch.int32, device=dev)
        full[name] = buf
        views[name] = buf[:n] if dtype == torch.int32 else buf[:n].view(torch.float32)
    return full, views


def _tails_intact(full, names_sizes):
    return {name: bool((full[name][n:] == _CANARY).all()) for name, (n, _) in names_sizes.items()}


class _CanaryWorkspace(api.Workspace):
    """A workspace of exactly the requested size followed by 4 KB of canary bytes."""

    def get(self, nbytes):
        if nbytes > self.size or self.buf is None:
            self.buf = torch.full((nbytes + 256 + 4096,), 0xA5, dtype=torch.uint8, device=self.device)
            self.base = (self.buf.data_ptr() + 255) & ~255
            self.size = nbytes
        return self.base, self.size

    def tail_intact(self):
        start = self.base - self.buf.data_ptr() + self.size
        return bool((self.buf[start:] == 0xA5).all())


_CANARY_CASES = [
    dict(V=4099, d=32, n_q=5, K=(1, 9), lengths=(1, 4), layout="prefix", seed=71),
    dict(V=5003, d=128, n_q=7, K=(1, 12), lengths=(1, 5), layout="prefix", seed=72),
    dict(V=3001, d=64, n_q=4, K=(1, 6), lengths=(1, 4), layout="own", seed=73, w_dtype="f32"),
    dict(V=1283, d=256, n_q=25, K=(1, 12), lengths=(1, 5), layout="prefix", seed=74,
         h_dtype="bf16", n_extra_rows=211),
    dict(V=2500, d=64, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=75, n_extra_rows=250),
]


@pytest.mark.parametrize("case", _CANARY_CASES, ids=[f"canary{i}" for i in range(len(_CANARY_CASES))])
def test_no_writes_past_outputs_or_workspace(jet, case):
    p = wl.make_problem(**case)
    pd = jet.to_device(p, "cuda")
    prob = api.make_problem(**pd)
    log(f"[gpu] canary {case} kernel={api.projection_kernel(prob)}")
    f, i = torch.float32, torch.int32
    sizes = dict(tok_logp=(prob.n_tok, f), row_lse=(prob.n_rows, f), cand_s=(prob.n_cand, f),
                 cand_q=(prob.n_cand, f), q_argmax=(prob.n_q, i), q_true=(prob.n_q, f),
                 q_expect=(prob.n_q, f), q_gold_nll=(prob.n_q, f), q_confidence=(prob.n_q, f),
                 q_mass=(prob.n_q, f), dev_flags=(1, i))
    full, views = _padded_outputs(sizes, "cuda")
    views["dev_flags"].zero_()
    ws = _CanaryWorkspace("cuda")
    jet.score_problem(pd, out=views, workspace=ws)
    torch.cuda.synchronize()
    assert int(views["dev_flags"][0]) == 0
    assert all(_tails_intact(full, sizes).values()), _tails_intact(full, sizes)
    assert ws.tail_intact()
    ref = jo.score(p)
    out = {k: v.cpu().numpy() for k, v in views.items()}
    compare(p, out, ref, f"canary {case}")


@pytest.mark.parametrize("w_dtype,d,n_fields,K", [
    ("bf16", 608, 45, (1, 26)), ("f32", 96, 45, (1, 26)),         # one launch
    ("bf16", 96, 170, (25, 26)), ("f32", 96, 170, (25, 26)),      # past 4096 slots
], ids=["bf16_one_launch", "f32_one_launch", "bf16_two_launch", "f32_gather"])
def test_restricted_no_writes_past_outputs_or_workspace(jet, w_dtype, d, n_fields, K):
    rp = wl.make_restricted(n_fields=n_fields, V=20000, d=d, K=K, seed=76, w_dtype=w_dtype)
    rd = jet.restricted_to_device(rp, "cuda")
    n_slots, n_f = int(rp["field_off"][-1]), len(rp["field_off"]) - 1
    f, i = torch.float32, torch.int32
    sizes = dict(slot_logit=(n_slots, f), slot_q=(n_slots, f), field_argmax=(n_f, i),
                 dev_flags=(1, i))
    full, views = _padded_outputs(sizes, "cuda")
    views["dev_flags"].zero_()
    ws = _CanaryWorkspace("cuda")
    jet.score_restricted_problem(rd, out=views, workspace=ws)
    torch.cuda.synchronize()
    assert int(views["dev_flags"][0]) == 0
    assert all(_tails_intact(full, sizes).values()), _tails_intact(full, sizes)
    assert ws.tail_intact()
    ref = jo.score_restricted(rp)
    tl = 1e-4 if w_dtype == "f32" else 2e-3
    assert np.max(np.abs(views["slot_logit"].cpu().numpy() - ref["slot_logit"])) <= tl


# ----------------------------------------------------------------------------------------
# concurrency and graph capture
# ----------------------------------------------------------------------------------------

_GRAPH_CASES = {
    "stream": dict(V=5003, d=128, n_q=9, K=(1, 12), layout="field", seed=81),
    "tiled_padded": dict(V=5003, d=128, n_q=9, K=(1, 12), lengths=(1, 6), layout="prefix", seed=81),
    "tiled": dict(V=3001, d=128, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=82,
                  h_dtype="bf16", n_extra_rows=300),
    "tiled_f32": dict(V=2500, d=64, n_q=30, K=(2, 8), lengths=(1, 6), layout="own", seed=83,
                      n_extra_rows=250),
}


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def test_concurrent_streams_with_own_workspaces(jet):
    """Calls on different streams with different workspaces may overlap; each gives the
    bits it gives alone."""
    probs = [jet.to_device(wl.make_problem(**c), "cuda") for c in _GRAPH_CASES.values()]
    alone = [api.score(**dp) for dp in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in probs]
    wss = [api.Workspace("cuda") for _ in probs]
    outs = []
    for _ in range(3):  # enqueue every problem on its own stream, several times, no syncs
        outs = [api.score(**dp, workspace=ws, stream=st) for dp, ws, st in zip(probs, wss, streams)]
    torch.cuda.synchronize()
    for a, b in zip(alone, outs):
        for k in a:
            assert torch.equal(_bits(a[k]), _bits(b[k])), k


def test_concurrent_streams_with_default_workspace(jet):
    """Calls without a workspace argument on different streams (the module's default
    workspace is one per device and stream), enqueued three times without synchronisation,
    give the bits each gives alone; so do the restricted path's."""
    probs = [jet.to_device(wl.make_problem(**c), "cuda") for c in _GRAPH_CASES.values()]
    rp = wl.make_restricted(n_fields=45, V=20000, d=608, K=(1, 26), seed=86)
    rd = {k: v for k, v in jet.restricted_to_device(rp, "cuda").items() if not k.startswith("host_")}
    alone = [api.score(**dp) for dp in probs]
    alone_r = api.score_restricted(**rd)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(len(probs) + 1)]
    assert len({s.cuda_stream for s in streams}) == len(streams)
    for _ in range(3):
        outs = [api.score(**dp, stream=st) for dp, st in zip(probs, streams)]
        out_r = api.score_restricted(**rd, stream=streams[-1])
    torch.cuda.synchronize()
    for a, b in zip(alone, outs):
        for k in a:
            assert torch.equal(_bits(a[k]), _bits(b[k])), k
    for k in alone_r:
        assert torch.equal(_bits(alone_r[k]), _bits(out_r[k])), k


@pytest.mark.parametrize("name", list(_GRAPH_CASES))
def test_graph_capture_replays_match_eager(jet, name):
    """The whole jet_score sequence (no memsets, no allocation, no host synchronisation) can
    be captured in a HIP graph; every replay, with other device work and synchronisations
    between replays, gives the eager bits."""
    dp = jet.to_device(wl.make_problem(**_GRAPH_CASES[name]), "cuda")
    eager = api.score(**dp)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ws = api.Workspace("cuda")
    out = {k: torch.empty_like(v) for k, v in eager.items()}
    with torch.cuda.stream(side):
        api.score(**dp, out=out, workspace=ws, stream=side)  # sizes the workspace first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        api.score(**dp, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out.values():
            v.fill_(-7)  # eager work between replays: scribble over the outputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(_bits(eager[k]), _bits(out[k])), (rep, k)
    del g


def test_restricted_graph_capture_replays_match_eager(jet):
    rp = wl.make_restricted(n_fields=45, V=20000, d=608, K=(1, 26), seed=84)
    rd = {k: v for k, v in jet.restricted_to_device(rp, "cuda").items() if not k.startswith("host_")}
    eager = api.score_restricted(**rd)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ws = api.Workspace("cuda")
    out = {k: torch.empty_like(v) for k, v in eager.items()}
    with torch.cuda.stream(side):
        api.score_restricted(**rd, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        api.score_restricted(**rd, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(_bits(eager[k]), _bits(out[k])), (rep, k)
    del g
