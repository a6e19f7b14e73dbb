"""Seeded random sweep of problem shapes through every projection plan, against the fp64
oracle (needs an MI355X).

Forty-two problems are drawn from one seed, six per plan family: the streaming kernel
(bf16 head, d % 64 == 0) with one 32-row tile and with 33 to 64 (fp32 H) or 128 (bf16
H) rows in one pass; the register-staged fallback (bf16 head, d not a multiple of 64);
the fp32 head on small problems (the k-split kernel); the tiled kernels just past the
streaming kernel's rows (one zero-padded row tile, or two with fp32 H); and the tiled
kernels with bf16 H and with fp32 H past 256 rows, d an even or odd number of 64-wide
stages.  Six more, from a second seed, are fp32 heads large enough for the fp32
streaming kernel.  Each draws its vocabulary size, d, layout (prefix row, one row per
field, a row per token), candidate counts and lengths, exact duplicates, temperature and
H dtype, and asserts the kernel the plan's documented rule picks.  Every output is
compared element by element over every row a token references plus a sample of
unreferenced rows.
"""
import numpy as np
import pytest

import oracle as jo
import workloads as wl
from tests.parity import compare, log

torch = pytest.importorskip("torch")
from candidate_likelihood_scoring_amd import api  # noqa: E402
pytestmark = pytest.mark.gpu

FAMILIES = ("stream", "stream_multi", "fallback", "f32_head", "tiled_mid", "tiled_bf16h",
            "tiled_f32h")


def plan_kernel(p):
    """The projection kernel of the plan's rule, from the problem's scalars."""
    rows, V, d, hf = p["n_rows"], p["V"], p["d"], p["h_dtype"] == "f32"
    if p["w_dtype"] == "f32":  # streaming with one workgroup per CU: 256-entry groups x row tiles
        tiles = 1 if rows <= 16 else -(-rows // 32)
        return "k_project_wg_f32" if -(-V // 256) * tiles >= 256 else "k_project_small_f32"
    if d % 64 == 0:
        if rows <= (64 if hf else 128) or V < 256:
            return "k_project_wg_bf16"
        return "k_project_tiled_m16x2" if hf else "k_project_tiled_m16"
    return "k_project_small_bf16"


def _cases(n=42, seed=4711):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fam = FAMILIES[i % len(FAMILIES)]
        pick = lambda xs: xs[int(rng.integers(0, len(xs)))]  # noqa: E731
        c = dict(T=float(pick([0.5, 1.0, 2.0, 3.7])), layout=pick(["prefix", "field", "own"]),
                 dups=int(rng.integers(0, 3)), seed=9000 + i, name=f"sweep{i}_{fam}",
                 K=(1, int(rng.integers(2, 13))), lengths=(1, int(rng.integers(1, 5))),
                 n_q=int(rng.integers(1, 6)), n_extra_rows=0)
        hd = pick(["f32", "bf16"])
        if fam == "stream":  # at most 2 questions x 8 candidates x 2 tokens: 32 rows
            c.update(d=pick([64, 128, 192, 256, 384, 512, 640, 960, 1024]), V=int(rng.integers(300, 120_000)),
                     h_dtype=hd, w_dtype="bf16", n_q=int(rng.integers(1, 3)),
                     K=(1, int(rng.integers(2, 9))), lengths=(1, int(rng.integers(1, 3))))
        elif fam in ("stream_multi", "tiled_mid"):  # one row per field, then unreferenced rows
            top = 64 if hd == "f32" else 128
            lo, hi = (33, top) if fam == "stream_multi" else (top + 1, 255)
            rows = int(rng.integers(lo, hi + 1))
            n_q = int(rng.integers(1, min(rows, 20) + 1))
            c.update(d=pick([128, 192, 256, 320, 384, 512]), V=int(rng.integers(256, 60_000)),
                     h_dtype=hd, w_dtype="bf16", layout="field", n_q=n_q, n_extra_rows=rows - n_q)
        elif fam == "fallback":  # never tiled: d is not a multiple of 64
            c.update(d=pick([32, 96, 160, 224, 288]), V=int(rng.integers(300, 60_000)),
                     h_dtype=hd, w_dtype="bf16")
        elif fam == "f32_head":
            c.update(d=pick([32, 64, 128, 160]), V=int(rng.integers(100, 30_000)),
                     h_dtype="f32", w_dtype="f32")
        elif fam == "tiled_bf16h":
            c.update(d=pick([64, 128, 192, 256, 320, 384]), V=int(rng.integers(256, 30_000)), h_dtype="bf16",
                     w_dtype="bf16", n_q=int(rng.integers(6, 15)), n_extra_rows=int(rng.integers(256, 500)))
        else:
            c.update(d=pick([64, 128, 192, 256, 320]), V=int(rng.integers(256, 30_000)),
                     h_dtype="f32", w_dtype="bf16", n_q=int(rng.integers(6, 15)),
                     n_extra_rows=int(rng.integers(256, 500)))
        out.append((fam, c))
    return out


def _f32_stream_cases(n=6, seed=4712):
    """fp32 heads large enough for the streaming kernel: V of 65,536 to 200,000 (256 to 782
    groups), 1 to 64 rows (the 16-row tile, one and two 32-row tiles), d with a 32-wide
    last stage or whole stages."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        pick = lambda xs: xs[int(rng.integers(0, len(xs)))]  # noqa: E731
        rows = (1, int(rng.integers(2, 17)), int(rng.integers(17, 65)))[i % 3]
        n_q = int(rng.integers(1, min(rows, 12) + 1))
        out.append(("f32_stream", dict(
            T=float(pick([0.5, 1.0, 2.0])), layout="field", dups=int(rng.integers(0, 3)),
            seed=9100 + i, name=f"sweep_f32_stream{i}", K=(1, int(rng.integers(2, 13))),
            n_q=n_q, n_extra_rows=rows - n_q, d=(32, 320, 96, 192, 64, 128)[i % 6],
            V=int(rng.integers(65_536, 200_000)), h_dtype="f32", w_dtype="f32")))
    return out


CASES = _cases() + _f32_stream_cases()


@pytest.mark.parametrize("fam,case", CASES, ids=[c["name"] for _, c in CASES])
def test_sweep(fam, case):
    from candidate_likelihood_scoring_amd import problem

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    p = wl.make_problem(**case)
    dev = problem.to_device(p, "cuda")
    kern = api.projection_kernel(api.make_problem(**dev))
    log(f"[gpu] {case['name']}: V={p['V']} d={p['d']} rows={p['n_rows']} tokens={len(p['tok_target'])} "
        f"H {p['h_dtype']} W {p['w_dtype']} T={p['T']} layout={case['layout']} dups={case['dups']} ({kern})")
    assert kern == plan_kernel(p), (fam, kern, plan_kernel(p))
    out = problem.to_numpy(problem.score_problem(dev))
    torch.cuda.synchronize()
    tok_row = np.arange(len(p["tok_target"])) if p["tok_row"] is None else np.asarray(p["tok_row"])
    rng = np.random.default_rng(case["seed"])
    spare = np.setdiff1d(np.arange(p["n_rows"]), tok_row)
    extra = rng.choice(spare, size=min(16, spare.size), replace=False) if spare.size else spare
    rows = np.union1d(np.unique(tok_row), extra)
    ref = jo.score(p, rows=rows)
    log(f"[gpu] errs {compare(p, out, ref, case['name'], sampled=True)} on {rows.size} rows")
