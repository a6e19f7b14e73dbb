"""Host logic of bench.py that runs without a device: the parity record a bench line carries
(its outputs against the oracle result of the CPU-baseline leg) and the refusal of more than
one GPU."""
import numpy as np

import bench
import oracle as jo
import workloads as wl


def _as_outputs(ref):
    return dict(tok_logp=np.asarray(ref["tok_logp"], np.float32),
                cand_q=np.asarray(ref["cand_q"], np.float32),
                q_argmax=np.asarray(ref["q_argmax"], np.int32))


def test_parity_record_full_vocabulary():
    p = wl.make_config("tiny")
    ref = jo.score(p)
    rec = bench._parity(p, _as_outputs(ref), ref, restricted=False)
    assert rec["within_tolerance"] and rec["decision_mismatches"] == 0
    assert rec["tokens"] == len(p["tok_target"]) and rec["questions"] == 1
    assert rec["max_abs_dlogp"] < 1e-6 and rec["tol_logp"] == 1e-4  # fp32 head
    # a log-probability off by more than the tolerance, and a wrong decision, are reported
    bad = _as_outputs(ref)
    bad["tok_logp"][3] += 3e-4
    bad["q_argmax"][0] = (bad["q_argmax"][0] + 1) % 4
    rec = bench._parity(p, bad, ref, restricted=False)
    assert not rec["within_tolerance"]
    assert abs(rec["max_abs_dlogp"] - 3e-4) < 1e-6
    assert rec["decision_mismatches"] == (1 if rec["decisions_compared"] else 0)


def test_parity_record_sampled_questions():
    """Only what the oracle computed (a sample of questions) is compared."""
    p = wl.make_problem(V=700, d=64, n_q=6, K=(2, 5), lengths=(1, 3), layout="own", seed=5,
                        h_dtype="bf16")
    co, qo = p["cand_tok_off"], p["q_cand_off"]
    rows = np.arange(co[qo[2]])  # the first two questions' rows (a row per token)
    ref = jo.score(p, rows=rows)
    out = _as_outputs(jo.score(p))
    out["tok_logp"][-1] = 0.5  # outside the sample: not compared
    rec = bench._parity(p, out, ref, restricted=False)
    assert rec["questions"] == 2 and rec["tokens"] == int(co[qo[2]])
    assert rec["within_tolerance"] and rec["tol_logp"] == 2e-3


def test_parity_record_restricted():
    rp = wl.make_restricted(n_fields=6, V=3000, d=64, K=(2, 9), seed=8)
    ref = jo.score_restricted(rp)
    out = dict(slot_logit=np.asarray(ref["slot_logit"], np.float32),
               slot_q=np.asarray(ref["slot_q"], np.float32),
               field_argmax=np.asarray(ref["field_argmax"], np.int32))
    rec = bench._parity(rp, out, ref, restricted=True)
    assert rec["within_tolerance"] and rec["slots"] == len(rp["field_ids"])


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
