"""The seeded generators: determinism and the structural rules of each workload."""
import hashlib

import numpy as np
import pytest

import workloads as wl


def _digest(p):
    h = hashlib.sha256()
    for k in sorted(p):
        v = p[k]
        if isinstance(v, np.ndarray):
            h.update(k.encode())
            h.update(v.tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", ["tiny", "tiny_tie", "binary_enum", "multi_token", "restricted",
                                  "restricted_max", "large_batch"])
def test_structure_deterministic(name):
    a = wl.make_config(name, with_weights=False)
    b = wl.make_config(name, with_weights=False)
    assert _digest(a) == _digest(b)


def test_weights_deterministic_and_chunk_independent():
    a = wl.head_weights(3000, 64, 7)
    b = wl.head_weights(3000, 64, 7)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    c = wl.head_weights(3000, 64, 8)
    assert not np.array_equal(a, c)
    h = wl.hidden_states(10, 64, 7, "f32")
    assert h.dtype == np.float32 and abs(float(h.std()) - 1.0) < 0.1


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    bits = wl.bf16_bits(x)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def _check_csr(p):
    co, qo = p["cand_tok_off"], p["q_cand_off"]
    assert co[0] == 0 and qo[0] == 0
    assert np.all(np.diff(co) >= 1) and np.all(np.diff(qo) >= 1)
    assert co[-1] == len(p["tok_target"]) and qo[-1] == len(co) - 1
    assert np.all((p["tok_target"] >= 0) & (p["tok_target"] < p["V"]))
    rows = np.arange(len(p["tok_target"])) if p["tok_row"] is None else p["tok_row"]
    assert np.all((rows >= 0) & (rows < p["n_rows"]))


def test_tiny_layout():
    p = wl.tiny(with_weights=False)
    _check_csr(p)
    assert p["n_rows"] == 8 and len(p["tok_target"]) == 11
    assert sorted(np.diff(p["cand_tok_off"]).tolist()) == [2, 3, 3, 3]
    assert all(p["tok_row"][o] == 0 for o in p["cand_tok_off"][:-1])  # first token from the prefix row
    t = wl.tiny(tie=True, with_weights=False)
    co = t["cand_tok_off"]
    assert np.array_equal(t["tok_row"][co[2]:co[3]], t["tok_row"][co[3]:co[4]])
    assert np.array_equal(t["tok_target"][co[2]:co[3]], t["tok_target"][co[3]:co[4]])


def test_binary_enum_layout():
    p = wl.binary_enum(with_weights=False)
    _check_csr(p)
    K = np.diff(p["q_cand_off"])
    assert len(K) == 32 and np.all(K[:8] == 2) and np.all((K[8:] >= 3) & (K[8:] <= 26))
    assert np.all(np.diff(p["cand_tok_off"]) == 1)
    for f in range(32):
        a, b = p["q_cand_off"][f], p["q_cand_off"][f + 1]
        assert np.all(p["tok_row"][a:b] == f)
        assert len(set(p["tok_target"][a:b].tolist())) == b - a


def test_multi_token_layout():
    p = wl.multi_token(with_weights=False)
    _check_csr(p)
    K = np.diff(p["q_cand_off"])
    assert K.tolist() == [64] * 8 + [5] * 8 + [2] * 8
    assert np.array_equal(p["tok_row"][:p["n_primary_tok"]], np.arange(p["n_primary_tok"]))
    assert p["tok_row"].max() < p["n_rows"]
    m = np.diff(p["cand_tok_off"])
    assert m.min() >= 1 and m.max() <= 12
    assert np.all(p["q_true_idx"][:16] == -1) and np.all(p["q_true_idx"][16:] == 1)


def test_large_batch_layout():
    p = wl.large_batch(with_weights=False)
    _check_csr(p)
    assert p["tok_row"] is None and p["n_rows"] == len(p["tok_target"])
    assert np.all(np.diff(p["q_cand_off"]) == 8) and len(p["q_cand_off"]) == 513


def test_restricted_layout():
    p = wl.restricted(with_weights=False)
    K = np.diff(p["field_off"])
    assert len(K) == 32 and np.all(K[:8] == 2)
    m = wl.restricted(max_variant=True, with_weights=False)
    assert len(np.unique(m["field_ids"])) == 832
