"""Pins for the oracle's top-k gate against closed forms, brute force and scipy.

Definition: ELDR page, "Core idea / structure / operation" (standard top-k
gating, unchanged) and GRACE-MoE page, section 3 (top-k routing).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


def _beats(v, a, b):
    """Total order written out: a precedes b (NaN counts as -inf)."""
    va = -math.inf if math.isnan(v[a]) else v[a]
    vb = -math.inf if math.isnan(v[b]) else v[b]
    return va > vb or (va == vb and a < b)


def _golden_cases():
    with open(os.path.join(GOLDEN, "gate_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_gate_golden(case):
    lg = np.array([[_val(v) for v in row] for row in case["logits"]], dtype=np.float32)
    ids, w = O.gate(lg, case["k"], bool(case["renormalize"]))
    np.testing.assert_array_equal(ids, np.array(case["ids"], dtype=np.int32))
    np.testing.assert_allclose(w.astype(np.float64), np.array(case["weights"]), rtol=0, atol=1e-7)


def test_gate_bruteforce_tiny_E():
    """Exactly one k-subset has every member before every non-member; it is the output."""
    rng = np.random.default_rng(1)
    for E in range(1, 8):
        for k in range(1, E + 1):
            for trial in range(6):
                if trial % 2:
                    row = rng.integers(-2, 2, size=E).astype(np.float32)   # tie storm
                else:
                    row = rng.standard_normal(E).astype(np.float32)
                if trial == 5 and E > 2:
                    row[0] = np.nan
                    row[1] = -0.0
                    row[2] = 0.0
                ids, _ = O.gate(row[None, :], k)
                v = [float(x) for x in row]
                winners = []
                for S in itertools.combinations(range(E), k):
                    rest = [e for e in range(E) if e not in S]
                    if all(_beats(v, a, b) for a in S for b in rest):
                        winners.append(set(S))
                assert len(winners) == 1
                assert set(ids[0].tolist()) == winners[0]
                # slots in descending order of the same total order
                for j in range(k - 1):
                    assert _beats(v, ids[0, j], ids[0, j + 1])


def test_gate_rows_have_k_distinct_ids():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((300, 40)).astype(np.float32)
    lg[::7] = np.round(lg[::7])                      # many exact ties
    ids, w = O.gate(lg, 6)
    assert ids.dtype == np.int32 and ids.shape == (300, 6)
    assert ((ids >= 0) & (ids < 40)).all()
    assert all(len(set(r)) == 6 for r in ids.tolist())
    assert (np.diff(w, axis=1) <= 0).all()            # weights non-increasing


def test_gate_weights_sum_to_one_and_k1_is_exactly_one():
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((500, 64)) * 3).astype(np.float32)
    _, w = O.gate(lg, 8)
    assert np.abs(w.astype(np.float64).sum(axis=1) - 1.0).max() <= 1e-6
    _, w1 = O.gate(lg, 1)
    assert (w1 == np.float32(1.0)).all()


def test_gate_renormalized_is_softmax_of_chosen_logits():
    """Full softmax, top-k, renormalise == softmax over the k chosen logits (scipy)."""
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((200, 32)) * 2).astype(np.float32)
    ids, w = O.gate(lg, 5, True)
    chosen = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    ref = scipy.special.softmax(chosen, axis=1)
    np.testing.assert_allclose(w, ref.astype(np.float32), rtol=0, atol=2e-7)
    # and equals renormalising the full softmax probabilities
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    p = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, p / p.sum(axis=1, keepdims=True), rtol=0, atol=2e-7)


def test_gate_unnormalized_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(5)
    lg = (rng.standard_normal((100, 16)) * 4).astype(np.float32)
    ids, w = O.gate(lg, 16, False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), axis=1),
                               rtol=0, atol=2e-7)
    # every expert appears once, in descending order of probability
    assert (np.sort(ids, axis=1) == np.arange(16)).all()


def test_gate_shift_invariance():
    """Adding the same exactly representable constant to a row changes nothing."""
    rng = np.random.default_rng(6)
    lg = (rng.integers(-64, 64, size=(100, 24)) / 8.0).astype(np.float32)  # ties, exact
    ids0, w0 = O.gate(lg, 4)
    ids1, w1 = O.gate(lg + np.float32(3.5), 4)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_array_equal(w0, w1)


def test_gate_signed_zero_equal():
    lg = np.array([[0.0, -0.0, -0.0, 0.0]], dtype=np.float32)
    ids, w = O.gate(lg, 4)
    np.testing.assert_array_equal(ids, [[0, 1, 2, 3]])
    np.testing.assert_array_equal(w, np.full((1, 4), 0.25, dtype=np.float32))


def test_gate_rejects_bad_k():
    with pytest.raises(ValueError):
        O.gate(np.zeros((2, 3), dtype=np.float32), 4)
    with pytest.raises(ValueError):
        O.gate(np.zeros((2, 3), dtype=np.float32), 0)
