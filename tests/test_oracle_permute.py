"""Pins for the oracle's dispatch permutation: hand examples, a Python sort, invariants.

Definition: GRACE-MoE page, section 1 (dispatch sends each token to the experts
that own it); priority segment from the ExpertPlex page, "Adaptive Persistent
Kernels" (decode tiles first).
"""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "permute_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_permute_golden(case):
    ids = np.array(case["topk_ids"], dtype=np.int32)
    T = ids.shape[0]
    x = np.arange(T, dtype=np.float32)[:, None] * np.ones((1, 3), dtype=np.float32)
    p = O.permute(ids, case["E"], case["n_shared"], case["n_priority"], x)
    np.testing.assert_array_equal(p["group_offsets"], case["group_offsets"])
    np.testing.assert_array_equal(p["sorted_to_flat"], case["sorted_to_flat"])
    np.testing.assert_array_equal(p["flat_to_sorted"], case["flat_to_sorted"])
    np.testing.assert_array_equal(p["x_sorted"][:, 0], case["token_of_sorted"])
    np.testing.assert_array_equal(p["sorted_token"], case["token_of_sorted"])


def _python_reference(ids, E, S, P):
    """The same sort written with Python's sorted() over explicit tuples."""
    T, k = len(ids), len(ids[0])
    nseg = 2 if P > 0 else 1
    items = []
    for t in range(T):
        for j in range(k):
            seg = 1 if (P > 0 and t >= P) else 0
            items.append((seg * E + ids[t][j], t * k + j))
    for s in range(S):
        for t in range(T):
            items.append((nseg * E + s, T * k + s * T + t))
    order = sorted(items)
    G = nseg * E + S
    offsets = [sum(1 for g, _ in items if g < gg) for gg in range(G + 1)]
    return [f for _, f in order], offsets


@pytest.mark.parametrize("seed", range(12))
def test_permute_matches_python_sort(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 40))
    E = int(rng.integers(1, 12))
    k = int(rng.integers(1, E + 1))
    S = int(rng.integers(0, 3))
    P = int(rng.integers(0, T + 1)) if seed % 2 else 0
    distinct = seed % 3 != 0
    if distinct:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)   # repeats allowed
    p = O.permute(ids, E, S, P)
    s2f, offs = _python_reference(ids.tolist(), E, S, P)
    np.testing.assert_array_equal(p["sorted_to_flat"], s2f)
    np.testing.assert_array_equal(p["group_offsets"], offs)


@pytest.mark.parametrize("seed", range(6))
def test_permute_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    T, E, k, S = 257, 37, 5, 2
    P = 40 if seed % 2 else 0
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    x = rng.standard_normal((T, 16)).astype(np.float32)
    p = O.permute(ids, E, S, P, x)
    N = T * (k + S)
    s2f = p["sorted_to_flat"].astype(np.int64)
    f2s = p["flat_to_sorted"].astype(np.int64)
    # bijection
    assert sorted(s2f.tolist()) == list(range(N))
    np.testing.assert_array_equal(s2f[f2s], np.arange(N))
    # group sizes == histogram of groups; offsets == exclusive scan
    group, token, G, nseg = O.assignment_groups(ids, E, S, P)
    hist = np.bincount(group, minlength=G)
    np.testing.assert_array_equal(np.diff(p["group_offsets"]), hist)
    assert p["group_offsets"][0] == 0 and p["group_offsets"][-1] == N
    # group id non-decreasing along the sorted order, flat index increasing inside a group
    gs = group[s2f]
    assert (np.diff(gs) >= 0).all()
    same = np.diff(gs) == 0
    assert (np.diff(s2f)[same] > 0).all()
    # rows are bit copies of the token rows
    assert np.array_equal(p["x_sorted"].view(np.uint32), x[token[s2f]].view(np.uint32))
    # shared groups hold every token once, in token order
    for s in range(S):
        g = nseg * E + s
        lo, hi = p["group_offsets"][g], p["group_offsets"][g + 1]
        np.testing.assert_array_equal(token[s2f[lo:hi]], np.arange(T))


def test_permute_priority_segment_precedes():
    rng = np.random.default_rng(7)
    T, E, k, P = 50, 8, 3, 10
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    p = O.permute(ids, E, 0, P)
    s2f = p["sorted_to_flat"]
    tok = s2f // k
    # the first P*k sorted rows are exactly the priority tokens' assignments
    assert (tok[: P * k] < P).all() and (tok[P * k:] >= P).all()
    assert p["group_offsets"][E] == P * k


def test_expert_of_group():
    g = np.arange(2 * 4 + 3)
    np.testing.assert_array_equal(O.expert_of_group(g, 4, 3, 2),
                                  [0, 1, 2, 3, 0, 1, 2, 3, 4, 5, 6])
