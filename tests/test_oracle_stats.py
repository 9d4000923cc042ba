"""Pins for the oracle's expert statistics: hand examples, brute force, numpy/sklearn.

Union: ELDR page, "What it solves".  Signature (count x IDF over a layer subset):
ELDR page, "Core idea / structure / operation".  Affinity and load from recorded
top-k selections: GRACE-MoE page, sections 3 and 4.
"""
import json
import os

import numpy as np
import pytest
from sklearn.feature_extraction.text import TfidfTransformer

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "stats_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_stats_golden(case):
    st = O.stats(np.array(case["topk_ids"], dtype=np.int32), case["E"],
                 np.array(case["req_offsets"], dtype=np.int32))
    for key in ("counts", "union_size", "union_mask", "affinity", "req_counts", "df"):
        np.testing.assert_array_equal(st[key], np.array(case[key]), err_msg=key)
    np.testing.assert_allclose(st["signature"], np.array(case["signature"], dtype=np.float32),
                               rtol=1e-7, atol=0)


def _brute(ids, E):
    """Pure-Python loops over tokens and slot pairs."""
    L, T, k = len(ids), len(ids[0]), len(ids[0][0])
    counts = [[0] * E for _ in range(L)]
    aff = [[[0] * E for _ in range(E)] for _ in range(L)]
    for l in range(L):
        for t in range(T):
            for a in ids[l][t]:
                counts[l][a] += 1
                for b in ids[l][t]:
                    aff[l][a][b] += 1
    return counts, aff


@pytest.mark.parametrize("seed", range(5))
def test_stats_bruteforce_and_invariants(seed):
    rng = np.random.default_rng(seed)
    L, T, E, k = 3, int(rng.integers(1, 60)), int(rng.integers(2, 20)), 0
    k = int(rng.integers(1, E + 1))
    ids = np.stack([np.argsort(rng.random((T, E)), axis=1)[:, :k] for _ in range(L)]).astype(np.int32)
    st = O.stats(ids, E)
    c, a = _brute(ids.tolist(), E)
    np.testing.assert_array_equal(st["counts"], c)
    np.testing.assert_array_equal(st["affinity"], a)
    counts = st["counts"].astype(np.int64)
    A = st["affinity"].astype(np.int64)
    assert (counts.sum(axis=1) == T * k).all()
    assert (st["union_size"] <= min(E, T * k)).all()
    np.testing.assert_array_equal(st["union_size"], (counts > 0).sum(axis=1))
    np.testing.assert_array_equal(st["union_size"], st["union_mask"].sum(axis=1))
    for l in range(L):
        np.testing.assert_array_equal(A[l], A[l].T)
        np.testing.assert_array_equal(np.diag(A[l]), counts[l])
        np.testing.assert_array_equal(A[l].sum(axis=1), k * counts[l])
        assert A[l].sum() == T * k * k
        M = np.zeros((T, E), dtype=np.int64)
        M[np.arange(T)[:, None], ids[l]] = 1
        np.testing.assert_array_equal(A[l], M.T @ M)      # numpy integer matmul


def test_stats_repeated_ids_count_each_slot():
    ids = np.array([[[1, 1, 0]]], dtype=np.int32)
    st = O.stats(ids, 3)
    np.testing.assert_array_equal(st["counts"], [[1, 2, 0]])
    np.testing.assert_array_equal(st["affinity"][0], [[1, 2, 0], [2, 4, 0], [0, 0, 0]])


def test_stats_requests_sum_and_blocks():
    rng = np.random.default_rng(9)
    L, T, E, k = 2, 96, 16, 4
    ids = np.stack([np.argsort(rng.random((T, E)), axis=1)[:, :k] for _ in range(L)]).astype(np.int32)
    req = np.array([0, 10, 10, 50, 96], dtype=np.int32)            # one empty request
    st = O.stats(ids, E, req)
    rc = st["req_counts"].astype(np.int64)
    lens = np.diff(req)
    np.testing.assert_array_equal(rc.sum(axis=2), k * lens[:, None] * np.ones((1, L), np.int64))
    np.testing.assert_array_equal(rc.sum(axis=0), st["counts"])
    # KV-block granularity: 8-token blocks inside each request add up to the request
    blocks = sorted(set(range(0, T + 1, 8)) | set(req.tolist()))
    stb = O.stats(ids, E, np.array(blocks, dtype=np.int32))
    for r in range(len(req) - 1):
        inside = [b for b in range(len(blocks) - 1) if req[r] <= blocks[b] and blocks[b + 1] <= req[r + 1]]
        np.testing.assert_array_equal(stb["req_counts"][inside].sum(axis=0), rc[r])


def test_idf_matches_sklearn_unsmoothed_tfidf():
    """sklearn's unsmoothed idf is ln(n/df) + 1; ours is that minus one."""
    rng = np.random.default_rng(10)
    L, T, E, k = 3, 320, 24, 3
    ids = np.stack([np.argsort(rng.random((T, E)) ** (1 + np.arange(E) / 4), axis=1)[:, :k]
                    for _ in range(L)]).astype(np.int32)
    req = np.arange(0, T + 1, 16, dtype=np.int32)
    st = O.stats(ids, E, req)
    R = len(req) - 1
    X = st["req_counts"].reshape(R, L * E)
    used = X.sum(axis=0) > 0
    tf = TfidfTransformer(norm=None, smooth_idf=False, sublinear_tf=False).fit(X[:, used])
    np.testing.assert_allclose(st["idf"].reshape(-1)[used], tf.idf_ - 1.0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st["signature"].reshape(R, -1)[:, used],
                               (X[:, used] * (tf.idf_ - 1.0)).astype(np.float32), rtol=1e-6, atol=1e-6)
    assert (st["idf"].reshape(-1)[~used] == 0).all()


def test_df_equal_R_gives_zero_signature_and_caller_idf():
    ids = np.array([[[0, 1], [0, 2], [0, 1]]], dtype=np.int32)   # expert 0 in every request
    req = np.array([0, 1, 2, 3], dtype=np.int32)
    st = O.stats(ids, 3, req)
    assert (st["signature"][:, 0, 0] == 0).all()
    idf = np.array([[0.5, 2.0, -1.0]], dtype=np.float32)
    st2 = O.stats(ids, 3, req, idf)
    np.testing.assert_array_equal(st2["signature"][:, 0, :],
                                  np.array([[0.5, 2.0, 0.0], [0.5, 0.0, -1.0], [0.5, 2.0, 0.0]], np.float32))
