"""Pins of the oracle's continuous (softmax-probability) request signature.

The ELDR page ("Core idea / structure / operation") compares its count x IDF
signature with continuous alternatives such as the softmax gate probability;
the oracle takes that alternative as the per-request sum of each token's
full-E softmax.  The pins check what that definition fixes: every token
contributes probabilities that sum to one, equal logits give 1/E each, a
constant shift of a token's logits changes nothing, two experts give the
logistic function, requests add up when split, and -inf / NaN logits drop out.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O


def _rand(L, T, E, seed):
    return np.random.default_rng(seed).normal(size=(L, T, E)).astype(np.float32) * 3


def test_each_token_adds_probability_one():
    lg = _rand(3, 40, 17, 0)
    offs = np.array([0, 5, 5, 19, 40], dtype=np.int32)
    sig = O.prob_signature(lg, offs)
    sizes = np.diff(offs).astype(np.float64)
    assert sig.shape == (4, 3, 17)
    assert np.allclose(sig.sum(axis=2), sizes[:, None], rtol=0, atol=1e-12)


def test_equal_logits_give_one_over_E():
    lg = np.full((2, 12, 7), 0.625, dtype=np.float32)
    sig = O.prob_signature(lg, np.array([0, 4, 12], dtype=np.int32))
    assert np.allclose(sig[0], 4 / 7, atol=1e-14) and np.allclose(sig[1], 8 / 7, atol=1e-14)


def test_shift_per_token_changes_nothing():
    # logits on a 2^-10 grid and integer shifts: the shifted float32 values are exact
    lg = (np.round(_rand(2, 20, 9, 1) * 1024) / 1024).astype(np.float32)
    shift = np.random.default_rng(2).integers(-20, 20, size=(2, 20, 1)).astype(np.float32)
    offs = np.array([0, 7, 20], dtype=np.int32)
    assert np.allclose(O.prob_signature(lg + shift, offs), O.prob_signature(lg, offs), rtol=1e-12, atol=1e-12)


def test_two_experts_is_logistic():
    lg = _rand(1, 6, 2, 3)
    sig = O.prob_signature(lg, np.arange(7, dtype=np.int32))        # one token per request
    d = lg[0, :, 0].astype(np.float64) - lg[0, :, 1].astype(np.float64)
    want = np.array([1.0 / (1.0 + math.exp(-v)) for v in d])
    assert np.allclose(sig[:, 0, 0], want, rtol=1e-14) and np.allclose(sig[:, 0, 1], 1 - want, rtol=1e-13)


def test_split_request_adds_up():
    lg = _rand(2, 30, 11, 4)
    whole = O.prob_signature(lg, np.array([3, 27], dtype=np.int32))
    parts = O.prob_signature(lg, np.array([3, 10, 18, 27], dtype=np.int32))
    assert np.allclose(parts.sum(axis=0), whole[0], rtol=1e-13, atol=1e-13)


def test_minus_inf_and_nan_drop_out():
    lg = np.full((1, 3, 4), -np.inf, dtype=np.float32)
    lg[0, 0, 2] = 5.0                                  # one finite logit: probability 1
    lg[0, 1, :] = [np.nan, 1.0, np.nan, 1.0]           # NaN counts as -inf: two equal survivors
    # token 2 is all -inf: contributes nothing
    sig = O.prob_signature(lg, np.array([0, 3], dtype=np.int32))
    assert np.array_equal(sig[0, 0], np.array([0.0, 0.5, 1.0, 0.5]))


def test_out_of_range_offsets_are_clamped():
    lg = _rand(1, 10, 5, 5)
    a = O.prob_signature(lg, np.array([-4, 3, 3, 50], dtype=np.int32))
    b = O.prob_signature(lg, np.array([0, 3, 3, 10], dtype=np.int32))
    assert np.array_equal(a, b)
