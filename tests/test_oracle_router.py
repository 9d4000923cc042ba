"""Pins of the oracle's router projection (CPU only).

The router is the step in front of the gate (ELDR page, "Core idea / structure
/ operation": top-k gating over per-expert router scores), read as
logits = x . W_r^T.  The pins check it against what the definition fixes
without re-typing it: unit token rows pick out columns of W_r, small integer
inputs give exact integer results that also obey linearity, permutations of
tokens and experts move rows and columns, and torch's own linear layer agrees
in float64.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def test_router_unit_rows_select_weight_columns():
    rng = np.random.default_rng(0)
    d, E = 24, 5
    w = _f32(rng.normal(size=(E, d)))
    x = np.eye(d, dtype=np.float32)                  # token t is the unit vector e_t
    lg = O.router(x, w, "f32")
    assert lg.shape == (d, E)
    assert np.array_equal(lg, w.T.astype(np.float64))


def test_router_hand_computed_case():
    x = _f32([[1, 2, 0], [3, -1, 2]])
    w = _f32([[1, 0, 0], [0, 1, 1], [2, 2, -1], [0, 0, 0]])
    # row 0: [1, 2, 1*2+2*2, 0] ; row 1: [3, -1+2, 6-2-2, 0]
    assert np.array_equal(O.router(x, w, "f32"), np.array([[1, 2, 6, 0], [3, 1, 2, 0]], dtype=np.float64))


def test_router_linearity_on_integers():
    rng = np.random.default_rng(1)
    d, E, T = 40, 7, 6
    x1 = rng.integers(-8, 9, size=(T, d)).astype(np.float32)
    x2 = rng.integers(-8, 9, size=(T, d)).astype(np.float32)
    w = rng.integers(-8, 9, size=(E, d)).astype(np.float32)
    lhs = O.router(3 * x1 - 2 * x2, w, "f32")        # every value and sum is an exact small integer
    rhs = 3 * O.router(x1, w, "f32") - 2 * O.router(x2, w, "f32")
    assert np.array_equal(lhs, rhs)


def test_router_permutations_move_rows_and_columns():
    rng = np.random.default_rng(2)
    T, d, E = 9, 16, 6
    x = _f32(rng.normal(size=(T, d)))
    w = _f32(rng.normal(size=(E, d)))
    pt, pe = rng.permutation(T), rng.permutation(E)
    base = O.router(x, w, "f32")
    assert np.array_equal(O.router(x[pt], w, "f32"), base[pt])
    assert np.array_equal(O.router(x, w[pe], "f32"), base[:, pe])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_matches_torch_linear_in_float64(dtype):
    rng = np.random.default_rng(3)
    T, d, E = 11, 64, 9
    xf = rng.normal(size=(T, d))
    wf = rng.normal(size=(E, d)) * 0.1
    if dtype == "bf16":
        x, w = O.f64_to_bf16_bits(xf), O.f64_to_bf16_bits(wf)
    else:
        x, w = _f32(xf), _f32(wf)
    ref = torch.nn.functional.linear(torch.from_numpy(O.to_f64(x, dtype)), torch.from_numpy(O.to_f64(w, dtype)))
    assert np.allclose(O.router(x, w, dtype), ref.numpy(), rtol=1e-13, atol=1e-13)
