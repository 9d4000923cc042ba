"""Pins for the oracle's grouped SwiGLU FFN and combine.

FFN: ExpertPlex page, "Instance vs module disaggregation" (the expert FFN holds
the bulk of a MoE layer); SwiGLU form h = W_down(silu(W_gate x) * W_up x).
Combine: GRACE-MoE page, section 1 (results are gathered back to the tokens).
Checked against hand values, torch.nn.functional in float64 (a library routine
independent of the oracle's formula) and closed-form special cases.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "ffn_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["ffn_cases"], ids=lambda c: c["name"])
def test_ffn_golden(case):
    x = np.array(case["x"], dtype=np.float32)
    wg = np.array(case["w_gate"], dtype=np.float32)
    wu = np.array(case["w_up"], dtype=np.float32)
    wd = np.array(case["w_down"], dtype=np.float32)
    offs = np.array([0, x.shape[0]], dtype=np.int32)
    h = O.grouped_ffn(x, offs, 1, 0, 1, wg, wu, wd, "f32")
    np.testing.assert_allclose(h, np.array(case["h"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", _golden()["combine_cases"], ids=lambda c: c["name"])
def test_combine_golden(case):
    y = O.combine(np.array(case["h_sorted"]), np.array(case["flat_to_sorted"]),
                  np.array(case["topk_w"], dtype=np.float32), case["T"], case["k"],
                  case["n_shared"])
    np.testing.assert_array_equal(y, np.array(case["y"]))


def _torch_swiglu(x, wg, wu, wd):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, wg, wu, wd))
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd).numpy()


def _bf16_bits(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_ffn_single_expert_is_dense_swiglu():
    """E = 1, k = 1, no shared experts: the grouped FFN is one dense SwiGLU MLP."""
    rng = np.random.default_rng(0)
    T, d, I = 37, 48, 80
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((1, I, d)) / 7).astype(np.float32)
    wu = (rng.standard_normal((1, I, d)) / 7).astype(np.float32)
    wd = (rng.standard_normal((1, d, I)) / 9).astype(np.float32)
    p = O.permute(np.zeros((T, 1), dtype=np.int32), 1, 0, 0, x)
    h = O.grouped_ffn(p["x_sorted"], p["group_offsets"], 1, 0, 1, wg, wu, wd, "f32")
    np.testing.assert_allclose(h, _torch_swiglu(x, wg[0], wu[0], wd[0]), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ffn_groups_are_per_expert_dense_mlps(dtype):
    rng = np.random.default_rng(1)
    T, E, k, S, P, d, I = 29, 6, 2, 1, 7, 32, 24
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    x32 = rng.standard_normal((T, d)).astype(np.float32)
    wg32 = (rng.standard_normal((E + S, I, d)) / 5).astype(np.float32)
    wu32 = (rng.standard_normal((E + S, I, d)) / 5).astype(np.float32)
    wd32 = (rng.standard_normal((E + S, d, I)) / 5).astype(np.float32)
    if dtype == "bf16":
        x, wg, wu, wd = (_bf16_bits(a) for a in (x32, wg32, wu32, wd32))
    else:
        x, wg, wu, wd = x32, wg32, wu32, wd32
    p = O.permute(ids, E, S, P, x)
    h = O.grouped_ffn(p["x_sorted"], p["group_offsets"], E, S, 2, wg, wu, wd, dtype)
    xe = O.to_f64(x, dtype)
    group, token, G, nseg = O.assignment_groups(ids, E, S, P)
    s2f = p["sorted_to_flat"].astype(np.int64)
    for n in range(h.shape[0]):
        f = s2f[n]
        e = ids.reshape(-1)[f] if f < T * k else E + (f - T * k) // T
        ref = _torch_swiglu(xe[token[f]][None, :], O.to_f64(wg[e], dtype),
                            O.to_f64(wu[e], dtype), O.to_f64(wd[e], dtype))[0]
        np.testing.assert_allclose(h[n], ref, rtol=1e-12, atol=1e-12)


def test_ffn_rows_subset_matches_full():
    rng = np.random.default_rng(2)
    T, E, k, d, I = 40, 5, 2, 16, 8
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg, wu = (rng.standard_normal((E, I, d)).astype(np.float32) for _ in range(2))
    wd = rng.standard_normal((E, d, I)).astype(np.float32)
    p = O.permute(ids, E, 0, 0, x)
    full = O.grouped_ffn(p["x_sorted"], p["group_offsets"], E, 0, 1, wg, wu, wd, "f32")
    rows = np.array([79, 0, 33, 5])
    sub = O.grouped_ffn(p["x_sorted"], p["group_offsets"], E, 0, 1, wg, wu, wd, "f32", rows=rows)
    # BLAS blocking depends on the row count: equal up to float64 rounding
    np.testing.assert_allclose(sub, full[rows], rtol=1e-12, atol=1e-12)


def test_ffn_zero_cases():
    rng = np.random.default_rng(3)
    d, I = 8, 12
    x = rng.standard_normal((5, d)).astype(np.float32)
    wg = rng.standard_normal((1, I, d)).astype(np.float32)
    wd = rng.standard_normal((1, d, I)).astype(np.float32)
    offs = np.array([0, 5], dtype=np.int32)
    assert (O.grouped_ffn(x, offs, 1, 0, 1, wg, np.zeros_like(wg), wd, "f32") == 0).all()
    assert (O.grouped_ffn(np.zeros_like(x), offs, 1, 0, 1, wg, wg, wd, "f32") == 0).all()


def test_two_shared_experts_equal_one_concatenated():
    """Two always-on experts of width I sum to one SwiGLU of width 2I (concatenated)."""
    rng = np.random.default_rng(4)
    T, d, I = 9, 16, 12
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg, wu = (rng.standard_normal((2, I, d)).astype(np.float32) for _ in range(2))
    wd = rng.standard_normal((2, d, I)).astype(np.float32)
    ids = np.zeros((T, 1), dtype=np.int32)
    wg3 = np.concatenate([np.zeros((1, I, d), np.float32), wg])
    wu3 = np.concatenate([np.zeros((1, I, d), np.float32), wu])
    wd3 = np.concatenate([np.zeros((1, d, I), np.float32), wd])
    p = O.permute(ids, 1, 2, 0, x)
    h = O.grouped_ffn(p["x_sorted"], p["group_offsets"], 1, 2, 1, wg3, wu3, wd3, "f32")
    y = O.combine(h, p["flat_to_sorted"], np.zeros((T, 1), np.float32), T, 1, 2)
    ref = _torch_swiglu(x, np.concatenate(wg), np.concatenate(wu), np.concatenate(wd, axis=1))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_combine_identity_experts_k1_returns_input():
    """k = 1 with identity experts (h_sorted := x_sorted) returns x exactly."""
    rng = np.random.default_rng(5)
    T, E = 64, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, 24)).astype(np.float32)
    ids, w = O.gate(lg, 1)
    p = O.permute(ids, E, 0, 0, x)
    y = O.combine(p["x_sorted"].astype(np.float64), p["flat_to_sorted"], w, T, 1, 0)
    assert np.array_equal(y.astype(np.float32).view(np.uint32), x.view(np.uint32))


def test_combine_identity_experts_renormalized_sum():
    rng = np.random.default_rng(6)
    T, E, k = 64, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, 24)).astype(np.float32)
    ids, w = O.gate(lg, k)
    p = O.permute(ids, E, 0, 0, x)
    y = O.combine(p["x_sorted"].astype(np.float64), p["flat_to_sorted"], w, T, k, 0)
    np.testing.assert_allclose(y, x.astype(np.float64), rtol=1e-6, atol=1e-6)


def test_combine_equals_scatter_matmul():
    """y = P h with P[t, f2s[t*k+j]] = w[t][j] and ones for shared rows (numpy matmul)."""
    rng = np.random.default_rng(7)
    T, E, k, S, d = 33, 7, 3, 2, 10
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    p = O.permute(ids, E, S, 0)
    N = T * (k + S)
    h = rng.standard_normal((N, d))
    Pm = np.zeros((T, N))
    f2s = p["flat_to_sorted"]
    for t in range(T):
        for j in range(k):
            Pm[t, f2s[t * k + j]] += w[t, j]
        for s in range(S):
            Pm[t, f2s[T * k + s * T + t]] += 1.0
    y = O.combine(h, f2s, w, T, k, S)
    np.testing.assert_allclose(y, Pm @ h, rtol=1e-13, atol=1e-13)


def test_bf16_conversions_match_torch():
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        [0.0, -0.0, 1.0, 65504.0, 3.0e38, -1e-40]]).astype(np.float32)
    bits = O.f64_to_bf16_bits(v.astype(np.float64))
    tb = torch.from_numpy(v).to(torch.bfloat16)
    np.testing.assert_array_equal(bits, tb.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), tb.to(torch.float64).numpy())
