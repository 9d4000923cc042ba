"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Each mutant replaces one oracle function with a version carrying a typical bug
(a dropped term, a wrong sign or index, a transposed operand, a lost tie rule);
at least one of the listed pin tests must then fail.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_gate as TG
import tests.test_oracle_permute as TP
import tests.test_oracle_ffn_combine as TF
import tests.test_oracle_stats as TS
import tests.test_oracle_router as TR
import tests.test_oracle_prob_signature as TQ
import tests.test_oracle_fp8 as T8

_orig = {name: getattr(O, name) for name in ("gate", "permute", "grouped_ffn", "combine", "stats",
                                              "silu_product", "assignment_groups", "router",
                                              "prob_signature", "fp8_e4m3_to_f64", "grouped_ffn_fp8w")}


def _gate_unstable(logits, k, renormalize=True):
    lg = np.asarray(logits, dtype=np.float32)
    key = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    # ties resolved towards the higher id
    order = np.array([sorted(range(lg.shape[1]), key=lambda e: (-row[e], -e)) for row in key])
    ids = order[:, :k].astype(np.int32)
    return ids, _orig["gate"](logits, k, renormalize)[1]


def _gate_nan_high(logits, k, renormalize=True):
    lg = np.asarray(logits, dtype=np.float32).copy()
    lg[np.isnan(lg)] = np.inf
    return _orig["gate"](lg, k, renormalize)


def _gate_no_renorm(logits, k, renormalize=True):
    return _orig["gate"](logits, k, False)


def _permute_unstable(topk_ids, E, n_shared=0, n_priority=0, x=None):
    p = _orig["permute"](topk_ids, E, n_shared, n_priority, x)
    offs = p["group_offsets"]
    s2f = p["sorted_to_flat"].copy()
    for g in range(len(offs) - 1):                  # reverse inside each group
        s2f[offs[g]:offs[g + 1]] = s2f[offs[g]:offs[g + 1]][::-1]
    f2s = np.empty_like(s2f)
    f2s[s2f] = np.arange(len(s2f))
    p.update(sorted_to_flat=s2f, flat_to_sorted=f2s)
    if x is not None:
        T, k = np.asarray(topk_ids).shape
        tok = np.where(s2f < T * k, s2f // k, (s2f - T * k) % T)
        p["x_sorted"] = np.asarray(x)[tok]
    return p


def _assign_shared_wrong(topk_ids, E, n_shared=0, n_priority=0):
    g, t, G, nseg = _orig["assignment_groups"](topk_ids, E, n_shared, n_priority)
    T, k = np.asarray(topk_ids).shape
    t = t.copy()
    t[T * k:] = t[T * k:][::-1]                     # shared rows of the wrong tokens
    return g, t, G, nseg


def _silu_wrong_sign(g, u):
    return u * g / (1.0 + np.exp(g))


def _silu_drops_gate(g, u):
    return u / (1.0 + np.exp(-g))


def _ffn_transposed_down(x_sorted, group_offsets, E, n_shared, nseg, w_gate, w_up, w_down,
                         dtype, rows=None):
    wd = np.ascontiguousarray(np.swapaxes(w_down, 1, 2)[:, :, :]) if w_down.shape[1] == w_down.shape[2] \
        else w_down[:, ::-1, :]
    return _orig["grouped_ffn"](x_sorted, group_offsets, E, n_shared, nseg, w_gate, w_up, wd, dtype, rows)


def _ffn_gate_up_swapped(x_sorted, group_offsets, E, n_shared, nseg, w_gate, w_up, w_down,
                         dtype, rows=None):
    return _orig["grouped_ffn"](x_sorted, group_offsets, E, n_shared, nseg, w_up, w_gate, w_down, dtype, rows)


def _combine_no_shared(h_sorted, flat_to_sorted, topk_w, T, k, n_shared, tokens=None, row_of_sorted=None):
    return _orig["combine"](h_sorted, flat_to_sorted, topk_w, T, k, 0, tokens, row_of_sorted)


def _combine_weight_index(h_sorted, flat_to_sorted, topk_w, T, k, n_shared, tokens=None, row_of_sorted=None):
    return _orig["combine"](h_sorted, flat_to_sorted, np.asarray(topk_w)[:, ::-1], T, k, n_shared,
                            tokens, row_of_sorted)


def _stats_no_diag(topk_ids, E, req_offsets=None, idf=None):
    st = _orig["stats"](topk_ids, E, req_offsets, idf)
    for l in range(st["affinity"].shape[0]):
        np.fill_diagonal(st["affinity"][l], 0)
    return st


def _stats_idf_inverted(topk_ids, E, req_offsets=None, idf=None):
    st = _orig["stats"](topk_ids, E, req_offsets, idf)
    if req_offsets is not None and idf is None:
        R = len(req_offsets) - 1
        df = st["df"].astype(np.float64)
        st["idf"] = np.where(df > 0, np.log(np.maximum(df, 1) / R), 0.0)
        st["signature"] = (st["req_counts"] * st["idf"][None]).astype(np.float32)
    return st


def _stats_union_off_by_one(topk_ids, E, req_offsets=None, idf=None):
    st = _orig["stats"](topk_ids, E, req_offsets, idf)
    st["union_mask"] = (st["counts"] > 1).astype(np.uint8)
    st["union_size"] = st["union_mask"].sum(axis=1).astype(np.int32)
    return st


def _router_transposed(x, w_router, dtype):
    # W_r read as [d][E]: the hidden index runs over W_r's rows
    w = O.to_f64(w_router, dtype)
    return O.to_f64(x, dtype) @ np.resize(w.T, w.shape)


def _router_drops_last_term(x, w_router, dtype):
    return O.to_f64(x, dtype)[:, :-1] @ O.to_f64(w_router, dtype)[:, :-1].T


def _prob_sig_over_tokens(logits, req_offsets):
    # softmax taken across the tokens of the batch instead of across the experts
    lg = np.asarray(logits, dtype=np.float64)
    offs = np.asarray(req_offsets, dtype=np.int64)
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return np.stack([p[:, max(0, offs[r]):min(lg.shape[1], offs[r + 1])].sum(axis=1) for r in range(len(offs) - 1)])


def _prob_sig_unnormalised(logits, req_offsets):
    lg = np.asarray(logits, dtype=np.float64)
    offs = np.asarray(req_offsets, dtype=np.int64)
    ex = np.exp(lg - lg.max(axis=2, keepdims=True))
    return np.stack([ex[:, max(0, offs[r]):min(lg.shape[1], offs[r + 1])].sum(axis=1) for r in range(len(offs) - 1)])


def _fp8_subnormals_as_normals(bits):
    # exponent field 0 read like the others: 2^-6 * (1 + m/8) instead of 2^-6 * m/8
    b = np.asarray(bits, dtype=np.uint8)
    v = _orig["fp8_e4m3_to_f64"](b)
    sub = ((b >> 3) & 0xF) == 0
    m = (b & 7).astype(np.float64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    return np.where(sub & (m > 0), sign * 2.0 ** -6 * (1 + m / 8), v)


def _fp8w_up_takes_gate_scale(x_sorted, group_offsets, E, n_shared, nseg, wq_gate, s_gate, wq_up, s_up,
                              wq_down, s_down, dtype="bf16", rows=None):
    return _orig["grouped_ffn_fp8w"](x_sorted, group_offsets, E, n_shared, nseg, wq_gate, s_gate, wq_up, s_gate,
                                     wq_down, s_down, dtype, rows)


def _fp8w_drops_down_scale(x_sorted, group_offsets, E, n_shared, nseg, wq_gate, s_gate, wq_up, s_up,
                           wq_down, s_down, dtype="bf16", rows=None):
    return _orig["grouped_ffn_fp8w"](x_sorted, group_offsets, E, n_shared, nseg, wq_gate, s_gate, wq_up, s_up,
                                     wq_down, np.ones_like(s_down), dtype, rows)


def _run_pins(pins):
    failures = 0
    for fn, args in pins:
        try:
            fn(*args)
        except AssertionError:
            failures += 1
        except Exception:           # a crash is a detection too
            failures += 1
    return failures


def _gate_cases():
    return [(TG.test_gate_golden, (c,)) for c in TG._golden_cases()] + [(TG.test_gate_bruteforce_tiny_E, ())]


_router_pins = lambda: [(TR.test_router_unit_rows_select_weight_columns, ()),
                        (TR.test_router_hand_computed_case, ())]

_prob_pins = lambda: [(TQ.test_each_token_adds_probability_one, ()), (TQ.test_equal_logits_give_one_over_E, ())]

_fp8_pins = lambda: [(T8.test_fp8_ffn_equals_fp32_ffn_on_exact_weights, ()),
                     (T8.test_fp8_ffn_scale_is_per_output_row, ())]

MUTANTS = {
    "fp8_subnormals_as_normals": ("fp8_e4m3_to_f64", _fp8_subnormals_as_normals,
                                  lambda: [(T8.test_all_codes_match_torch_float8_e4m3fn, ()),
                                           (T8.test_landmark_codes, ())]),
    "fp8_up_takes_gate_scale": ("grouped_ffn_fp8w", _fp8w_up_takes_gate_scale, _fp8_pins),
    "fp8_drops_down_scale": ("grouped_ffn_fp8w", _fp8w_drops_down_scale, _fp8_pins),
    "prob_signature_wrong_axis": ("prob_signature", _prob_sig_over_tokens, _prob_pins),
    "prob_signature_unnormalised": ("prob_signature", _prob_sig_unnormalised, _prob_pins),
    "router_weights_transposed": ("router", _router_transposed, _router_pins),
    "router_drops_last_hidden_term": ("router", _router_drops_last_term, _router_pins),
    "gate_ties_to_higher_id": ("gate", _gate_unstable, _gate_cases),
    "gate_nan_as_plus_inf": ("gate", _gate_nan_high, _gate_cases),
    "gate_skips_renormalisation": ("gate", _gate_no_renorm,
                                   lambda: [(TG.test_gate_weights_sum_to_one_and_k1_is_exactly_one, ())]),
    "permute_unstable_within_group": ("permute", _permute_unstable,
                                      lambda: [(TP.test_permute_golden, (c,)) for c in TP._cases()]),
    "permute_shared_rows_wrong_token": ("assignment_groups", _assign_shared_wrong,
                                        lambda: [(TP.test_permute_invariants, (s,)) for s in range(2)]),
    "silu_wrong_sign": ("silu_product", _silu_wrong_sign,
                        lambda: [(TF.test_ffn_golden, (c,)) for c in TF._golden()["ffn_cases"]]),
    "silu_drops_gate_factor": ("silu_product", _silu_drops_gate,
                               lambda: [(TF.test_ffn_single_expert_is_dense_swiglu, ())]),
    "ffn_down_misindexed": ("grouped_ffn", _ffn_transposed_down,
                            lambda: [(TF.test_ffn_single_expert_is_dense_swiglu, ())]),
    "ffn_gate_up_swapped": ("grouped_ffn", _ffn_gate_up_swapped,
                            lambda: [(TF.test_ffn_golden, (c,)) for c in TF._golden()["ffn_cases"]]),
    "combine_drops_shared": ("combine", _combine_no_shared,
                             lambda: [(TF.test_combine_golden, (c,)) for c in TF._golden()["combine_cases"]]),
    "combine_weight_slots_reversed": ("combine", _combine_weight_index,
                                      lambda: [(TF.test_combine_golden, (c,)) for c in TF._golden()["combine_cases"]]),
    "affinity_without_diagonal": ("stats", _stats_no_diag,
                                  lambda: [(TS.test_stats_golden, (c,)) for c in TS._cases()]),
    "idf_inverted": ("stats", _stats_idf_inverted,
                     lambda: [(TS.test_stats_golden, (c,)) for c in TS._cases()]),
    "union_needs_two_hits": ("stats", _stats_union_off_by_one,
                             lambda: [(TS.test_stats_golden, (c,)) for c in TS._cases()]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, mutant, pins = MUTANTS[name]
    monkeypatch.setattr(O, attr, mutant)
    assert _run_pins(pins()) > 0, f"no pin caught mutant {name}"


def test_pins_pass_on_unmutated_oracle():
    for name in sorted(MUTANTS):
        assert _run_pins(MUTANTS[name][2]()) == 0, name
