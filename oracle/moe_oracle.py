"""CPU oracle for one Mixture-of-Experts layer's expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the test suite, the smoke check of the package entry file and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing) and does
not import it.

Every function is the plain definition of its step, written with numpy in
float64 (library primitives - a stable sort, a matmul, `np.add.at` - serve as
single steps; nothing is blocked, fused or reordered beyond the definition).

Sources (the three pages this work is built from):
  * ELDR page - "ELDR: Expert-Locality-Aware Decode Routing for PD-Disaggregated
    MoE Serving" summary.  Section "What it solves": a decode step reads the
    weights of every distinct expert any token of the batch picked.  Section
    "Core idea / structure / operation": the request signature is the per-expert
    top-k activation count reweighted by IDF, over a subset of layers, recorded
    during prefill; the gate itself is standard top-k gating, unchanged.
  * ExpertPlex page - "ExpertPlex: ... Adaptive Persistent Kernels" summary.
    Section "Instance vs module disaggregation": the expert FFN holds ~95 % of
    the parameters.  Section "Adaptive Persistent Kernels": expert work is cut
    into tiles popped from a queue, decode tiles first at tile boundaries.
  * GRACE-MoE page - "GRACE-MoE: grouping, replication and locality-aware
    routing".  Section 1 (background): every MoE layer dispatches tokens to the
    experts that own them and combines the results back.  Section 3 (key
    observations): experts co-activate under top-k routing.  Section 4 (method):
    profiled per-layer expert selections give an affinity matrix and load
    statistics.

Readings where the pages are silent (each is listed in the design notes):
  R1 gate: the k largest fp32 logits; ties go to the lower expert id; -0.0 and
     +0.0 are equal; NaN ranks as -inf.  Slots are in descending order.
     Weights are the softmax over the k chosen logits (renormalize=1), else the
     full-E softmax probability of each chosen expert (renormalize=0).
  R2 permutation: a stable counting sort of the assignments by group, by flat
     index f; routed f = t*k + j, shared f = T*k + s*T + t.  Routed group
     g = seg(t)*E + e with seg(t) = 1 for t >= n_priority > 0 (else 0); shared
     groups follow all routed ones.
  R3 expert FFN: SwiGLU, h = W_down (silu(W_gate x) * (W_up x)), weights in the
     [out][in] layout, no biases.  Shared experts are always on with weight 1.
  R4 statistics: M[t][e] = number of slots of token t that picked e (0/1 for a
     gate output); counts = column sums; union = experts with a nonzero count;
     affinity = M^T M; per-request counts over token ranges; idf = ln(R/df)
     (0 where df = 0); signature = request count * idf.
  R5 router (in front of the gate): logits = x . W_r^T, a bias-free linear map
     of the hidden state, W_r [E][d].
  R7 FP8 expert weights: OCP E4M3 codes with one fp32 scale per weight row
     (per output feature); the FFN is then the same definition.
  R6 continuous signature (the alternative the ELDR page compares against):
     per request, layer and expert, the sum of the tokens' full-E softmax
     probabilities, no IDF.

Parity pins: see tests/test_oracle_*.py - every function here is checked against
closed forms, library routines, invariants and brute force, not against itself.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


# --------------------------------------------------------------------------
# value conversion (exact)
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their raw 16-bit patterns."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an input array stored as 'f32' or 'bf16' bits."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 to bfloat16 (via float32, both round-to-nearest-even)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    out[nan] = 0x7FC0
    return out


# --------------------------------------------------------------------------
# step 0: router projection (in front of the gate)
# --------------------------------------------------------------------------
def router(x: np.ndarray, w_router: np.ndarray, dtype: str) -> np.ndarray:
    """Router scores logits[t][e] = sum_i x[t][i] * w_router[e][i], in float64.

    ELDR page, "Core idea / structure / operation": the gate is standard top-k
    gating over per-expert router scores of each token.  The pages do not spell
    the router out; reading R5 takes it as a bias-free linear map of the hidden
    state, weights [E][d] in the [out][in] layout.  `x` and `w_router` hold
    bf16 bit patterns (dtype "bf16") or float32 values ("f32").
    """
    return to_f64(x, dtype) @ to_f64(w_router, dtype).T


# --------------------------------------------------------------------------
# step 1: softmax top-k gate
# --------------------------------------------------------------------------
def gate(logits: np.ndarray, k: int, renormalize: bool = True):
    """Top-k gating over fp32 router logits.

    ELDR page, "Core idea / structure / operation": the method leaves the gate as
    standard top-k gating; GRACE-MoE page, section 3: each token activates its
    top-k experts.  Reading R1 fixes order, ties, NaN and the weights.

    Returns (ids int32 [T][k], weights float32 [T][k]).
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    key = lg.astype(np.float64)
    key = np.where(np.isnan(key), -np.inf, key)       # NaN ranks as -inf
    # a stable sort on the negated value: larger logit first, equal logits
    # (including -0.0 == +0.0) keep the lower expert id first
    order = np.argsort(-key, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(key, order[:, :k], axis=1)
    with np.errstate(invalid="ignore"):           # rows of only -inf/NaN give NaN weights
        if renormalize:
            z = np.exp(chosen - chosen[:, :1])
            w = z / z.sum(axis=1, keepdims=True)
        else:
            m = key.max(axis=1, keepdims=True)
            w = np.exp(chosen - m) / np.exp(key - m).sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


# --------------------------------------------------------------------------
# step 2: dispatch as a permutation into per-expert groups
# --------------------------------------------------------------------------
def assignment_groups(topk_ids: np.ndarray, E: int, n_shared: int = 0,
                      n_priority: int = 0):
    """Group and token of every assignment, in flat-index order (reading R2).

    GRACE-MoE page, section 1: a MoE layer sends each token to the experts in
    charge of it; on one GPU that send is a regrouping of the token rows.
    Returns (group [N], token [N], G, nseg).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    nseg = 2 if n_priority > 0 else 1
    tok = np.repeat(np.arange(T), k)
    seg = np.where((n_priority > 0) & (tok >= n_priority), 1, 0)
    g_routed = seg * E + ids.reshape(-1)
    g_shared = nseg * E + np.repeat(np.arange(n_shared), T)
    t_shared = np.tile(np.arange(T), n_shared)
    group = np.concatenate([g_routed, g_shared]).astype(np.int64)
    token = np.concatenate([tok, t_shared]).astype(np.int64)
    return group, token, nseg * E + n_shared, nseg


def permute(topk_ids: np.ndarray, E: int, n_shared: int = 0, n_priority: int = 0,
            x: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Counting sort of the assignments into contiguous expert groups.

    Sort key (group, flat index); group_offsets is the exclusive scan of the
    group sizes; sorted_token[n] is the token that assignment sorted_to_flat[n]
    belongs to, and x_sorted[n] a bit copy of that token's hidden row.
    """
    group, token, G, _ = assignment_groups(topk_ids, E, n_shared, n_priority)
    N = group.shape[0]
    s2f = np.argsort(group, kind="stable")         # stable: ties keep flat order
    f2s = np.empty(N, dtype=np.int64)
    f2s[s2f] = np.arange(N)
    sizes = np.bincount(group, minlength=G)
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    out = {"group_offsets": offsets.astype(np.int32),
           "sorted_to_flat": s2f.astype(np.int32),
           "flat_to_sorted": f2s.astype(np.int32),
           "sorted_token": token[s2f].astype(np.int32)}
    if x is not None:
        out["x_sorted"] = np.ascontiguousarray(np.asarray(x)[token[s2f]])
    return out


def expert_of_group(g: np.ndarray, E: int, n_shared: int, nseg: int) -> np.ndarray:
    """Routed group g = seg*E + e maps to e; shared group nseg*E + s to E + s."""
    g = np.asarray(g, dtype=np.int64)
    return np.where(g < nseg * E, g % E, E + (g - nseg * E))


# --------------------------------------------------------------------------
# step 3: grouped SwiGLU expert FFN
# --------------------------------------------------------------------------
def silu_product(gate_pre: np.ndarray, up_pre: np.ndarray) -> np.ndarray:
    """silu(g) * u with silu(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return up_pre * gate_pre / (1.0 + np.exp(-gate_pre))


def grouped_ffn(x_sorted: np.ndarray, group_offsets: np.ndarray, E: int, n_shared: int,
                nseg: int, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
                dtype: str, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """h[n] = W_down[e] (silu(W_gate[e] xs[n]) * (W_up[e] xs[n])) in float64.

    ExpertPlex page, "Instance vs module disaggregation": the expert FFN is the
    bulk of the layer; reading R3 fixes its form.  Inputs are taken at their
    exact stored values; nothing is rounded in between.  `rows` selects sorted
    rows to compute (default: all); the result has one row per selected row.
    """
    offs = np.asarray(group_offsets, dtype=np.int64)
    N = int(offs[-1])
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = np.searchsorted(offs, sel, side="right") - 1
    exp_of_row = expert_of_group(grp, E, n_shared, nseg)
    d = w_gate.shape[2]
    h = np.zeros((sel.shape[0], d), dtype=np.float64)
    for e in np.unique(exp_of_row):
        pick = np.nonzero(exp_of_row == e)[0]
        xs = to_f64(np.asarray(x_sorted)[sel[pick]], dtype)
        wg = to_f64(w_gate[e], dtype)
        wu = to_f64(w_up[e], dtype)
        wd = to_f64(w_down[e], dtype)
        a = silu_product(xs @ wg.T, xs @ wu.T)
        h[pick] = a @ wd.T
    return h


def fp8_e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    ex = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ex.astype(np.float64) - 7.0))
    return np.where((ex == 15) & (m == 7), np.nan, sign * mag)


def grouped_ffn_fp8w(x_sorted: np.ndarray, group_offsets: np.ndarray, E: int, n_shared: int, nseg: int,
                     wq_gate: np.ndarray, s_gate: np.ndarray, wq_up: np.ndarray, s_up: np.ndarray,
                     wq_down: np.ndarray, s_down: np.ndarray, dtype: str = "bf16",
                     rows: Optional[np.ndarray] = None) -> np.ndarray:
    """The expert FFN with FP8 E4M3 weights and one fp32 scale per weight row:
    W[e][r][:] = fp8(wq[e][r][:]) * s[e][r], then exactly `grouped_ffn`'s
    definition in float64.  ExpertPlex page, "Experimental results" (the
    models table): one of the two evaluated models, GLM-5.1-FP8, is an
    FP8-quantised MoE served in that form; the page does not give the format,
    and reading R7 takes OCP E4M3 codes with one scale per weight row."""
    offs = np.asarray(group_offsets, dtype=np.int64)
    N = int(offs[-1])
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = np.searchsorted(offs, sel, side="right") - 1
    exp_of_row = expert_of_group(grp, E, n_shared, nseg)
    d = wq_gate.shape[2]
    h = np.zeros((sel.shape[0], d), dtype=np.float64)
    for e in np.unique(exp_of_row):
        pick = np.nonzero(exp_of_row == e)[0]
        xs = to_f64(np.asarray(x_sorted)[sel[pick]], dtype)
        wg = fp8_e4m3_to_f64(wq_gate[e]) * np.asarray(s_gate[e], dtype=np.float64)[:, None]
        wu = fp8_e4m3_to_f64(wq_up[e]) * np.asarray(s_up[e], dtype=np.float64)[:, None]
        wd = fp8_e4m3_to_f64(wq_down[e]) * np.asarray(s_down[e], dtype=np.float64)[:, None]
        a = silu_product(xs @ wg.T, xs @ wu.T)
        h[pick] = a @ wd.T
    return h


# --------------------------------------------------------------------------
# step 4: combine back to token order
# --------------------------------------------------------------------------
def combine(h_sorted: np.ndarray, flat_to_sorted: np.ndarray, topk_w: np.ndarray,
            T: int, k: int, n_shared: int, tokens: Optional[np.ndarray] = None,
            row_of_sorted=None) -> np.ndarray:
    """y[t] = sum_j w[t][j] h[f2s[t*k+j]] + sum_s h[f2s[T*k+s*T+t]] in float64.

    GRACE-MoE page, section 1: the second exchange of a MoE layer gathers the
    expert outputs back to their tokens; the router weights scale the routed
    experts, shared experts enter with weight 1 (reading R3).  `h_sorted` is a
    float64 array indexed by sorted row (or, with `row_of_sorted`, a mapping from
    sorted row to a row of `h_sorted`).
    """
    f2s = np.asarray(flat_to_sorted, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    d = h_sorted.shape[1]
    y = np.zeros((toks.shape[0], d), dtype=np.float64)

    def row(n):
        return h_sorted[n if row_of_sorted is None else row_of_sorted[n]]

    for i, t in enumerate(toks):
        acc = np.zeros(d, dtype=np.float64)
        for j in range(k):
            acc += w[t, j] * row(f2s[t * k + j])
        for s in range(n_shared):
            acc += row(f2s[T * k + s * T + t])
        y[i] = acc
    return y


# --------------------------------------------------------------------------
# step 5: expert-activation statistics
# --------------------------------------------------------------------------
def stats(topk_ids: np.ndarray, E: int, req_offsets: Optional[np.ndarray] = None,
          idf: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Per-layer counts, union, affinity; per-request counts, idf, signature.

    ELDR page, "What it solves": a decode step reads every distinct expert of
    the batch (the union).  ELDR page, "Core idea / structure / operation": the
    signature is the top-k activation count per expert reweighted by IDF, over a
    layer subset.  GRACE-MoE page, section 3 and section 4: co-activation of
    experts and per-expert load come from recorded top-k selections.
    `topk_ids` is [L][T][k] (routed ids only).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    L, T, k = ids.shape
    counts = np.zeros((L, E), dtype=np.int64)
    affinity = np.zeros((L, E, E), dtype=np.int64)
    for l in range(L):
        np.add.at(counts[l], ids[l].reshape(-1), 1)
        # every ordered pair of slots (j1, j2) of a token, j1 == j2 included
        np.add.at(affinity[l], (ids[l][:, :, None], ids[l][:, None, :]), 1)
    union_mask = (counts > 0).astype(np.uint8)
    out = {"counts": counts.astype(np.int32),
           "union_mask": union_mask,
           "union_size": union_mask.sum(axis=1).astype(np.int32),
           "affinity": affinity.astype(np.int32)}
    if req_offsets is None:
        return out
    offs = np.asarray(req_offsets, dtype=np.int64)
    R = offs.shape[0] - 1
    req = np.zeros((R, L, E), dtype=np.int64)
    for r in range(R):
        lo, hi = max(0, offs[r]), min(T, offs[r + 1])
        for l in range(L):
            if hi > lo:
                np.add.at(req[r, l], ids[l, lo:hi].reshape(-1), 1)
    df = (req > 0).sum(axis=0)                        # [L][E] documents per term
    if idf is None:
        with np.errstate(divide="ignore"):
            idf64 = np.where(df > 0, np.log(float(R) / np.maximum(df, 1)), 0.0)
    else:
        idf64 = np.asarray(idf, dtype=np.float32).astype(np.float64)
    sig = (req.astype(np.float64) * idf64[None, :, :]).astype(np.float32)
    out.update({"req_counts": req.astype(np.int32), "df": df.astype(np.int32),
                "idf": idf64, "signature": sig})
    return out


def prob_signature(logits: np.ndarray, req_offsets: np.ndarray) -> np.ndarray:
    """Continuous request signature [R][L][E]: for each request, layer and
    expert, the sum over the request's tokens of the full-E softmax probability.

    ELDR page, "Core idea / structure / operation": the paper compares its
    count x IDF signature against continuous alternatives such as the softmax
    gate probability.  Reading R6 takes that alternative as the plain
    per-request sum of each token's softmax over all E experts, without IDF;
    NaN logits count as -inf, a token whose logits are all -inf adds nothing,
    and requests own token ranges as in `stats` (clamped to [0, T]).
    `logits` is [L][T][E] float32.
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    L, T, E = lg.shape
    m = lg.max(axis=2, keepdims=True)
    live = m > -np.inf                                   # tokens with a finite logit
    ex = np.where(live, np.exp(lg - np.where(live, m, 0.0)), 0.0)
    den = ex.sum(axis=2, keepdims=True)
    p = np.where(live, ex / np.where(live, den, 1.0), 0.0)
    offs = np.asarray(req_offsets, dtype=np.int64)
    R = offs.shape[0] - 1
    out = np.zeros((R, L, E), dtype=np.float64)
    for r in range(R):
        lo = min(max(offs[r], 0), T)
        hi = min(max(offs[r + 1], lo), T)
        out[r] = p[:, lo:hi, :].sum(axis=1)
    return out


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------
def moe_layer(logits, x, w_gate, w_up, w_down, k, dtype, n_shared=0, n_priority=0,
              renormalize=True, tokens=None) -> Dict[str, np.ndarray]:
    """gate -> permute -> grouped FFN -> combine for the selected tokens (float64 y).

    Only the sorted rows the selected tokens need go through the FFN, so a
    sample of tokens of a large batch stays cheap.
    """
    T, E = np.asarray(logits).shape
    ids, w = gate(logits, k, renormalize)
    p = permute(ids, E, n_shared, n_priority, x)
    nseg = 2 if n_priority > 0 else 1
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    f2s = p["flat_to_sorted"].astype(np.int64)
    flat = [t * k + j for t in toks for j in range(k)]
    flat += [T * k + s * T + t for t in toks for s in range(n_shared)]
    need = np.unique(f2s[np.asarray(flat, dtype=np.int64)])
    h = grouped_ffn(p["x_sorted"], p["group_offsets"], E, n_shared, nseg,
                    w_gate, w_up, w_down, dtype, rows=need)
    where = {int(n): i for i, n in enumerate(need)}
    y = combine(h, f2s, w, T, k, n_shared, tokens=toks, row_of_sorted=where)
    return {"ids": ids, "w": w, "perm": p, "h_rows": need, "h": h, "y": y}
