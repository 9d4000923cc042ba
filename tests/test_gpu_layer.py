"""End-to-end parity of the whole expert path at the five workload shapes.

The GPU runs the layer exactly as the benchmark does (MoeLayer: gate ->
permute -> grouped FFN -> combine, plus statistics).  Integer outputs are
compared with the oracle in full, bit for bit.  The FFN output of every
sorted row and the layer output of every token are compared with the
oracle's float64 values (the GPU buffers are filled with NaN bit patterns
first, so a row that no tile writes fails).  The router and FP8 variants
compare a sample of tokens that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from helpers import GATE_W_ATOL, SIG_RTOL, TOL, announce, f64_of, np_of, rel_max_err, require_gpu

import top_expert_routing_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"

CONFIGS = ["tiny", "olmoe_decode", "olmoe_decode_local", "qwen3_prefill", "dsv2_decode_t16",
           "dsv2_decode_t64", "dsv2_decode_t128", "dsv2_decode_t256", "gptoss_mixed"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _sample_tokens(T, P, n=12):
    picks = {0, T - 1, T // 2}
    if P:
        picks |= {0, P - 1, P, min(T - 1, P + 1)}
    rng = np.random.default_rng(T)
    picks |= set(rng.integers(0, T, size=n).tolist())
    return np.array(sorted(picks))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CONFIGS)
def test_layer_parity(name):
    announce(f"layer {name}")
    wl = workloads.make(name, DEV)
    s = wl.spec
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down,
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize),
                         stats_layers=s.stats_layers, req_offsets=wl.req_offsets, device=DEV)
    for buf in (layer.h_sorted, layer.y):          # NaN bit patterns: rows no tile writes stay NaN
        buf.view(torch.uint8).fill_(0xFF)
    stats_ids = torch.empty((s.stats_layers, s.T, s.k), dtype=torch.int32, device=DEV)
    for l in range(1, s.stats_layers):
        moe.gate(wl.stats_logits[l].contiguous(), s.k, True, stats_ids[l], torch.empty((s.T, s.k), device=DEV))
    layer.forward(wl.logits, wl.x)
    stats_ids[0].copy_(layer.topk_ids)
    layer.stats(stats_ids)
    torch.cuda.synchronize()
    nbytes = moe.ffn_workspace_bytes(s.N, s.E, s.S, layer.nseg, s.d, s.I, wl.torch_dtype)
    assert int(layer.ffn_ws[nbytes - 4:nbytes].view(torch.int32).item()) == 0, "a tile-queue wait gave up"

    logits = np_of(wl.logits)
    ids_ref, w_ref = O.gate(logits, s.k, bool(s.renormalize))
    np.testing.assert_array_equal(np_of(layer.topk_ids), ids_ref)
    assert np.abs(np_of(layer.topk_w).astype(np.float64) - w_ref).max() <= GATE_W_ATOL

    p_ref = O.permute(ids_ref, s.E, s.S, s.n_priority)
    for key in ("group_offsets", "sorted_to_flat", "flat_to_sorted"):
        np.testing.assert_array_equal(np_of(layer.perm[key]), p_ref[key], err_msg=key)
    np.testing.assert_array_equal(np_of(layer.perm["sorted_token"]), p_ref["sorted_token"])

    # statistics over the layer stack, in full
    all_ids = np.stack([ids_ref] + [O.gate(np_of(wl.stats_logits[l]), s.k)[0]
                                    for l in range(1, s.stats_layers)])
    np.testing.assert_array_equal(np_of(stats_ids), all_ids)
    st_ref = O.stats(all_ids, s.E, np_of(wl.req_offsets))
    for key in ("counts", "union_size", "union_mask", "affinity", "req_counts"):
        np.testing.assert_array_equal(np_of(layer.stats_out[key]), st_ref[key], err_msg=key)
    sig, sref = np_of(layer.stats_out["signature"]).astype(np.float64), st_ref["signature"].astype(np.float64)
    assert np.all(np.abs(sig - sref) <= SIG_RTOL * np.abs(sref))

    # every sorted row of the FFN output and every token of the layer output
    x = np_of(wl.x)
    p_x = O.permute(ids_ref, s.E, s.S, s.n_priority, x)
    h_ref = O.grouped_ffn(p_x["x_sorted"], p_x["group_offsets"], s.E, s.S, layer.nseg, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), s.dtype)
    h_gpu = f64_of(layer.h_sorted)
    assert not np.isnan(h_gpu).any(), "sorted rows left unwritten"
    h_err = rel_max_err(h_gpu, h_ref)
    y_ref = O.combine(h_ref, p_x["flat_to_sorted"], w_ref, s.T, s.k, s.S)
    y_gpu = f64_of(layer.y)
    assert not np.isnan(y_gpu).any(), "tokens left unwritten"
    y_err = rel_max_err(y_gpu, y_ref)
    announce(f"layer {name}: h err {h_err:.2e}, y err {y_err:.2e} over all {s.N} rows / {s.T} tokens, "
             f"union {np_of(layer.stats_out['union_size'])}")
    assert h_err <= TOL[s.dtype], h_err
    assert y_err <= TOL[s.dtype], y_err


@pytest.mark.parametrize("name", ["olmoe_decode", "dsv2_decode_t16", "dsv2_decode_t256"])
def test_layer_fused_combine_parity(name):
    """The layer with the combine folded into the down projection
    (MoeLayer(fused_combine=True), packed weights): every token of y within the
    bf16 tolerance of the oracle."""
    announce(f"layer {name} fused combine")
    wl = workloads.make(name, DEV)
    s = wl.spec
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype,
                         *(moe.pack_weights(w) for w in (wl.w_gate, wl.w_up, wl.w_down)),
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV,
                         packed_weights=True, fused_combine=True)
    layer.y.view(torch.uint8).fill_(0xFF)
    layer.forward(wl.logits, wl.x)
    torch.cuda.synchronize()
    logits = np_of(wl.logits)
    ids_ref, w_ref = O.gate(logits, s.k, bool(s.renormalize))
    x = np_of(wl.x)
    p_x = O.permute(ids_ref, s.E, s.S, s.n_priority, x)
    h_ref = O.grouped_ffn(p_x["x_sorted"], p_x["group_offsets"], s.E, s.S, layer.nseg, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), s.dtype)
    y_ref = O.combine(h_ref, p_x["flat_to_sorted"], w_ref, s.T, s.k, s.S)
    y_gpu = f64_of(layer.y)
    assert not np.isnan(y_gpu).any(), "tokens left unwritten"
    y_err = rel_max_err(y_gpu, y_ref)
    announce(f"layer {name} fused combine: y err {y_err:.2e} over {s.T} tokens")
    assert y_err <= TOL[s.dtype], y_err


@pytest.mark.parametrize("name", ["tiny", "olmoe_decode"])
def test_layer_with_router_parity(name):
    """The layer with the router projection in front of the gate: logits within
    the fp32-accumulation bound of the oracle's router, then the rest of the path
    decided on the GPU's logits (top-k ids in the same precision on both sides)."""
    announce(f"layer {name} with router")
    wl = workloads.make(name, DEV)
    s = wl.spec
    g = torch.Generator().manual_seed(77)
    w_r = (torch.randn((s.E, s.d), generator=g) * 0.02).to(wl.torch_dtype).to(DEV)
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down,
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV,
                         w_router=w_r)
    layer.forward(None, wl.x)
    torch.cuda.synchronize()
    x, wr = np_of(wl.x), np_of(w_r)
    lg_ref = O.router(x, wr, s.dtype)
    bound = (s.d + 1) * 2.0 ** -24 * (np.abs(O.to_f64(x, s.dtype)) @ np.abs(O.to_f64(wr, s.dtype)).T)
    logits = np_of(layer.logits)
    assert np.all(np.abs(logits.astype(np.float64) - lg_ref) <= bound + 1e-30)
    ids_ref, _ = O.gate(logits, s.k, bool(s.renormalize))
    np.testing.assert_array_equal(np_of(layer.topk_ids), ids_ref)
    toks = _sample_tokens(s.T, s.n_priority)
    ref = O.moe_layer(logits, x, np_of(wl.w_gate), np_of(wl.w_up), np_of(wl.w_down), s.k, s.dtype,
                      n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), tokens=toks)
    y_err = rel_max_err(f64_of(layer.y[torch.from_numpy(toks).to(DEV)]), ref["y"])
    assert y_err <= TOL[s.dtype], y_err


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_prefill", "gptoss_mixed"])
def test_layer_fp8_gemm_parity(name):
    """The prefill-sized layer on pre-packed FP8 codes, which runs the FFN on
    the GEMM kernel: every sorted row of h and every token of y within the bf16
    tolerance of the oracle's FP8 FFN and combine (buffers poisoned first)."""
    announce(f"layer {name} with fp8 weights on the GEMM")
    wl = workloads.make(name, DEV)
    s = wl.spec
    q = [moe.quantize_fp8_rows(w) for w in (wl.w_gate, wl.w_up, wl.w_down)]
    fp8p = (moe.pack_fp8_codes(q[0][0]), q[0][1], moe.pack_fp8_codes(q[1][0]), q[1][1], moe.pack_fp8_codes(q[2][0]),
            q[2][1])
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down,
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV,
                         fp8_weights=fp8p, packed_weights=True)
    for buf in (layer.h_sorted, layer.y):
        buf.view(torch.uint8).fill_(0xFF)
    layer.forward(wl.logits, wl.x)
    torch.cuda.synchronize()
    logits, x = np_of(wl.logits), np_of(wl.x)
    ids, w = O.gate(logits, s.k, bool(s.renormalize))
    np.testing.assert_array_equal(np_of(layer.topk_ids), ids)
    p = O.permute(ids, s.E, s.S, s.n_priority, x)
    nseg = 2 if s.n_priority > 0 else 1
    h_ref = O.grouped_ffn_fp8w(p["x_sorted"], p["group_offsets"], s.E, s.S, nseg,
                               *(np_of(t) for pair in q for t in pair), dtype=s.dtype)
    h_gpu = f64_of(layer.h_sorted)
    assert not np.isnan(h_gpu).any(), "sorted rows left unwritten"
    h_err = rel_max_err(h_gpu, h_ref)
    y_ref = O.combine(h_ref, p["flat_to_sorted"], w, s.T, s.k, s.S)
    y_gpu = f64_of(layer.y)
    assert not np.isnan(y_gpu).any(), "tokens left unwritten"
    y_err = rel_max_err(y_gpu, y_ref)
    announce(f"layer {name} fp8 gemm: h err {h_err:.2e}, y err {y_err:.2e}")
    assert h_err <= TOL[s.dtype], h_err
    assert y_err <= TOL[s.dtype], y_err


@pytest.mark.parametrize("name", ["olmoe_decode", "dsv2_decode_t16", "dsv2_decode_t256"])
def test_layer_fp8_weights_parity(name):
    """The layer with FP8 expert weights (E4M3 codes, fp32 row scales): routing
    bit for bit as with bf16 weights, and the output of sampled tokens against
    the oracle's gate -> permute -> FP8 FFN -> combine on the same codes."""
    announce(f"layer {name} with fp8 weights")
    wl = workloads.make(name, DEV)
    s = wl.spec
    q = [moe.quantize_fp8_rows(w) for w in (wl.w_gate, wl.w_up, wl.w_down)]
    fp8 = (q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1])
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down,
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV,
                         fp8_weights=fp8)
    layer.forward(wl.logits, wl.x)
    torch.cuda.synchronize()
    logits, x = np_of(wl.logits), np_of(wl.x)
    ids, w = O.gate(logits, s.k, bool(s.renormalize))
    np.testing.assert_array_equal(np_of(layer.topk_ids), ids)
    p = O.permute(ids, s.E, s.S, s.n_priority, x)
    toks = _sample_tokens(s.T, s.n_priority)
    T, k = ids.shape
    f2s = p["flat_to_sorted"].astype(np.int64)
    flat = [t * k + j for t in toks for j in range(k)] + [T * k + e * T + t for t in toks for e in range(s.S)]
    need = np.unique(f2s[np.asarray(flat, dtype=np.int64)])
    nseg = 2 if s.n_priority > 0 else 1
    h = O.grouped_ffn_fp8w(p["x_sorted"], p["group_offsets"], s.E, s.S, nseg, *(np_of(t) for t in fp8),
                           dtype=s.dtype, rows=need)
    h_err = rel_max_err(f64_of(layer.h_sorted[torch.from_numpy(need).to(DEV)]), h)
    assert h_err <= TOL[s.dtype], h_err
    y_ref = O.combine(h, f2s, w, T, k, s.S, tokens=toks, row_of_sorted={int(n): i for i, n in enumerate(need)})
    y_err = rel_max_err(f64_of(layer.y[torch.from_numpy(toks).to(DEV)]), y_ref)
    assert y_err <= TOL[s.dtype], y_err
    # the same layer on pre-packed codes: the same bits
    fp8p = (moe.pack_fp8_codes(fp8[0]), fp8[1], moe.pack_fp8_codes(fp8[2]), fp8[3], moe.pack_fp8_codes(fp8[4]), fp8[5])
    lp = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down, n_shared=s.S,
                      n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV, fp8_weights=fp8p,
                      packed_weights=True)
    lp.forward(wl.logits, wl.x)
    torch.cuda.synchronize()
    assert torch.equal(lp.y, layer.y)


@pytest.mark.parametrize("name", ["olmoe_decode", "dsv2_decode_t16", "dsv2_decode_t256", "qwen3_prefill",
                                  "gptoss_mixed"])
def test_layer_packed_weights_matches_unpacked(name):
    """The layer on pre-packed weights gives the unpacked layer's outputs bit for
    bit (that layer is checked against the oracle in test_layer_parity)."""
    announce(f"layer {name} with packed weights")
    wl = workloads.make(name, DEV)
    s = wl.spec
    kw = dict(n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize), device=DEV)
    plain = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down, **kw)
    packed = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, *(moe.pack_weights(w) for w in
                                                                     (wl.w_gate, wl.w_up, wl.w_down)),
                          packed_weights=True, **kw)
    plain.forward(wl.logits, wl.x)
    packed.forward(wl.logits, wl.x)
    torch.cuda.synchronize()
    assert torch.equal(packed.h_sorted, plain.h_sorted)
    assert torch.equal(packed.y, plain.y)
