"""Whole-layer oracle consistency and the synthetic workload recipes (CPU)."""
import numpy as np
import torch

import workloads
from oracle import moe_oracle as O


def _np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def test_moe_layer_sampled_tokens_match_full():
    wl = workloads.custom(T=40, E=6, k=2, d=32, I=24, dtype="bf16", S=1, n_priority=9, seed=3)
    args = (_np(wl.logits), _np(wl.x), _np(wl.w_gate), _np(wl.w_up), _np(wl.w_down), 2, "bf16")
    full = O.moe_layer(*args, n_shared=1, n_priority=9)
    toks = np.array([39, 0, 17])
    part = O.moe_layer(*args, n_shared=1, n_priority=9, tokens=toks)
    np.testing.assert_allclose(part["y"], full["y"][toks], rtol=1e-12, atol=1e-12)


def test_moe_layer_k1_identity_experts():
    """With one routed expert per token and identity experts the layer returns x."""
    wl = workloads.custom(T=32, E=4, k=1, d=16, I=16, dtype="f32", seed=4)
    ids, w = O.gate(_np(wl.logits), 1)
    p = O.permute(ids, 4, 0, 0, _np(wl.x))
    y = O.combine(p["x_sorted"].astype(np.float64), p["flat_to_sorted"], w, 32, 1, 0)
    assert np.array_equal(y.astype(np.float32), _np(wl.x))


def test_workloads_deterministic_and_shaped():
    a = workloads.make("tiny", "cpu")
    b = workloads.make("tiny", "cpu")
    assert workloads.content_hash(a.logits, a.x, a.w_gate, a.w_up, a.w_down) == \
        workloads.content_hash(b.logits, b.x, b.w_gate, b.w_up, b.w_down)
    s = a.spec
    assert a.logits.shape == (s.T, s.E) and a.logits.dtype == torch.float32
    assert a.x.shape == (s.T, s.d)
    assert a.w_gate.shape == (s.E, s.I, s.d) and a.w_down.shape == (s.E, s.d, s.I)
    # N(0, 1/fan_in) expert weights in the tiny recipe
    assert abs(float(a.w_gate.std()) - 1 / np.sqrt(s.d)) < 0.01
    assert abs(float(a.w_down.std()) - 1 / np.sqrt(s.I)) < 0.01


def test_olmoe_domains_shrink_the_union():
    """Same-domain batches touch fewer distinct experts (ELDR page, 'What it solves')."""
    mixed = workloads.make("olmoe_decode", "cpu", with_weights=False)
    local = workloads.make("olmoe_decode_local", "cpu", with_weights=False)
    k = mixed.spec.k
    u_mixed = O.stats(O.gate(_np(mixed.logits), k)[0][None], 64)["union_size"][0]
    u_local = O.stats(O.gate(_np(local.logits), k)[0][None], 64)["union_size"][0]
    assert u_local < u_mixed


def test_zipf_workload_is_skewed():
    wl = workloads.make("dsv2_decode_t256", "cpu", with_weights=False)
    ids, _ = O.gate(_np(wl.logits), wl.spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=64)
    assert counts.max() > 0.5 * wl.spec.T       # a hot expert takes most tokens
    assert (counts == 0).sum() > 0              # and some experts stay cold


def test_request_offsets():
    q = workloads.make("qwen3_prefill", "cpu", with_weights=False)
    assert q.req_offsets.shape[0] == 129 and int(q.req_offsets[-1]) == 8192
    assert q.stats_logits.shape == (8, 8192, 128)
    g = workloads.SPECS["gptoss_mixed"]
    offs = workloads.synth.request_offsets(g)
    assert offs.shape[0] == 66 and int(offs[64]) == 64 and int(offs[-1]) == 4160
